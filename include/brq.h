/*
 * brq.h -- structured orthogonal rotation + group quantization on MI355X (gfx950).
 *
 * C ABI of libbrq.so.  Every data pointer passed to a hot call is a DEVICE
 * pointer owned by the caller; the library never frees or keeps it.  Hot calls
 * (brq_rotate*, brq_rotate_quantize_pack, brq_dequant_unrotate, brq_requant,
 * brq_qlinear, brq_orp_geo_*) are asynchronous on the caller's HIP stream
 * (`stream` is a hipStream_t, NULL = the default stream), never allocate and
 * never synchronise; a fault inside a kernel shows up at the caller's next
 * synchronisation.  A hot call issues nothing but kernel launches on
 * `stream`, so it can be captured into a HIP graph (once called outside the
 * capture: the first call of a kernel may set its attributes); the
 * pointers and workspace captured are then those of every replay.  Launch failures are
 * returned as BRQ_ERR_HIP.  Errors are returned, never thrown; the last
 * error's detail text is kept per thread (brq_last_error).
 *
 * Sources of the operations (gist.science explainers):
 *  [HARP] "HARP: Hadamard-Preconditioned Adaptive Rotation Processor for
 *         Extreme LLM Quantization", technical summary sections 1, 2.1, 2.2, 2.4.
 *  [PolarQuant] "PolarQuant: Optimal Gaussian Weight Quantization via Hadamard
 *         Rotation for LLM Compression", technical overview sections 1 and 2.
 *  [ORPQuant] "ORPQuant: geometric orthogonal residual projection for
 *         multiplier-free power-of-two transformer quantization", technical
 *         summary section 2.
 */
#ifndef BRQ_H
#define BRQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BRQ_OK = 0,
  BRQ_ERR_INVALID_ARGUMENT = 1, /* malformed call: shapes, NULLs, radices ...  */
  BRQ_ERR_UNSUPPORTED = 2,      /* well-formed but outside what is implemented */
  BRQ_ERR_ALIGNMENT = 3,        /* pointer or leading dimension misaligned     */
  BRQ_ERR_WORKSPACE = 4,        /* workspace missing or too small              */
  BRQ_ERR_HIP = 5               /* HIP runtime error (no device, launch, alloc)*/
} brq_status;

typedef enum { BRQ_F32 = 0, BRQ_BF16 = 1, BRQ_F16 = 2 } brq_dtype;

/* How the b_t x b_t blocks of each stage are given. */
typedef enum {
  BRQ_HADAMARD = 0,  /* blocks = NULL; every radix a power of two; block of
                        stage t is H_b/sqrt(b), H_b the +-1 Sylvester matrix in
                        natural order ([HARP] 2.2, the base mixer G_b).        */
  BRQ_SHARED = 1,    /* one [b_t][b_t] block per stage, used by every group  */
  BRQ_PER_GROUP = 2  /* [d/b_t][b_t][b_t] per stage, one block per group c     */
} brq_block_mode;

typedef enum { BRQ_ABSMAX = 0, BRQ_CODEBOOK_NORM = 1 } brq_qkind;

typedef struct brq_plan brq_plan;

/* Group quantizer after the rotation.
 *  kind ABSMAX ([PolarQuant] section 1, the linear map for values uniform on
 *    [-alpha, alpha]): per contiguous group of `group` values along a row,
 *    alpha = max|v|, h = (2^bits - 1)/2, code = clamp(rint(fma(v, h/alpha, h)),
 *    0, 2^bits - 1) in float32 (rint: half to even), scales are float32 alpha
 *    [m][n/group]; alpha = 0 gives codes 0.
 *  kind CODEBOOK_NORM ([PolarQuant] section 2): r = ||v||_2 of the group,
 *    z = v * (sqrt(group)/r), code = #{k : z > (c_k + c_{k+1})/2} for the
 *    2^bits ascending float32 centroids in `codebook`; scales are float16 r
 *    [m][n/group]; r = 0 gives codes 0.
 *  Codes of a row form one little-endian bit stream: code k of the row sits in
 *  stream bits [k*bits, (k+1)*bits), stream bit p = bit (p mod 8) of byte p/8.
 *  The code array is [m][n*bits/8] bytes, rows contiguous.
 *  bits in 2..5; group a power of two in 64..1024 dividing n. */
typedef struct {
  int32_t kind;       /* brq_qkind                                     */
  int32_t bits;       /* 2..5                                          */
  int32_t group;      /* 64, 128, 256, 512 or 1024                     */
  float codebook[32]; /* CODEBOOK_NORM: 2^bits ascending centroids     */
} brq_quant;

/* Name of a status code (static string). */
const char* brq_status_string(brq_status s);

/* Detail text of the last error returned on this thread ("" if none). */
const char* brq_last_error(void);

/* Library ABI version (major*100 + minor). */
int32_t brq_version(void);

/*
 * Create a transform plan for dimension d ([HARP] 2.1): a mixed-radix
 * schedule radix[0..n_stages) with prod(radix) = d; stage t applies
 * b_t x b_t blocks to the groups {base + k*S_t : k < b_t}, S_t =
 * prod_{s>t} b_s (digit 0 most significant, last stage stride 1); the group
 * index is c = (i / (b_t*S_t))*S_t + i % S_t; a group's output
 * y[base + j*S_t] = sum_k B_{t,c}[j][k] x[base + k*S_t].
 * The transform is M = B_{m-1} ... B_0 D with D = diag(signs) ([HARP] section
 * 1: random signs, then the Hadamard-like stages).
 *   blocks: host float32, layout per `mode` (stage after stage, each block
 *           row-major [j][k]); NULL for BRQ_HADAMARD.
 *   signs:  host int8 +-1 of length d, or NULL for all +1.
 * The host arrays are copied; the plan owns device copies on the current HIP
 * device, is immutable and may be used concurrently from several streams.
 * Errors: INVALID_ARGUMENT (out == NULL, d < 2, n_stages not in 1..16,
 * prod(radix) != d, radix < 2, blocks missing, a sign not +-1, bad mode),
 * UNSUPPORTED (radix > 64, d > 2^22, Hadamard radix not a power of two),
 * HIP (no device or allocation failure; nothing is leaked). */
brq_status brq_plan_create(brq_plan** out, int32_t d, int32_t n_stages, const int32_t* radix,
                           const float* blocks, int32_t mode, const int8_t* signs);

/*
 * HARP blocks from their parameters ([HARP] section 2.2: every block is
 * B_{t,c}(theta) = Q_{t,c}(theta) G_b, Q a Givens rotation for b = 2 and the
 * Cayley map of a skew-symmetric matrix for b > 2, G the base mixer; section
 * 2.4: the parameters may be stored as int8).  Builds the `ngroups` b x b
 * blocks of one stage on the device:
 *   theta_q: device int8 [ngroups][np], np = 1 for b = 2, b(b-1)/2 above;
 *            theta = scale * q.  b > 2: A[i][j] = theta[i*b - i*(i+1)/2 + j-i-1]
 *            for i < j, A[j][i] = -A[i][j], Q = (I - A)^{-1} (I + A);
 *            b = 2: Q = [[cos theta, -sin theta], [sin theta, cos theta]].
 *   base:    device float32 G [b][b] row-major, or NULL for the normalised
 *            Sylvester Hadamard matrix H_b / sqrt(b) (b a power of two).
 *   blocks:  device float32 [ngroups][b][b], block rows B[j][k] as in
 *            brq_plan_create; computed in float64, rounded once.
 * Asynchronous on `stream`; theta_q, base and blocks are owned by the caller.
 * Errors: INVALID_ARGUMENT (b not in 2..64, ngroups not in 0..2^31-1, NULL
 * pointers with ngroups > 0, NULL base for a radix that is not a power of
 * two, scale not finite), HIP.  Parameters are not range-checked (-128 is
 * read as -128). */
brq_status brq_harp_blocks(int32_t b, int64_t ngroups, const int8_t* theta_q, float scale,
                           const float* base, float* blocks, void* stream);

/*
 * Several brq_harp_blocks calls at once (the stages of a plan, [HARP]
 * section 2.2; they are independent): job i builds jobs[i].ngroups blocks
 * of radix jobs[i].b exactly as brq_harp_blocks(b, ngroups, theta_q, scale,
 * base, blocks) would, bit for bit.  Jobs of radix 3..32 share launches (up
 * to 16 jobs each), so a stage of few large blocks overlaps stages of many
 * small ones; radix 2 and radices above 32 launch on their own.  jobs is a
 * host array of n_jobs entries (device pointers inside, as brq_harp_blocks);
 * outputs must not overlap.  Asynchronous on `stream`.  Errors: as
 * brq_harp_blocks for each job (nothing is launched if one is invalid),
 * INVALID_ARGUMENT (n_jobs < 0, jobs NULL with n_jobs > 0), HIP. */
typedef struct brq_harp_job {
  int32_t b;
  int64_t ngroups;
  const int8_t* theta_q;
  float scale;
  const float* base;
  float* blocks;
} brq_harp_job;
brq_status brq_harp_blocks_batch(int32_t n_jobs, const brq_harp_job* jobs, void* stream);

/*
 * A per-group plan from HARP parameters: stage t's blocks are
 * brq_harp_blocks(radix[t], d / radix[t], ...) of its parameters.
 *   theta_q: host int8, the stages' parameters one after the other, each
 *            stage's groups c in order (c as in brq_plan_create).
 *   scales:  host float32 [n_stages], theta = scales[t] * q.
 *   bases:   host float32 G blocks of all stages, [b_t][b_t] each, one after
 *            the other; NULL for Sylvester at every stage (all radices powers
 *            of two).  With all parameters zero the plan is the RHT.
 *   signs:   as brq_plan_create.
 * Builds the blocks on the current device and waits for them, then proceeds
 * as brq_plan_create(..., BRQ_PER_GROUP, signs).  Errors: as brq_plan_create
 * and brq_harp_blocks. */
brq_status brq_plan_create_harp(brq_plan** out, int32_t d, int32_t n_stages, const int32_t* radix,
                                const int8_t* theta_q, const float* scales, const float* bases,
                                const int8_t* signs);

/*
 * Plan serialisation.  brq_plan_serialize writes a byte image of the plan:
 * a plan made by brq_plan_create_harp as its int8 parameters, scales and base
 * mixers ([HARP] section 2.4: int8 parameter storage), any other plan as its
 * float32 blocks; then the signs; then a 64-bit hash of the image.  With
 * buf == NULL it only sets *size; otherwise cap must be at least that size.
 * The blocks are read back from the device (the call waits for them).
 * brq_plan_deserialize rebuilds the plan on the current device (as
 * brq_plan_create or brq_plan_create_harp would); serialising the result
 * gives the same bytes.  Errors: INVALID_ARGUMENT (NULLs, cap too small, not
 * an image, wrong hash, truncated or trailing bytes, a header that
 * brq_plan_create would refuse), UNSUPPORTED (an image version other than
 * 1), HIP. */
brq_status brq_plan_serialize(const brq_plan* plan, void* buf, size_t cap, size_t* size);
brq_status brq_plan_deserialize(brq_plan** out, const void* buf, size_t size);

/* Free a plan and its device arrays; NULL is allowed.  The caller must make
 * sure no queued work still uses the plan. */
brq_status brq_plan_destroy(brq_plan* plan);

/* Dimension of a plan (0 for NULL). */
int32_t brq_plan_dim(const brq_plan* plan);

/*
 * Workspace bytes needed by brq_rotate / brq_rotate_inverse (pass left = NULL
 * or right = NULL for one side), brq_rotate_quantize_pack and
 * brq_dequant_unrotate for an m x n matrix.  The workspace holds the float32
 * intermediate between passes (m*n*4 bytes when one is needed, else 0).
 */
size_t brq_workspace_bytes(const brq_plan* left, const brq_plan* right, int64_t m, int64_t n);

/*
 * One-sided rotation.  side 0 (RIGHT, row-contiguous): every row of
 * x [rows][cols] (or every d-long chunk of a row when d < cols, block-diagonal)
 * becomes M x, i.e. Y = X M^T.  side 1 (LEFT, column direction): d == rows and
 * every column becomes M x, i.e. Y = M X.  brq_rotate_inverse applies M^T
 * instead (the exact inverse for orthogonal blocks; [PolarQuant] section 2:
 * the Hadamard transform is its own inverse).
 *   x, y: device arrays of type xt / yt (F32, BF16, F16) with leading
 *         dimensions ldx, ldy (elements, >= cols).  y may equal x only when
 *         xt == yt and ldx == ldy.
 *   ws:   device workspace of brq_workspace_bytes(...) bytes (may be NULL if
 *         that is 0).
 * Errors: INVALID_ARGUMENT (NULL pointers, d does not divide cols / d != rows,
 * ld < cols, bad dtype or side), WORKSPACE, HIP.  rows == 0 is a no-op. */
brq_status brq_rotate(const brq_plan* plan, int32_t side, const void* x, int32_t xt, int64_t ldx,
                      void* y, int32_t yt, int64_t ldy, int64_t rows, int64_t cols, void* ws,
                      size_t ws_bytes, void* stream);
brq_status brq_rotate_inverse(const brq_plan* plan, int32_t side, const void* x, int32_t xt,
                              int64_t ldx, void* y, int32_t yt, int64_t ldy, int64_t rows,
                              int64_t cols, void* ws, size_t ws_bytes, void* stream);

/*
 * Two-sided rotate, quantize and pack ([HARP] 2: the two-sided processor
 * U W V^T ahead of the quantizer; [PolarQuant] 2 for the codebook kind):
 * W' = M_U W M_V^T (left or right may be NULL: identity), then the group
 * quantizer `q` along the rows of W'.
 *   w:      device [m][n] of type wt, leading dimension ldw (elements).
 *   left:   d == m; right: d divides n (block-diagonal when d < n).
 *   codes:  device [m][n*bits/8] bytes; scales: device [m][n/group]
 *           (float32 alpha for ABSMAX, float16 r for CODEBOOK_NORM).
 *   ws:     device workspace, brq_workspace_bytes(left, right, m, n) bytes.
 * Errors: INVALID_ARGUMENT (NULLs, shapes, bits/group/kind), UNSUPPORTED
 * (group not a power of two in 64..1024), WORKSPACE, HIP. */
brq_status brq_rotate_quantize_pack(const brq_plan* left, const brq_plan* right, const void* w,
                                    int32_t wt, int64_t m, int64_t n, int64_t ldw,
                                    const brq_quant* q, uint8_t* codes, void* scales, void* ws,
                                    size_t ws_bytes, void* stream);

/*
 * Inverse of the above: unpack, dequantize (ABSMAX: v = alpha*(code/h - 1);
 * CODEBOOK_NORM: v = r*c[code]/sqrt(group)), then W = M_U^T V M_V.
 *   out: device [m][n] of type ot, leading dimension ldo.
 * Errors as brq_rotate_quantize_pack. */
brq_status brq_dequant_unrotate(const brq_plan* left, const brq_plan* right, const uint8_t* codes,
                                const void* scales, const brq_quant* q, int64_t m, int64_t n,
                                void* out, int32_t ot, int64_t ldo, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * PolarQuant's downstream chain ([PolarQuant] section 3: weights quantized
 * by PolarQuant, restored, then quantized again with absmax INT4 do better
 * than absmax INT4 alone): unpack and dequantize `codes`/`scales` with q_in,
 * undo the right-side plan (W = V' M_V, as brq_dequant_unrotate with no left
 * plan), then quantize and pack the restored rows with q_out, which must be
 * ABSMAX.  The restored weights reach the second quantizer in float32.
 *   codes, scales:         device inputs as brq_rotate_quantize_pack wrote them.
 *   codes_out, scales_out: device [m][n*q_out.bits/8] bytes, float32 [m][n/q_out.group].
 *   ws: device workspace of brq_requant_workspace_bytes(...) bytes: 0 when one
 *       fused pass takes the call (a right Hadamard plan with d = 64..256,
 *       q_in.group and q_out.group at most 1024), else 2*m*n*4 for the
 *       restored matrix and the steps' own workspace.
 * Errors: INVALID_ARGUMENT (NULLs, shapes, either quantizer, q_out not
 * ABSMAX), UNSUPPORTED, WORKSPACE, HIP. */
size_t brq_requant_workspace_bytes(const brq_plan* right, const brq_quant* q_in,
                                   const brq_quant* q_out, int64_t m, int64_t n);
brq_status brq_requant(const brq_plan* right, const uint8_t* codes, const void* scales,
                       const brq_quant* q_in, int64_t m, int64_t n, const brq_quant* q_out,
                       uint8_t* codes_out, void* scales_out, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * The quantized linear layer at decode ([HARP] section 2: W' = M_U W M_V^T is
 * what gets quantized; at inference the activations are rotated online,
 * section 2.4): with W = M_U^T W' M_V, Y = X W^T is computed as
 *   X~ = X M_V^T (brq_rotate, right side, in the activation type),
 *   Z  = X~ W'^T with W' the absmax codes/scales of brq_rotate_quantize_pack,
 *        dequantized in the product's prologue (integer levels 2c - L on the
 *        MFMA units, each group's partial sum scaled by alpha / L in float32),
 *   Y  = Z M_U (every row z becomes M_U^T z; brq_rotate_inverse, right side).
 * left or right may be NULL (identity).
 *   x:      device [T][ldx] activations, xt F16 or BF16 (16-byte aligned rows
 *           when right is NULL).
 *   codes, scales: device, as brq_rotate_quantize_pack wrote them for an
 *           [m][n] weight (4-byte aligned); q: that call's quantizer (ABSMAX,
 *           groups of 64 or 128).  With 16-byte aligned codes the product
 *           stages the weight through LDS: from 64 tokens with n a multiple
 *           of 256 and m of 256 (a GEMM-shaped kernel), else with n a
 *           multiple of 512; otherwise a slower kernel reads it directly
 *           (same results to the float32 rounding of the group sums).
 *   y:      device [T][ldy] of type yt.
 *   ws:     device workspace of brq_qlinear_workspace_bytes(...) bytes.  On
 *           return, when right is not NULL, its first T*n*2 bytes hold X~ as
 *           a row-major [T][n] array of the activation type.
 * m must be a multiple of 256 for T <= 16 and of 128 above.  Asynchronous
 * on `stream`.  Errors: INVALID_ARGUMENT (dtypes, shapes, NULLs, q not
 * ABSMAX), UNSUPPORTED (m, group), ALIGNMENT, WORKSPACE, HIP. */
size_t brq_qlinear_workspace_bytes(const brq_plan* left, const brq_plan* right, const brq_quant* q,
                                   int64_t T, int64_t m, int64_t n);
brq_status brq_qlinear(const brq_plan* left, const brq_plan* right, const void* x, int32_t xt,
                       int64_t ldx, int64_t T, const uint8_t* codes, const void* scales,
                       const brq_quant* q, int64_t m, int64_t n, void* y, int32_t yt, int64_t ldy,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * brq_qlinear for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation, kernels and results as brq_qlinear, without the `ws`
 * argument.  Its scratch is a device array of brq_qlinear_noalloc_limit()
 * bytes (64 MiB) inside the library, one per GPU, held until the process
 * ends; the call allocates nothing.  A call whose brq_qlinear_workspace_bytes
 * exceeds the limit returns BRQ_ERR_WORKSPACE (at the 70B down projection,
 * 8192 x 28672 with 2-bit groups of 64, up to 128 tokens fit).  Every call on
 * one GPU uses that GPU's array: calls that overlap on one GPU (other streams
 * or threads) race and must be serialised by the caller.  Nothing in the
 * array needs to start at zero; it keeps the last call's contents.  Errors:
 * as brq_qlinear, plus WORKSPACE for a call beyond the limit.
 */
size_t brq_qlinear_noalloc_limit(void);
brq_status brq_qlinear_noalloc(const brq_plan* left, const brq_plan* right, const void* x,
                               int32_t xt, int64_t ldx, int64_t T, const uint8_t* codes,
                               const void* scales, const brq_quant* q, int64_t m, int64_t n,
                               void* y, int32_t yt, int64_t ldy, void* stream);

/*
 * ORP GEO quantizer ([ORPQuant] technical summary, section 2: the geometric
 * discrete basis search and the GEO scales).  Per group of `group`
 * consecutive inputs w of a row, after the optional preconditioning
 * w_p = w * smooth (one float32 product per element):
 *   b1: the nearest level to u = w_p * fl(1/alpha), alpha = max |w_p|, of the
 *       asymmetric power-of-two lattice with zero: 2^(bits-1) negative levels
 *       -1, -1/2, ..., -2^-(2^(bits-1)-1), zero, and 2^(bits-1)-1 positive
 *       levels 1, 1/2, ..., 2^-(2^(bits-1)-2) (3 bits: -1 -1/2 -1/4 -1/8 0
 *       1/4 1/2 1); codes index the levels in ascending order; a tie goes to
 *       the lower code; decided in float32.
 *   b2: inside micro-blocks of 2*stride entries, entry i of the first half
 *       pairs with i + stride and b2 takes (b1[i], b1[i+stride]) to
 *       sigma * (-b1[i+stride], b1[i]), sigma = +1 when
 *       d = w_p[i+stride] b1[i] - w_p[i] b1[i+stride] >= 0 (b2 follows the
 *       Gram-Schmidt residual of w_p against b1), else -1.  b2 is orthogonal
 *       to b1 and ||b2|| = ||b1||.
 *   c1 = <w_p, b1> / ||b1||^2, c2 = <w_p, b2> / ||b1||^2 (the least-squares
 *       scales for orthogonal bases); a group with alpha = 0 gets the zero
 *       code everywhere and c1 = c2 = 0.
 * Outputs (device, caller-owned):
 *   codes [m][n*bits/8]: LSB-first bit stream of b1 codes per row (as for
 *         brq_quant), 4-byte aligned;
 *   signs [m][n/16]: one bit per pair, 1 for sigma = -1; the pair whose first
 *         entry is i has number (i / (2*stride))*stride + i % (2*stride) and
 *         sits at bit (number mod 8) of byte number/8 of its row;
 *   coef  [m][n/group][2] float32 (c1, c2), 8-byte aligned.
 * w: device [m][ldw] of type wt (F32/BF16/F16), 16-byte aligned rows;
 * smooth: device float32 [n] (16-byte aligned) or NULL.  bits 2..5, group
 * 64/128/256/512 dividing n, stride a power of two with 2*stride <= group.
 * Asynchronous on `stream`.  Errors: INVALID_ARGUMENT (dtype, shape, NULLs,
 * stride, group not dividing n), UNSUPPORTED (bits, group), ALIGNMENT, HIP. */
typedef struct {
  int32_t bits;   /* 2..5                          */
  int32_t group;  /* 64, 128, 256 or 512           */
  int32_t stride; /* pair stride S: power of two   */
} brq_orp;

brq_status brq_orp_geo_quantize(const void* w, int32_t wt, int64_t m, int64_t n, int64_t ldw,
                                const float* smooth, const brq_orp* q, uint8_t* codes,
                                uint8_t* signs, float* coef, void* stream);

/*
 * The ORP dequantizer: w_p^ = c1 b1 + c2 b2 per group (in the preconditioned
 * domain; rounded once from float32, c1 b1 being exact), from the outputs of
 * brq_orp_geo_quantize.  out: device [m][ldo] of type ot, 16-byte aligned
 * rows.  Errors as brq_orp_geo_quantize. */
brq_status brq_orp_geo_dequant(const uint8_t* codes, const uint8_t* signs, const float* coef,
                               const brq_orp* q, int64_t m, int64_t n, void* out, int32_t ot,
                               int64_t ldo, void* stream);

/*
 * Host helper: the 2^bits Lloyd-Max centroids for N(0,1), ascending, rounded
 * to float32 ([PolarQuant] section 2: MSE-optimal centroids for the standard
 * normal, table stored in float32).  bits in 1..5; centroids has 2^bits
 * entries.  Errors: INVALID_ARGUMENT, UNSUPPORTED (did not converge).
 */
brq_status brq_lloyd_max_gaussian(int32_t bits, float* centroids);

/*
 * Kernel timing (diagnostics).  While enabled, every kernel launched by the
 * hot calls on this process is bracketed by a pair of HIP events recorded on
 * the stream it is launched on; brq_profile_read waits for those events and
 * returns, for the idx-th distinct kernel name (in order of first launch),
 * the summed duration in milliseconds and the launch count since the last
 * reset.  Enabling adds two event records per launch and nothing else.
 * Errors: INVALID_ARGUMENT (idx out of range or NULL outputs), HIP.
 */
brq_status brq_profile_enable(int32_t on);
brq_status brq_profile_reset(void);
int32_t brq_profile_count(void);
brq_status brq_profile_read(int32_t idx, char* name, size_t name_len, double* total_ms,
                            int64_t* launches);

/*
 * Kernel selection (diagnostics and tests).  BRQ_PATH_AUTO (the default)
 * picks the fastest kernels that take a call: the fused two-sided MFMA
 * kernels, the row Hadamard kernel, the stage pass, else the multi-stage
 * tile pass.  BRQ_PATH_TILE sends every call to the tile pass, which takes
 * every plan and shape, so its results can be checked and timed on shapes a
 * faster kernel would otherwise take.  The setting is process-wide and read
 * at each call; results agree to the tolerances of the transform, not bit
 * for bit.  Errors: INVALID_ARGUMENT for an unknown value.
 */
typedef enum { BRQ_PATH_AUTO = 0, BRQ_PATH_TILE = 1 } brq_path;
brq_status brq_set_path(int32_t path);

#ifdef __cplusplus
}
#endif

#endif /* BRQ_H */
