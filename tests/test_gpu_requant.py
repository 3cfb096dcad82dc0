"""GPU parity of PolarQuant's downstream chain (brq_requant): codebook-norm
codes are dequantized, rotated back and quantized again with absmax, against
oracle.chain on the same codes and norms -- the fused row pass and the
composed path (dequantize + unrotate into the workspace, then the quantizer)."""

import numpy as np
import pytest

import synthetic as S
from oracle import chain as C
from oracle import lloydmax as LM
from oracle import quant as Q
from oracle import transform as T
from parity import check_absmax_scales, check_codes
from gpu_util import announce, to_dev

pytestmark = pytest.mark.gpu


def _case(rng, m, n, d, bits_in, signs):
    """PolarQuant-encoded weights: the library's own quantizer on seeded
    heavy-tailed weights (codes and norms are then inputs to both sides)."""
    import butterfly_rotation_quantization_amd as brq
    cb = LM.lloyd_max_gaussian(bits_in)[0].astype(np.float32)
    side = S.random_plan(rng, (2,) * int(np.log2(d)), "hadamard", with_signs=signs)
    p = brq.Plan(side.d, side.radix, side.mode, None, side.signs)
    w = S.to_storage(S.gaussian_mixture_weights(rng, m, n), "bf16")
    codes, norms = brq.rotate_quantize_pack(None, p, to_dev(w, "bf16"), bits_in, d,
                                            "codebook_norm", cb)
    plan_o = T.Plan(side.d, side.radix, T.HADAMARD, None,
                    None if side.signs is None else side.signs.astype(np.float64))
    return p, plan_o, cb, codes, norms


@pytest.mark.parametrize("m,n,d,bits_in,bits_out,g_out,signs", [
    (64, 4096, 128, 5, 4, 128, False),    # PolarQuant Q5 -> INT4, the pages' chain
    (19, 12288, 128, 5, 4, 64, False),
    (33, 1024, 128, 4, 4, 256, False),
    (8, 2048, 256, 5, 2, 1024, True),     # other widths, groups, signs
    (21, 192, 64, 3, 5, 64, True),
    (11, 1024, 512, 5, 4, 128, False),    # composed: d = 512 is not fused
])
def test_requant_parity(m, n, d, bits_in, bits_out, g_out, signs):
    import butterfly_rotation_quantization_amd as brq
    rng = np.random.default_rng(m * 7 + n + bits_out)
    announce(f"requant m={m} n={n} d={d} b{bits_in}->b{bits_out} g{g_out}")
    p, plan_o, cb, codes, norms = _case(rng, m, n, d, bits_in, signs)
    brq.profile_reset()
    brq.profile_enable(True)
    c_out, a_out = brq.requant(p, codes, norms, m, n, bits_in, d, bits_out, g_out, codebook=cb)
    brq.profile_enable(False)
    names = list(brq.profile_read())
    fused = d <= 256
    assert any(k.startswith("rowhad requant") for k in names) == fused, names
    ci = Q.unpack(codes.cpu().numpy(), bits_in, n)
    ref, alpha, w = C.requant(ci, norms.cpu().numpy(), cb, d, plan_o, bits_out, g_out)
    got = Q.unpack(c_out.cpu().numpy(), bits_out, n)
    what = f"requant d={d} b{bits_in}->b{bits_out} g{g_out}"
    check_absmax_scales(a_out.cpu().numpy(), alpha, w, what)
    info = check_codes(got, ref, Q.absmax_band(w, bits_out, g_out), what, bits_out)
    assert np.array_equal(Q.pack(got, bits_out), c_out.cpu().numpy())
    print(info, flush=True)


def test_requant_equals_the_two_calls():
    """The fused pass gives the codes of dequant_unrotate to float32 followed
    by the stand-alone quantizer, bit for bit outside the band."""
    import butterfly_rotation_quantization_amd as brq
    rng = np.random.default_rng(5)
    m, n, d = 48, 4096, 128
    p, plan_o, cb, codes, norms = _case(rng, m, n, d, 5, False)
    c1, a1 = brq.requant(p, codes, norms, m, n, 5, d, 4, 128, codebook=cb)
    restored = brq.dequant_unrotate(None, p, codes, norms, m, n, 5, d, "codebook_norm", cb)
    c2, a2 = brq.rotate_quantize_pack(None, None, restored, 4, 128)
    w = restored.cpu().numpy().astype(np.float64)
    band = Q.absmax_band(w, 4, 128)
    check_codes(Q.unpack(c1.cpu().numpy(), 4, n), Q.unpack(c2.cpu().numpy(), 4, n), band, "fused vs two calls", 4)
    assert np.abs(a1.cpu().numpy() - a2.cpu().numpy()).max() <= 1e-6 * np.abs(a2.cpu().numpy()).max()


def test_requant_polar_projection_full_size():
    """One PolarQuant projection at full size (gate, 12288 x 4096): sampled
    rows against the oracle."""
    import butterfly_rotation_quantization_amd as brq
    rng = np.random.default_rng(12)
    m, n, d = 12288, 4096, 128
    announce("requant full projection 12288x4096 Q5 -> INT4 g128")
    p, plan_o, cb, codes, norms = _case(rng, m, n, d, 5, False)
    c_out, a_out = brq.requant(p, codes, norms, m, n, 5, d, 4, 128, codebook=cb)
    rows = np.sort(rng.choice(m, size=64, replace=False))
    ci = Q.unpack(codes[rows].cpu().numpy(), 5, n)
    ref, alpha, w = C.requant(ci, norms[rows].cpu().numpy(), cb, d, plan_o, 4, 128)
    got = Q.unpack(c_out[rows].cpu().numpy(), 4, n)
    check_absmax_scales(a_out[rows].cpu().numpy(), alpha, w, "full projection")
    check_codes(got, ref, Q.absmax_band(w, 4, 128), "full projection", 4)
