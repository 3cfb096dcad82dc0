"""CPU fp64 oracle for structured-rotation + group quantization.

TEST INFRASTRUCTURE ONLY.  Nothing in the library package imports, links or
calls this package; only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path: it is plain numpy/scipy in float64, written from the pages below.

Sources (cited in every function by short key and section):

* [HARP] "HARP: Hadamard-Preconditioned Adaptive Rotation Processor for
  Extreme LLM Quantization", gist.science explainer, technical summary
  (sections 1, 2.1, 2.2, 2.4).
* [PolarQuant] "PolarQuant: Optimal Gaussian Weight Quantization via Hadamard
  Rotation for LLM Compression", gist.science explainer, technical overview
  (section 1 "background", section 2 "method").
* [ORPQuant] "ORPQuant: geometric orthogonal residual projection for
  multiplier-free power-of-two transformer quantization", gist.science
  explainer, technical summary (section 2: the two-basis search and the GEO
  scales).

Modules:

* ``transform`` -- mixed-radix stage product, dense orthogonal matrix, RHT,
  one- and two-sided application and inverses.
* ``quant`` -- group absmax quantizer, norm-scaled codebook quantizer,
  decision-band accounting, LSB-first bit packing.
* ``lloydmax`` -- Lloyd-Max centroids/thresholds for N(0, 1).
* ``harp`` -- HARP blocks from int8 parameters: Givens / Cayley factor times
  the base mixer ([HARP] sections 2.1, 2.2, 2.4).
* ``chain`` -- PolarQuant's downstream chain: restore, then absmax INT4
  ([PolarQuant] section 3).
* ``linear`` -- the quantized linear layer at decode: rotate the activations,
  multiply by the quantized rotated weight, unrotate the output ([HARP] 2).
* ``orp`` -- ORP's GEO mode: a power-of-two primary basis, an orthogonal
  secondary basis by stride exchange and sign flips, least-squares scales
  ([ORPQuant] section 2).

Readings of points the pages leave open are stated where they are used and
listed together in the design notes of the repository.
"""

from . import transform, quant, lloydmax, harp, chain, linear, orp  # noqa: F401
