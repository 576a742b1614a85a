"""fp64 CPU oracle for calibrated E4M3 paged KV attention.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
statement of what the hot path computes, written in numpy float64. It shares
no code with the HIP library (no kernels, headers, helpers, tables or
constants) and neither imports the other. Only ``tests/``, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path never does.

Sources. The method is described by three pull-request pages:

* "[Model][SM70] Calibrated E4M3 KV cache for Qwen4Exp QSA with MTP"
  (sections Purpose, Status and history, Validation on 4xV100 TP4);
* "[Model][SM70][FP8] Integrate calibrated E4M3 QSA KV capacity path"
  (sections Purpose, Changes, Validation boundary);
* "[Experiment][SM70] Qualify E4M3 KV with MTP3"
  (sections Problem and resulting behavior, CT252 runtime findings).

The pages are prose: they fix that the main K/V cache is stored as
calibrated E4M3 with one finite positive K scale and one V scale per layer,
that decoding is exact, that the scales are applied outside the per-element
loops, and that the split-context temporary output is FP32. Every arithmetic
detail they leave open is settled by a stated reading (see each function's
docstring); the E4M3 format itself follows the OCP 8-bit floating point
specification (OFP8, E4M3 variant with no infinities and max 448).

Modules:

* ``e4m3``      -- exact E4M3 decode and saturating round-to-nearest-even encode
* ``calibrate`` -- per-tensor amax and scale = amax / 448
* ``kv_write``  -- quantising scatter into the paged caches
* ``attention`` -- paged decode / verify / chunk attention in fp64
* ``splits``    -- split-context partials (o, m, l) and their reduction

Every function is pinned by tests under ``tests/`` to something other than
itself: brute force on small inputs, closed forms, library routines (torch's
float8_e4m3fn cast, scaled_dot_product_attention in float64) and invariants.
No function here is "parity unpinned".
"""

from .e4m3 import e4m3_decode, e4m3_encode, E4M3_MAX  # noqa: F401
from .calibrate import calibrate_amax, quotient_f32  # noqa: F401
from .kv_write import quant_write, new_caches, quantise  # noqa: F401
from .attention import paged_attention, paged_attention_f16, gather_sequence_kv  # noqa: F401
from .splits import split_partials, split_reduce, split_bounds  # noqa: F401
