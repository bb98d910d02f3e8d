"""Plain CPU oracle for the quantized-weight matrix products (TEST INFRASTRUCTURE).

This package is the checker, not the product.  Only the test suite, the smoke
check of ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The GPU library never calls into it and shares no code with it.

What it computes, in fp64 unless a stored format says otherwise:

* ``codecs``  -- IEEE binary16 (via numpy's float64->float16 rounding) and the
  OCP 8-bit e4m3fn encoding (written here from the format's definition).
* ``quant``   -- round-to-nearest group quantizers producing the canonical byte
  layouts: symmetric int8/int4 with fp16 group scales, the asymmetric 4-bit
  256-superblock format, per-channel fp8/int8 weights and per-token fp8/int8
  activations.
* ``ref``     -- dequantization, the fp64 product ``y = x_hat . w_hat^T``, its
  magnitude bound ``B = |x_hat| . |w_hat|^T`` and the pass/fail comparator.
* ``proxy``   -- RWKVQuant's weights-only coarse-to-fine proxy (P_c, P_f) and
  its SQ/VQ routing, with the readings its header lists.

Every function is pinned by ``tests/test_oracle_*.py`` against facts that do not
come from the oracle itself (brute force, closed forms, exact round trips,
exhaustive codec tables).  Two readings are pinned only by the library's own
specification, not by the source pages ("parity unpinned by the pages"): the
int4 symmetric range (codes -7..7, scale absmax/7) and the asymmetric
superblock's two-level scale rule and sub-code packing.
"""

from . import codecs, proxy, quant, ref  # noqa: F401
