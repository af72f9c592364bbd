"""Plain, slow, CPU-only oracle for fine-grained FP8 quantization and block GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library and does
not import it.

The oracle writes out the method as the pages define it, in numpy, with
explicit rounding steps:

* ``e4m3``     - the E4M3 number format (1 sign, 4 exponent, 3 mantissa bits,
                 largest finite 448) as a 256-entry table; saturating
                 round-to-nearest-even encode by nearest-value search.
* ``quant``    - online quantization with one FP32 scale per 1x128 activation
                 tile, per 128x1 column tile, and per 128x128 weight block;
                 scale = tile amax / 448, codes = E4M3(x / scale); plus the
                 caller-scale mode used by delayed/static scale policies.
* ``gemm``     - block-scaled GEMM: FP8 x FP8 partial products summed per
                 128-wide K block (exact in float64), multiplied by the two
                 block scales, summed over blocks, then rounded to the output
                 type (BF16 or FP32).
* ``policies`` - current-max, amax-history and fixed-calibration scale
                 policies over a drifting tile sequence.
* ``examples`` - the pages' worked examples (two tiles near 0.1 and with a
                 20.0 outlier; per-tensor vs fine-grained GEMM error).
"""
from . import e4m3, quant, gemm, policies, examples  # noqa: F401
