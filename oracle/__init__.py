"""Plain CPU oracle for the FA-quantization hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library and never
imports it.

Everything here is written from the pages' descriptions, in numpy and in fp64
where the arithmetic is floating point:

* ``formats``   - the number formats (INT8, FP8 E4M3FN, E2M1, E8M0, bf16),
                  each grid built by enumerating its codes;
* ``quantize``  - the quantizers of the three FA combinations of the
                  msModelSlim "FA 量化" knowledge-base page (section 分支组合:
                  组合 1 INT8 per-head static, 组合 2 FP8 per-token dynamic,
                  组合 3 MXFP4 per-block dynamic) and of the rotate -> FP8
                  block-quant path of the MindIE SD "量化" page (section
                  FA量化 / 技术特点);
* ``attention`` - attention on the dequantized operands with the probability
                  quantization rule (tile-local max over 128-key tiles).

Parity pins: see the header of each module.  The probability-quantization
rule inside ``attention`` is a reading (the pages are silent on how the
softmax output enters the low-bit PV product, so they print no value for
it); the oracle's arithmetic for it is pinned by hand-worked two-key closed
forms for every rule, invariants and special cases (see ``attention``).
"""

from . import formats, quantize, attention  # noqa: F401
