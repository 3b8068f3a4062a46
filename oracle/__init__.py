"""CPU oracle for the MXFP8 MoE expert grouped-GEMM hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call,
link or execute anything in this package: it is used by ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else.  It shares no code with the HIP library or its Python
binding; the two meet only in the seeded input generators, which hold none
of the method's arithmetic.

Everything is plain NumPy in float64 (every MXFP8 value, every bf16 value
and every product of two MXFP8 values is exact in float64), written to be
read against its sources, not to be fast:

* ``mxfp8``   -- E4M3 / E8M0 codecs, row-wise and column-wise group
                 quantization, dequantization, the dequantize-then-column-wise
                 requantization and the grouped bias-gradient reduction.
* ``gemm``    -- the three grouped GEMMs (forward, dgrad, wgrad) as loops of
                 per-expert matmuls of dequantized operands, plus the
                 comparison tolerance.
* ``swiglu``  -- the gated activation between the two expert linears of the
                 fused expert-MLP workload (the pages do not define it:
                 parity unpinned).

Sources (pages of the NVIDIA TransformerEngine pull requests):

* "[Pytorch] Add support for row-wise quanted input for grouped gemm"
  (PR #3244): Description; review thread on ``scale_shape``; Greptile
  Summary flowchart.
* "[PyTorch] Fix distributed BF16 weights and trim NVFP4 saved state in the
  fused grouped MLP" (PR #3545): Description; Changes; commit messages.
* "Improve device-init grouped linear module with single grouped weight
  support" (PR #3224): Greptile Summary; review on CUDA ``m_splits``.

The pages fix none of the MXFP8 arithmetic (scale rule, rounding,
saturation).  The oracle takes it from the OCP Microscaling Formats (MX)
v1.0 specification (section 5 for the E8M0 scale and E4M3 element
encodings, section 6.3 for the conversion of a block of 32 values), with
round-to-nearest-even and saturation to the largest finite E4M3 value.
"""

from . import mxfp8, gemm, swiglu  # noqa: F401
