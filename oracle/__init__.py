"""CPU oracle for the grouped expert MLP -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 numpy code written from the definitions; it is what the
GPU path is checked against and it shares no code with that path.  Only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may
import it; the product path never calls it.

Modules
  numerics  bf16 round-to-nearest-even, OCP E4M3FN rounding, E8M0 shared
            exponents, MXFP8 block quantize / dequantize (row-wise and
            per-expert-segment column-wise)
  permute   stable counting-sort permutation of (token, slot) pairs by expert
  mlp       grouped expert MLP forward and backward, per-expert loop, fp64
  router    softmax -> top-k -> renormalise router (the fused router's oracle)

Parity status: every function here is pinned by a CPU test (brute force,
library cross-checks, closed forms or invariants); none is "parity unpinned".
"""
