"""CPU oracle for the exact attention forward pass -- TEST INFRASTRUCTURE ONLY.

Nothing on the product path may import, call or execute anything in this package.
Only the tests, the smoke check of the package entry and the CPU-baseline leg of
the benchmark use it. It shares no code with the GPU path: it takes float64
arrays (widened exactly from the 16-bit inputs) and returns float64 results.

Sources, cited by title and section throughout:

* [V1] "6.1 FlashAttention V1 in detail" (infra-guide-du8.pages.dev, CUDA
  programming and kernel optimization guide).
* [IO] "FlashAttention: IO-Aware Tiling, Online Softmax Mathematics, Memory
  Hierarchy Dynamics, and Kernel Evolution" (llms.blog).
* [TL] "FlashAttention: optimize data movement before counting FLOPs"
  (tokenlab.fyi study note on Dao et al., arXiv:2205.14135).

Modules:

* ``dense``  -- the plain definition: S = scale*Q K^T, three-pass safe softmax,
  O = P V and LSE = m + ln l, all in float64.
* ``tiled``  -- a separate online-softmax checker that walks key tiles in any
  order with the (m, l, u) recurrence. It does not import ``dense``.
* ``backward`` -- dQ, dK, dV and D of the backward pass from their definitions
  ([V1] §6.1, [IO] "Backward Pass Recomputation").
* ``splitkv`` -- attention over one key range (a block's O, m, l) and the merge
  of blocks with the two-block rule of [IO] "Online Softmax Mathematics".
* ``fp8`` -- E4M3 encode/decode (OCP format), power-of-two block scales per 64
  rows, block quantization, and exact attention on the dequantized inputs ([IO],
  FlashAttention-3: FP8 with block-level quantization and dynamic scales).

Every function is pinned by tests that do not re-type its formula: the worked
example printed in [TL], closed forms, invariants, a brute-force fsum evaluation
and torch's CPU float64 attention. No function here is "parity unpinned".
"""
