"""CPU oracle for the 2-bit + FP4-delta MoE layer forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call,
link or execute anything in this package: only the tests, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.

The oracle is a plain, slow, obviously-correct restatement of what the method
computes, written from the public description of the vLLM-Moet project
(README "Frontier MoE on consumer Blackwell (SM120)" as carried by the
pickgithub.com project payload, and the airanks.app page
"kacper-daftcode/vLLM-Moet").  Real-valued math is float64; every
quantisation decision is exact integer arithmetic.  It shares no code with
the HIP path in ``bit_moe_expert_nvfp4_amd``.

Modules:
  formats  - e2m1 / e4m3fn / bf16 codecs and NVFP4 decode
  requant  - NVFP4 -> sign-symmetric 2-bit requantisation and the FP4 delta
             (exact integer search, in plain C under ``oracle/c``)
  layout   - packing of the oracle's plain arrays into the library's tiled
             storage layout (written independently of the kernels)
  route    - router top-k, routing weights, token permutation
  ffn      - expert FFN with fixed rounding points, combine, FP4 GEMM,
             expert-cache residency mask and miss count
  gate     - confidence gate (largest next-token probability below tau)
"""
