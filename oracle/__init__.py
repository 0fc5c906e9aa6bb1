"""CPU oracle for block-scaled 4-bit weight x bf16 activation products (W4A16).

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, FP64 statement of what
the GPU library computes, written from the pages' definitions:

* formats  - the E2M1, Codebook10, Q4_0, E4M3, UE4M3 and FP16 codes, RNE encoders;
* layouts  - the canonical byte layouts of NVFP4, ROCmFP4 Dual / FAST and Q4_0;
* ref      - exact dequantisation, the FP64 product y = x W^T and its bound;
* pack     - the data-free NVFP4 round-to-nearest packer, the ROCmFP4
             exhaustive finite-UE4M3 MSE scale search (C inner loop in csrc/)
             and the Q4_0 signed abs-max packer.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it. The GPU library never imports, links or calls anything here, and nothing
here imports the GPU library: the two share no code. Seeded inputs come from the
separate ``synth`` module.

Parity pins: every function is pinned by tests under tests/ against the pages'
printed facts, closed forms, brute force or exact rational arithmetic. The
canonical byte order inside a block is a reading (the pages do not print one)
and is pinned only by hand-packed fixtures; conformance with third-party NVFP4
or ROCmFPX files is parity unpinned (no such files are available).
"""

FORMATS = ("nvfp4", "rocmfp4_dual", "rocmfp4_fast", "q4_0")
