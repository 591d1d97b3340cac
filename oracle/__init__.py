"""CPU oracle for the NVFP4 mixture-of-experts expert path (test infrastructure).

This package is a plain, slow, FP64 NumPy statement of what the GPU path
computes.  It exists to check the GPU path and for nothing else: only the
tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it.  It shares no code with the HIP library and does not import it.

Pages cited throughout (title -> short tag used in the citations):

* "[Kernel] Add NVFP4 MoE CUTLASS support for SM120" -> vLLM PR #29242
* "SM120 (RTX Blackwell) NVFP4 MoE: CUTLASS Grouped Block-Scaled GEMM Produces
  Invalid Output; FlashInfer Requires Extensive Patching" -> FlashInfer #2723
* "[NVFP4] NVFP4 MOE emulation fallback for H100/MI300/MI350, standardize
  TritonExperts usage for OCP MX emulation" -> vLLM PR #35737
* "Report: NVFP4 kernel selection on SM120/SM121" -> unsloth PR #10417

Modules:

* ``nvfp4``   the block format: E2M1 codes, E4M3 block scales, FP32 global scale
* ``routing`` softmax / top-k / renormalise router
* ``moe``     permutation by expert and the W4A4 / W4A16 expert layer
* ``bruteforce`` per-token dense loop used to pin ``moe``

Parity pins live in ``tests/test_oracle_*.py``.  Parity unpinned: the value of
the intermediate global scale ``g2`` (a calibration convention, not a result).
"""
