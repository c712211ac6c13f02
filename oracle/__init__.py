"""CPU oracle for paged decode and prefill attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy code that defines what the HIP path must compute.
Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import it; the product library never calls into it and shares no code with
it (the pool layout formula is written out here independently).

Modules
  sizing     KV-cache size closed form and block counts
  layout     pool element index formula, scatter of logical K/V into a pool,
             gather of a sequence's K/V through its block table
  attention  two-pass softmax decode attention over gathered K/V, split-K with
             log-sum-exp merge, causal prefill of a sequence's newest tokens
  allocator  reference model of the refcounted block allocator with
             copy-on-write

Parity status (every function below is pinned by a CPU test unless listed):
  the last-bit rounding and accumulation order of the GPU path are bounded only
  by tolerances -- the pages print no attention output values ("parity
  unpinned" for bit patterns of floating-point outputs; values are pinned).
"""
