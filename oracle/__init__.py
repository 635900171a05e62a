"""CPU oracle for the shape-keyed autotuned matmul.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import, call, link or execute anything in this package.
The GPU library (gemm_autotuning_amd) never imports it and shares no code,
header, table or helper with it; the only code both sides use is the seeded
input generator (gemm_autotuning_amd.workloads), which holds none of the
method's arithmetic.

Modules
  gemm      fp64 reference matmul (C, built by build_oracle.py), exact decode
  numerics  exact decoders / RNE encoders of fp32, fp16, bf16, fp8 e4m3fn
  key       reference tuning key (fields, texts, 32-byte packing)
  bound     reference roofline time bound and shared-memory fit rule
  select    reference plan and adaptive selection on scripted timings
  cachefile reference reader of the tuning-results file
"""
