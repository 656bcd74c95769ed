"""CPU oracle for Kimi Delta Attention prefill (TEST INFRASTRUCTURE ONLY).

Only tests/, the smoke check in __graft_entry__ and the benchmark's
cpu_baseline leg may import anything here.  The product path (the HIP library
and its Python binding) never imports, links or executes this package.

Contents:
  kda_oracle.c   fp64 token recurrence, segment maps, exclusive affine scan (C)
  oracle.py      ctypes wrapper of the above
  exact.py       exact-rational (fractions.Fraction) recurrence and scan for tiny inputs
  chunked.py     fp64 numpy chunk-form algebra (checks the chunked rewriting)
  build.py       gcc build of kda_oracle.c
"""
