"""fp64 CPU oracle for exact attention (test infrastructure only: imported by
the tests, the smoke check and the benchmark's CPU baseline, never by the GPU
library)."""
