"""Hardware throughput probes for gfx950 (exp, fma, bf16 matrix cores, their
overlap on one SIMD, and HBM bandwidth); see probes.hip and run.py."""
