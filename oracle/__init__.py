"""fp64 CPU oracle of the fused linear + cross-entropy path.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the graft entry point's smoke
check and by the benchmark's CPU-baseline leg, never by the product library.
"""
