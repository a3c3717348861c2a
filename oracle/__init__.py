"""Float64 CPU oracle for the MPQ layer solver.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the package smoke check and
by bench.py's CPU-baseline leg.  The GPU library never imports or links it.
"""
