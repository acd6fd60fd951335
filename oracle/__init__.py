"""fp64 CPU oracle of the CommunityKV decode step -- test infrastructure only.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark use it.
"""
