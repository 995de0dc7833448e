"""CPU oracle of the multi-branch verification step (test infrastructure only:
tests, the package smoke check and the benchmark's CPU-baseline leg use it)."""
