"""fp64 CPU oracle of the FreeSolo FS-L attention forward.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg import this package.  It shares no code with the HIP path.
"""
from .pyoracle import Oracle, PlainFsb, Problem, build, make_problem, problem_from, with_prior

__all__ = ["Oracle", "PlainFsb", "Problem", "build", "make_problem", "problem_from", "with_prior"]
