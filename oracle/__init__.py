"""CPU oracle of the leader-side arithmetic (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never does.
"""
