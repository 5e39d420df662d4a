"""fp64 CPU oracle for the Mamba-2 ReplaySSM decode path.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path.
"""
