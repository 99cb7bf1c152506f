"""fp64 CPU oracle for the KDA path.  Test infrastructure only: imported by the
tests, the smoke check and the benchmark's CPU-baseline leg, never by the
product path."""
