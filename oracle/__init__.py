"""fp64 CPU oracle -- test infrastructure only (tests/, __graft_entry__.smoke(),
bench.py's cpu_baseline leg).  Shares no code with the HIP library."""
