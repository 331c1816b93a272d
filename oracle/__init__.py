"""fp64 CPU oracle (test infrastructure only; see ropekv_oracle's header)."""
