"""fp64 CPU oracle (test infrastructure only; see tq_oracle's header)."""
