"""fp64 CPU oracle (test infrastructure only; see qknr_oracle)."""
