"""CPU oracle package (test infrastructure only; see kvq_oracle's header)."""
