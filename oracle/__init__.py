"""CPU oracle (test infrastructure only): see uq_oracle."""
