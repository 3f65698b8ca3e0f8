"""CPU oracle (test infrastructure only; see nsa_oracle)."""
