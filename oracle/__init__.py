"""CPU oracle (test infrastructure only; see medusa_oracle)."""
