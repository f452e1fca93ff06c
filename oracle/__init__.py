"""CPU float64 oracle (test infrastructure only; see cartattn_oracle)."""
