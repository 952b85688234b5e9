"""CPU oracle (test infrastructure only; see msa_oracle)."""
