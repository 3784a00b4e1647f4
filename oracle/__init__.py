"""CPU oracle for the MSA hot path (test infrastructure only; see msa_oracle)."""
