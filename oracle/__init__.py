"""CPU oracle for the DHSA prefill path (test infrastructure only; see dhsa_oracle)."""
