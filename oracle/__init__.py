"""CPU oracle for the DSA stage (test infrastructure only; see dsa_oracle.c)."""
