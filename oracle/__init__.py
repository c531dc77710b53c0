"""CPU oracle package (test infrastructure only; see qlin_oracle)."""
