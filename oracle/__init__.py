"""CPU oracle (test infrastructure only): see oracle.oscar_oracle."""
