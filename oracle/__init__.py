"""CPU oracle (test infrastructure only; see kvq_oracle.py)."""
