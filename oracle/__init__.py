"""CPU oracle (test infrastructure only; see mkv_oracle.py)."""
