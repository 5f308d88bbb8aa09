"""CPU fp64 oracle (test infrastructure only; see llama_oracle.py)."""
