"""CPU oracle (test infrastructure only; see oracle/ras.py)."""
