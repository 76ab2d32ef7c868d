"""CPU oracle of the mixture-of-experts layer (test infrastructure only; see oracle.py)."""
