"""Test infrastructure: the double-precision CPU oracle (see oracle.py)."""
