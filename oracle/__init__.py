"""TEST INFRASTRUCTURE ONLY: the plain fp64 CPU oracle (see oracle.py)."""
