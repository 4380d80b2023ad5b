"""fp64 CPU oracle (test infrastructure; never imported by the library)."""
