"""fp64 CPU oracle of the selective SSM scan (test infrastructure only)."""
