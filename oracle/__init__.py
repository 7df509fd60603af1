"""CPU oracle for the Loki decode step (test infrastructure only)."""
