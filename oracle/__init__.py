"""CPU oracle for the edge-aware attention layer (test infrastructure only)."""
