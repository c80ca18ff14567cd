"""CPU oracle of Fathom's read path (test infrastructure only)."""
