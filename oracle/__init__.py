"""CPU oracle for the decode MoE block (test infrastructure only)."""
