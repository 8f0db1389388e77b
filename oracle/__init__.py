"""CPU oracle for packed-KV decode attention (test infrastructure only)."""
