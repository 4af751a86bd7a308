"""CPU oracle of the speculative-decoding step (test infrastructure only)."""
