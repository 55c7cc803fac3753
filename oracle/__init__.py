"""Double-precision CPU oracle of the sparse MoE layer forward pass (test infrastructure only)."""
