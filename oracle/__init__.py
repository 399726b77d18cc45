"""CPU oracle of the L3 layer: test infrastructure, never the product path."""
