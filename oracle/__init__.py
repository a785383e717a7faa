"""CPU fp64 oracle of the DoRA hot path (test infrastructure only; see dora_oracle)."""
