"""CPU oracle of the EXL3 linear: test infrastructure only (see exl3_oracle)."""
