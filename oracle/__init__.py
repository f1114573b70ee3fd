"""Float64 CPU oracle (test infrastructure only; see shampoo_oracle)."""
