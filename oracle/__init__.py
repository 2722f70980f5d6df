"""Float64 CPU oracle (test infrastructure only; see gmm_oracle)."""
