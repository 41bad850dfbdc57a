"""Oracle package (test infrastructure only; see sf_oracle's header)."""
