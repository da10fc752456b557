"""CPU oracle for the QLoRA hot path (test infrastructure only; see qlora_oracle)."""
