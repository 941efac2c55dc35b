"""MI355X-native exact attention forward (FlashAttention-style), bf16/fp16."""
