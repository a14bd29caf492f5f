"""MI355X-native grouped-query attention step with RoPE over a bf16 KV cache."""
