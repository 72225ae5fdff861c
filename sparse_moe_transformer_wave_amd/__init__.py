"""MI355X-native Flint-style sparse MoE FFN layer (placeholder; binding follows)."""
