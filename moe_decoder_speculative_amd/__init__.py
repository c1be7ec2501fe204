"""MI355X-native MoE speculative verification step (placeholder; binding below)."""
