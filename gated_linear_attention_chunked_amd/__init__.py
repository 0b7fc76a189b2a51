"""MI355X-native recurrent-memory linear-attention forward scan (placeholder; binding below)."""
