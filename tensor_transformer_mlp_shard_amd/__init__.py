"""MI355X-native tensor-parallel Transformer shard (placeholder; binding follows)."""
