"""MI355X-native ring-attention shard (placeholder; binding added with the C ABI)."""
