"""MI355X-native IO-aware attention forward and split-KV decode (placeholder until the binding)."""
