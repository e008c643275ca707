"""MI355X exact attention: fused forward and split-KV decode (binding added with the library)."""
