"""MI355X-native Mamba-2 SSD chunked scan (placeholder; binding added with the library)."""
