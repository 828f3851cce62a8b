"""MI355X-native selective-scan hot path (placeholder; binding added with the C ABI)."""
