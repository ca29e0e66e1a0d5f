"""MI355X-native block-scaled small-M decode GEMV (placeholder; binding added with the library)."""
