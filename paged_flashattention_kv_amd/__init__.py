"""MI355X-native paged attention (placeholder until the binding lands)."""
