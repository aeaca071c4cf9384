"""MI355X-native W4A16 matmul (placeholder, filled in below)."""
