"""MI355X-native exact attention forward pass (package under construction)."""
