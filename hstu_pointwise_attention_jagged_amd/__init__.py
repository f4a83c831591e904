"""MI355X-native HSTU layer forward (placeholder; the binding lands with the library)."""
