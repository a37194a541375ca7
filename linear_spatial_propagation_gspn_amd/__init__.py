"""MI355X-native GSPN 2D line-scan linear propagation (placeholder until the binding lands)."""
