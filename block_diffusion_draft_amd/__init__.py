"""MI355X-native DFlash 2 block-draft step (placeholder; binding added below)."""
