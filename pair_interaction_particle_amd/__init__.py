"""MI355X-native pair-interaction path (features -> pair MLP -> biased attention)."""
