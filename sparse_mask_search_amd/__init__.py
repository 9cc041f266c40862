"""MI355X-native transposable N:M mask search (placeholder; binding added below)."""
