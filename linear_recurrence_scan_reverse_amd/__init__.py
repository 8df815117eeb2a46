"""MI355X-native RL credit-assignment scans (binding is added with the HIP library)."""
