"""MI355X-native causal kernelized linear attention (binding in progress)."""
