"""MI355X-native fused all-reduce + residual-add + RMSNorm epilogue (one GPU's share)."""
