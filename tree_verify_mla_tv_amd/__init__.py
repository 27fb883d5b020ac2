"""MI355X-native tree-verify MLA-absorb attention (HIP kernels behind a C ABI)."""
