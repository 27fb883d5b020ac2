"""MI355X-native tree-verify MLA-absorb attention: HIP kernels behind a C ABI.

`tree_verify_mla_tv_amd.tv` is the Python binding of libtv.so (include/tv.h);
`tree_verify_mla_tv_amd.workloads` draws the seeded synthetic inputs.
"""
