"""MI355X-native LSA memory-indexer selection path.

`sparse_kv_retrieval_amd.lsa` is the Python binding over the C-ABI library
`liblsa.so` (hand-written HIP kernels for gfx950). `sparse_kv_retrieval_amd.synth`
is the seeded synthetic-input generator. The binding is imported on demand so
that the generator can be used on machines without a GPU.
"""
__all__ = ["synth", "lsa"]
