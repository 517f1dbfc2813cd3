"""libkvarn: KVarN 2-bit KV-cache quantizer for MI355X (gfx950), HIP kernels behind a C ABI.

`kv_cache_bit_amd.kvarn` is the ctypes binding (import it to load libkvarn.so);
`kv_cache_bit_amd.synth` draws seeded synthetic inputs; `kv_cache_bit_amd.build`
compiles the library in-tree.
"""
