"""MI355X-native hybrid (chunked-prefill + decode) paged attention step.

The product is the C-ABI library libhybridattn.so (hand-written HIP for
gfx950): paged_kv_append writes a step's new K/V into the paged pools through
a slot mapping, then hybrid_attn_fwd runs one varlen, right-aligned causal,
paged attention forward over the packed mixed batch.  `binding` is a thin
ctypes layer over it; `workload` builds seeded synthetic inputs.
"""
