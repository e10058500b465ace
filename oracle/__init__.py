"""CPU oracle for one mixed chunked-prefill attention step.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg may import or run anything in this package.  It
shares no code with the HIP library in chunked_prefill_mixed_hybrid_amd/.
"""
from .oracle import BF16, F32, Oracle, build, default  # noqa: F401
from .brute import bf16_bits_to_f64, dense_attention, mask_matrix, to_f64  # noqa: F401
