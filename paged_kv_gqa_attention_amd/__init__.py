"""paged_kv_gqa_attention_amd: paged-KV grouped-query attention for MI355X (gfx950).

The compute lives in ``libpa.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/pa.h``).  ``binding`` marshals torch tensors into that
ABI; ``synth`` draws seeded synthetic workloads.  Importing the package loads
nothing: the shared library is opened on first use and a missing build raises.
"""
__all__ = ["binding", "synth"]
