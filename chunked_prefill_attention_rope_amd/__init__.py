"""Chunked prefill with past (RoPE, KV-cache append, GQA attention) on MI355X.

The compute path is the C-ABI library ``libcp.so`` (hand-written HIP kernels
for gfx950) declared in ``include/cp.h``; ``chunked_prefill_attention_rope_amd.cp``
is its thin ctypes binding.  Importing this package loads nothing; importing
``.cp`` loads the library and raises if it has not been built.
"""
