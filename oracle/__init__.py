"""CPU oracle for the paged KV-cache attention path.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()``
and the bench's CPU-baseline leg may import anything here. The
product path (the HIP library and its Python binding) never imports, calls or
falls back to this package, and this package imports nothing from the product.

What it holds:

* ``paged``     -- NumPy float64 reference of the whole hot path: scatter of new
                   K/V into a pool of 16-token blocks through a slot mapping,
                   whole-block copies, materialising a sequence's contiguous K/V
                   by walking its block table, and textbook softmax attention for
                   decode (one query per sequence, grouped KV heads) and for a
                   causal prefill chunk over cached plus new tokens.
* ``brute``     -- the same attention as pure-Python scalar loops (``math.exp``,
                   no NumPy arithmetic), for tiny inputs; it pins ``paged``.
* ``allocator`` -- a pure-Python model of the block allocator (null block 0,
                   LIFO free list, refcounted sharing, copy-on-write, tail-first
                   free) that yields the block ids, slots and copy pairs the
                   native allocator must reproduce exactly.

Sources (cited by page title and section in each function): the three pages
"(2) vLLM Internals: From PagedAttention to Removing PagedAttention",
"vLLM: what PagedAttention turned into" and "My Understanding of vLLM and
PagedAttention". None of them prints an attention formula; the oracle uses the
plain definition of scaled softmax attention, which the paged method claims to
compute exactly while reading keys and values from scattered blocks.

Parity status: every function here is pinned by CPU tests against worked
examples from the pages, closed forms, brute force and invariants. No function
is "parity unpinned".
"""
from . import allocator, brute, paged  # noqa: F401
