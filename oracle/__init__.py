"""Oracle for the compressed sparse attention layer (c4a / c128a DSA).

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, fp64 CPU statement
of what the layer computes, written from the descriptions in the pages
"DeepSeek DSA、DeepSeek V4与vLLM Hybrid KV Cache详解" (gentlecold.top) and
"DeepSeek V4 稀疏注意力完全解剖" (zoe.im).  It exists so that tests can check
the HIP library against an independent statement of the method.

Who may use it: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product path (the C-ABI library and
its Python binding) never imports, calls or links anything here, and nothing
here imports the product.  The two share no code; the only thing both sides
consume is the seeded input generator, which holds none of the method's
arithmetic.

Modules: ``codecs`` (bf16 / fp8 e4m3fn storage formats), ``dsa`` (the
per-step definitions: RoPE, counts, window, compressor, indexer, Top-k,
attention) and ``layer`` (a decode token or prefill chunk composed from
them, with the state the layer keeps).
"""

from . import codecs  # noqa: F401
from . import dsa  # noqa: F401
from . import layer  # noqa: F401
