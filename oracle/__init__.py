"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference that the HIP library is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The product path (``paged_kv_cache_18_amd``)
never imports, calls or links anything in here, and nothing in here imports
the product path: the two share no code.  The only module both sides use is
``paged_kv_cache_18_amd.workloads``, which draws seeded random inputs and holds
none of the method's arithmetic.

Sources (cited by page title and section throughout):

* "The 8GB VRAM Breakthrough: How PagedAttention and Dynamic KV-Cache
  Quantization Unlock 64k Context on Consumer GPUs" -- cited as *8GB page*.
* "Capitulo 8 -- Gerenciamento de KV Cache de Proxima Geracao" (LLM Primer VI)
  -- cited as *Primer ch. 8*.
* "A Ideia de 60 Anos Que Domou a Memoria da GPU" -- cited as *60-year page*.
* "PagedAttention aplica memoria virtual ao cache KV de LLMs" -- cited as
  *3-minute page*.

Modules
-------
allocator   LIFO block pool with refcounts, sequences, fork, copy-on-write.
quant       fp16 rounding, asymmetric INT4 and FP8 E4M3 codecs (fp32 IEEE).
layout      the pool byte layout, read from the C header's specification.
attention   logical K/V rebuild through the block table + float64 softmax
            attention (the plain definition).
accounting  slot, waste and byte closed forms.

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (values the pages print, closed forms, library routines,
invariants, brute force).  Nothing here is "parity unpinned".
"""
