"""CPU oracle for the CacheBlend per-layer KV fusion step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library or its Python binding; both sides only read the same seeded inputs.

What it computes, from the CacheBlend paper (arXiv 2405.16444, "CacheBlend:
Fast Large Language Model Serving for RAG with Cached Knowledge Fusion") and the
explainer pages about it:

* ``rope``   -- rotary tables in fp64 rounded to fp32, rotation of interleaved
                pairs, and the re-rotation of a chunk's cached keys by its new
                offset (paper section 4.3, footnote 3; aifetchly guide,
                "RoPE Delta Positional Realignment").
* ``layer``  -- a plain Llama decoder layer (RMSNorm, GQA causal attention,
                SwiGLU MLP) used as full prefill (paper section 7, "Full KV
                recompute" baseline).
* ``blend``  -- the fusor: HKVD count, top-k selection by K deviation,
                one selective-recompute layer step (paper section 4.2, Figure 5b;
                section 4.3, KV deviation of section 4.1), gradual filtering
                across layers (section 4.3, Figure 9) and the stack driver.
* ``prepass``-- construction of single-layer inputs whose cached KV comes from
                an isolated prefill and whose hidden states come from a full
                prefill of the same layer.

Arithmetic is numpy in the dtype of the arrays passed in: fp32 by default
(the precision the fusor's reference is specified in), fp64 where a pin
compares against an fp64 reference.  Values written into a KV cache or
handed to the next layer can be rounded to the storage dtype (``store``),
since the cache and the layer outputs are stored tensors.

Parity status of each function is listed in its docstring; every function
here is pinned by a ``-m "not gpu"`` test against closed forms, brute force,
or an independent PyTorch-CPU fp64 layer, except where a docstring says
"parity unpinned".
"""
