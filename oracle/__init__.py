"""CPU oracle for the decoder forward pass -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct implementation of what the GPU library
computes, written from the pages' definitions in numpy float64 (and a
pure-Python loop version for the tiny model). Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import it;
the library in ``decoder_forward_pass_amd`` never does, and this package
imports nothing from the library. The two share only the seeded inputs of
``synthetic``.

Modules:
  numerics  -- f16 rounding and widening, bf16 widening, uint4 and symmetric int4
               dequantisation
  paged     -- where a key or value of a position lands in the paged KV pool
  sampling  -- seeded sampling of a token from a row of logits, and its PCG32 streams
  model     -- the numpy float64 decoder: full, cached, chunked, batched, greedy
  loops     -- a second, loop-only decoder for tiny shapes

Parity unpinned (stated conventions both sides share, with nothing on the
pages to check them against): the sign/orientation of the RoPE rotation, the
grouped-query head mapping h -> h // (H / H_kv), the logit-scale final gain,
and the uint4 code chooser (which only generates inputs).
"""
