"""CPU fp64 oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  The library under ``exact_attention_online_amd`` never imports it and
shares no code with it: the two meet only through the seeded inputs of ``attn_inputs``.

What it computes (citations are page title + section):
  * ``attention.forward`` / ``attention.backward``: plain softmax attention and its analytic
    gradients, in float64, from the definition (no online softmax, no tiling of the arithmetic).
    "FlashAttention-2 ... (OpenReview discussion)": the method is exact, so its result is the
    plain definition; "FlashAttention (NeurIPS 2022) notes", sections "(Safe) Softmax" and
    "Backward - Recomputation".
  * ``online.forward_tiled``: the tiled one-pass recurrence of the "Online Softmax" and
    "FlashAttention" sections of the NeurIPS 2022 notes, with the unnormalised accumulator and
    single final division of the FlashAttention-2 author response.  A model of the algorithm,
    checked against the definition; never used as the GPU's reference.
  * ``fp8``: the block quantisation and incoherent processing of "FlashAttention-3 ...
    (abstract)": a Sylvester Hadamard transform with random signs, OCP e4m3 encoding, one scale
    per 128-row block.

Pins (tests/test_oracle_*.py): hand-derived worked examples in tests/golden/, closed forms
(one key, uniform scores, causal row 0), invariants (rows of P sum to one, causal future
independence, shift and permutation invariance, GQA = repeated MHA), central finite differences
on tiny inputs, torch float64 SDPA/autograd, and the e4m3 code table of the OCP definition.
"""
