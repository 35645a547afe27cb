"""CPU oracle for the DSA lightning-indexer hot path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
product path (the HIP library and its Python binding) never imports, calls or
links it, and this package imports nothing from the product path.

It is a plain, slow, obviously-checkable restatement of what the indexer
computes, written from three Megatron-LM pull-request pages:

* PR 8403 (the ``dsa_indexer_rope_fp32`` and ``dsa_indexer_scoring_precision``
  options of the cuDNN DSA indexer),
* PR 5992 ("[dev] [DeepSeek-V4] Add compact BF16 and MXFP8 DSA indexer support"),
* PR 7522 (KPool pooled-key DSA indexer, NoPE, precision flags).

Modules:

* ``formats`` - bf16 / OCP E4M3FN / UE8M0 codecs, a correctly rounded fp32
  fused multiply-add, and the pinned exponential used by the KPool softmax.
* ``oracle`` - geometry, preprocessing (key LayerNorm then RoPE), quantisation,
  KPool compression, scoring, top-k and pool expansion.
* ``exact`` - an exact-rational brute force (``fractions.Fraction``) used to
  pin ``oracle`` on tiny inputs.

Floating point: preprocessing and KPool compression run in fp32 because the
pages fix that precision (PR 8403, "What does this PR do?": the key
LayerNorm -> RoPE chain is kept in FP32; PR 7522, "Changes": a BF16 gate and an
FP32 bias). Every fp32 operation is an individually rounded numpy float32
operation (no fused multiply-add unless ``formats.fma32`` is called by name).
Scoring dequantises the operands exactly and works in fp64.
"""

from . import formats, oracle, exact  # noqa: F401
