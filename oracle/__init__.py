"""Plain CPU oracle for block-diffusion drafting with target-context KV injection.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package
(``block_diffusion_drafting_ctx_amd``) imports, links or calls this package;
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, headers, tables or helpers with
the HIP path.

Everything is written as the plain definition of each step in numpy,
computed in float64 (the pages fix no precision), one sequence at a time,
without blocking, fusion or reordering.  Sources, cited by page title and
section (all three pages are news/explainer articles about DFlash):

* "DFlash: how block diffusion boosts NVIDIA Blackwell throughput"
  (dothoosh.com), section "Block-diffusion architecture": a whole block of
  masked future tokens is drafted in one forward pass; hidden states taken
  from several target layers are fused into one dense context feature; that
  feature enters the Key and Value projections of every draft layer and the
  projected entries stay in the draft KV cache across iterations.
* "DFlash-2: z-lab boosts speculative-decoding throughput" (dothoosh.com),
  section "DFlash-2 mechanisms": the drafter is non-causal; section
  "Architecture-upgrade details", local-convolution bullet: a short-range
  convolution between attention and MLP limits mixing to nearby positions.
  Sections "Performance results" / "Optimising for maximum speed" /
  "Precision cost" print (acceptance rate, mean acceptance length) pairs.
* "NVIDIA tests DFlash to cut LLM inference bottlenecks" (stechtimes.com),
  section "DFlash moves token drafting to parallel compute": the target model
  keeps the verification pass, so the output path of the target is unchanged
  (lossless).

Where the pages are silent (layer form, positions, norm epsilon, tie-break,
conv form, ...) each function states the reading it takes.

Parity status of each function (what pins it, in ``tests/test_oracle_*``):

* ``rmsnorm``            -- pinned: closed form on hand values, torch
                            ``rms_norm`` routine, scale invariance.
* ``rope``               -- pinned: identity at position 0, norm preservation,
                            relative-position invariance, hand-computed 2-d
                            rotation.
* ``gqa_attention``      -- pinned: float64 brute-force triple loop, torch
                            ``scaled_dot_product_attention``, single-key
                            identity, GQA == MHA with replicated heads.
* ``depthwise_conv3``    -- pinned: unit-tap special cases, ``numpy.correlate``.
* ``fuse_features``      -- pinned: K=1 / W=I closed form, concat-order
                            permutation invariant.
* ``draft_layer`` / ``draft_block`` -- pinned: composition against torch
                            ``nn.functional`` building blocks, non-causality
                            and position-dependence invariants.
* ``argmax_lowest`` / ``greedy_verify`` -- pinned: ``numpy.argmax`` on finite
                            data, planted ties and NaNs, full / zero acceptance,
                            and the lossless invariant on a tiny random target.
* ``sample_verify``      -- pinned: the emitted token's distribution,
                            integrated over a grid of uniforms, equals the
                            target's softmax (the lossless property); the
                            low-temperature limit equals ``greedy_verify``;
                            full acceptance draws the bonus by inverse CDF.
* ``kv8_quantize`` / 8-bit cache path -- pinned: brute-force nearest
                            integer search with ties to even, the half-step
                            error bound, exactly representable runs, zero
                            runs, the stored context K equal to the 8-bit
                            round trip of the 16-bit path's (rotated) K, and a
                            single-key block whose attention output is the
                            round trip of its own V.
* ``AcceptanceStats``    -- pinned: the pages' printed (rate, mean length)
                            pairs (``tests/golden/acceptance_stats.txt``).
* real-model acceptance behaviour -- parity unpinned (needs trained weights).
"""

from .draft import (  # noqa: F401
    OracleDims,
    DraftWeights,
    LayerWeights,
    DraftState,
    rmsnorm,
    rope,
    silu,
    gqa_attention,
    depthwise_conv3,
    swiglu_mlp,
    fuse_features,
    draft_layer,
    lm_head_logits,
    fuse_ctx,
    draft_block,
    kv8_quantize,
    kv8_dequantize,
    kv8_roundtrip,
)
from .verify import argmax_lowest, greedy_verify, inverse_cdf, sample_verify, verify_step, AcceptanceStats  # noqa: F401
from .tiny_target import TinyTarget  # noqa: F401
from .spec_loop import greedy_generate, speculative_generate  # noqa: F401
