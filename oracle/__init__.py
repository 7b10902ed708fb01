"""CPU oracle for one block-diffusion denoising round.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU
baseline may import this package.  The HIP library never calls it, and it
imports nothing from the HIP path: the two share no code.

It is a plain NumPy float64 implementation of what the round computes,
written from these pages:
  [P1] aitujian.cn article on Clover-35B-A3B-Preview (Chinese): section 三
       (LowConfidence decoding loop, its rules, pseudocode and the toy
       fallback model), section 四 (backbone: 40 layers, 256 routed experts
       with top-8 routing and one shared expert per layer), section 五 (the
       block touches a union of experts).
  [P2] goremy.ai, "What Is Clover-35B-A3B? Block Diffusion on a Qwen3.6
       MoE": "How does confidence-threshold block decoding work?" and "What
       is the MoE coreset and why does it matter?".
  [P3] 10100.com article on Clover-35B-A3B-Preview, part 01 (structure).
  The generation loop follows [P1] 三 (block_decode: blocks after blocks,
  stop after a block ending in EOS) and [P2] "What generation controls ship
  by default?" (max_new_tokens is the hard limit; requests beyond 131072
  tokens including room for the final block are rejected).

Readings taken where the pages are silent (each listed in the design notes):
  * threshold test is ``conf >= threshold`` ([P1] 三 pseudocode);
  * accept and fallback act on still-masked positions only, so committed
    tokens never change ([P1] 三 rules; [P2] decoding loop step 2);
  * ties: lowest token id for the vocabulary argmax, lowest position for the
    fallback, lowest expert id for top-K and for the coreset ranking;
  * MASK is a sentinel (-1), never a vocabulary candidate;
  * router: softmax over all experts, top-K by logit, weights renormalised
    over the K selected ones;
  * expert FFN is SwiGLU, silu(z) = z / (1 + exp(-z));
  * the shared expert is added ungated;
  * pre-norm residual layer h + MoE(RMSNorm(h)), eps 1e-6, unit gain, and a
    final RMSNorm before the LM head;
  * coreset score = the raw softmax probability of each token's top-K picks;
    the coreset is the shortest prefix of experts ranked by summed score
    whose mass reaches top_p of the total; each token then re-takes its
    top-min(K, |C|) inside the coreset and renormalises;
  * generation stops after a block whose LAST token is EOS (the pseudocode
    tests block[-1]); max_new_tokens cuts the returned tokens but the final
    block is resolved whole; the history state is not modelled (the caller's
    forward receives the prefix and may ignore it);
  * INT4 weights (the format is not on the pages): two 4-bit codes per byte,
    low nibble first, code n standing for n - 8, one bf16 scale per row and
    128-column group.

Parity unpinned: the shared-expert gating, the coreset score choice, the
re-routing rule after the coreset and the Zipf router bias are readings the
pages print no numbers for; they are checked against the stated reading only.
"""

from .decode import (  # noqa: F401
    MASK,
    bf16_round,
    rmsnorm,
    silu,
    route,
    coreset_select,
    reroute,
    swiglu_expert,
    moe_layer,
    moe_given_routing,
    moe_stack,
    lm_head_confidence,
    INT4_GROUP,
    int4_dequantize,
    commit,
    resolve_block,
    MAX_REQUEST_TOKENS,
    request_fits,
    generate,
)
