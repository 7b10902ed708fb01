/*
 * bdd.h -- C ABI of the block-diffusion decode round on AMD MI355X (gfx950).
 *
 * One denoising round of a masked block, as the pages describe it:
 *   [P1] aitujian.cn article on Clover-35B-A3B-Preview (Chinese):
 *        section 三 (LowConfidence decoding loop: rules and pseudocode),
 *        section 四 (40 layers, 256 routed experts, top-8, one shared expert),
 *        section 五 (a 32-position block touches a union of experts).
 *   [P2] goremy.ai, "What Is Clover-35B-A3B? Block Diffusion on a Qwen3.6 MoE":
 *        "How does confidence-threshold block decoding work?" and
 *        "What is the MoE coreset and why does it matter?".
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a DEVICE pointer owned by the caller, dense
 *     and row-major in the layout stated.  The library keeps no pointer
 *     after a call returns and allocates no device memory: scratch space
 *     comes from the caller's workspace, sized by the *_workspace_bytes
 *     queries (256-byte aligned base required).
 *   - Weights are stored [out][in] (input dimension contiguous), in bf16
 *     (BDD_BF16) or fp32 (BDD_F32); arithmetic accumulates in fp32.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream)
 *     and return without waiting.  Outputs are valid once the stream has
 *     reached that point.  Every kernel of a call runs on `stream`.  Calls
 *     that share a workspace must not overlap.
 *   - Arguments are checked on the host before anything is enqueued; a
 *     failed check returns a negative status and enqueues nothing.  A
 *     launch failure returns BDD_ERR_HIP.  bdd_last_error() describes the
 *     last failure of the calling thread.  No exception crosses the ABI.
 *   - MASK is -1 and is never a vocabulary candidate.
 *   - Supported shapes: 1 <= T <= 64; 1 <= K <= min(E, 32); E <= 256; H a
 *     multiple of 128 for the MoE layer (of 32 for the LM head alone); I,
 *     I_shared multiples of 32; H <= 2048 for the LM head when T > 16 (the
 *     block's normalised hidden states are kept in the 160 KiB LDS of one CU;
 *     a block of more than 32 positions is kept half of H at a time, and the
 *     LM head still streams its weight once).
 */
#ifndef BDD_H
#define BDD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BDD_MASK (-1)

typedef enum {
  BDD_UNRESOLVED = 1,       /* bdd_generate: a block kept masked positions after max_steps rounds */
  BDD_OK = 0,
  BDD_ERR_INVALID_ARG = -1, /* null pointer, out-of-range size or parameter */
  BDD_ERR_UNSUPPORTED = -2, /* valid but outside the supported shapes      */
  BDD_ERR_WORKSPACE = -3,   /* workspace missing, too small or misaligned  */
  BDD_ERR_HIP = -4          /* a HIP runtime call or launch failed         */
} bdd_status;

/* BDD_INT4: 4-bit weight-only matrices ([P3] 10100.com article on
 * Clover-35B-A3B-Preview, part 03: an INT4 deployment; the pages give no
 * format, the one read here is): two codes per byte, the low nibble the even
 * column, a nibble n standing for n - 8, one bf16 scale per row and
 * 128-column group, w[r][c] = (n - 8) * scale[r][c / 128].  Packed by
 * bdd_pack_int4 (expert matrices) or bdd_lmhead_pack_int4 (LM head).  In a
 * 4-bit MoE layer the router and the activations stay bf16. */
typedef enum { BDD_F32 = 0, BDD_BF16 = 1, BDD_INT4 = 2 } bdd_dtype;

/* Shapes of one MoE layer and the block.  T block positions, H hidden, E
 * routed experts, K experts per token, I routed-expert intermediate,
 * I_shared shared-expert intermediate (0: no shared expert), wdtype the
 * storage type of every weight (a bdd_dtype). */
typedef struct {
  int32_t T, H, E, K, I, I_shared;
  int32_t wdtype;
} bdd_moe_dims;

/* Device pointers to one MoE layer's weights ([P1] section 四).
 *   w_router    [E][H]          router logits l = xhat W_r^T + b (bf16 when
 *                               wdtype is BDD_INT4)
 *   router_bias [E] fp32        may be NULL (no bias)
 *   w_gate_up   [E][2I][H]      expert e: rows 0..I-1 gate, I..2I-1 up
 *   w_down      [E][H][I]
 *   ws_gate_up  [2I_shared][H]  shared expert (ignored when I_shared == 0)
 *   ws_down     [H][I_shared]
 * With wdtype BDD_INT4 the four expert tensors are packed by bdd_pack_int4
 * (w_gate_up: E matrices of 2I x H, w_down: E matrices of H x I, the shared
 * expert's one each); I and I_shared must then be multiples of 128. */
typedef struct {
  const void *w_router;
  const float *router_bias;
  const void *w_gate_up;
  const void *w_down;
  const void *ws_gate_up;
  const void *ws_down;
} bdd_moe_weights;

/* round_info[4] written by the commit: number of positions written this
 * round, fallback flag (1 when no masked position reached the threshold and
 * the most confident one was forced), masked positions left, resolved flag. */
enum { BDD_RI_COMMITTED = 0, BDD_RI_FALLBACK = 1, BDD_RI_MASKED_LEFT = 2, BDD_RI_RESOLVED = 3 };

/* ------------------------------------------------------------------------ */

/* Workspace bytes bdd_moe_block_forward needs for these dims (0 if the dims
 * are invalid). */
size_t bdd_moe_workspace_bytes(const bdd_moe_dims *d);

/* One MoE FFN layer on a block ([P1] sections 四 and 五; [P2] coreset section).
 *   h        [T][H] fp32   block hidden states entering the layer (read only)
 *   The layer normalises h (RMSNorm, eps 1e-6, unit gain; stored as wdtype),
 *   routes each position to its top-K experts (softmax over all E router
 *   logits, K largest logits, ties to the lower expert id, weights
 *   renormalised over the K picks), optionally restricts routing to the
 *   block coreset, runs each expert of the union once over all positions
 *   routed to it (SwiGLU: silu(x W_g^T) * (x W_u^T), then W_d), adds the
 *   ungated shared expert, and combines:
 *     y_t = sum_k w_tk * Expert_{idx_tk}(xhat_t) + Shared(xhat_t).
 *   coreset_top_p  >= 1: no coreset.  In (0,1): each expert's mass is the sum
 *                  of the softmax scores of the positions that picked it; the
 *                  coreset is the shortest prefix of experts ranked by mass
 *                  (ties to the lower id) whose mass reaches top_p of the
 *                  total; each position then re-takes its min(K,|C|) largest
 *                  logits inside the coreset and renormalises.
 *   y          [T][H] fp32 out    the layer output (residual not added)
 *   xhat_out   [T][H] wdtype out  normalised input (may be NULL)
 *   topk_idx   [T][K] int32 out   picked experts in descending-logit order;
 *                                 -1 in slots beyond min(K,|C|)
 *   topk_w     [T][K] fp32 out    their weights (0 in unused slots)
 *   n_distinct [1] int32 out      size of the union of experts read
 *   coreset_bits [ceil(E/32)] uint32 out, coreset_size [1] int32 out:
 *                                 coreset membership bitset and size (both
 *                                 may be NULL; without coreset every expert
 *                                 with positive mass is reported) */
bdd_status bdd_moe_block_forward(const bdd_moe_dims *d, const bdd_moe_weights *w,
                                 const float *h, float coreset_top_p, float *y,
                                 void *xhat_out, int32_t *topk_idx, float *topk_w,
                                 int32_t *n_distinct, uint32_t *coreset_bits,
                                 int32_t *coreset_size, void *ws, size_t ws_bytes,
                                 void *stream);

/* Block coreset selection alone ([P2] "What is the MoE coreset"): from the
 * routing of a block, sum each expert's softmax scores over the positions
 * that picked it, rank experts by that mass (descending, ties to the lower
 * id) and keep the shortest ranked prefix reaching top_p of the total mass
 * (top_p >= 1: every expert with positive mass).
 *   router_prob [T][E] fp32   softmax scores p_te
 *   topk_idx    [T][K] int32  each position's picks (entries < 0 ignored)
 *   coreset_bits [ceil(E/32)] uint32 out, coreset_size [1] int32 out,
 *   expert_mass [E] fp32 out (may be NULL).
 * Needs no workspace. */
bdd_status bdd_coreset_select(const float *router_prob, const int32_t *topk_idx,
                              int32_t T, int32_t E, int32_t K, float top_p,
                              uint32_t *coreset_bits, int32_t *coreset_size,
                              float *expert_mass, void *stream);

/* Bytes of the packed LM-head weight (0 if the arguments are invalid).
 * BDD_INT4 needs H to be a multiple of 128. */
size_t bdd_lmhead_packed_bytes(int32_t V, int32_t H, int32_t dtype);

/* Packs the LM-head weight w_lm [V][H] (dtype) into the tile layout the LM
 * head streams, once, at load time: rows are grouped in tiles of 16, and for
 * each tile and each MFMA k-step (32 bf16 or 16 fp32 elements of the hidden
 * dimension) the 16 x k-step block is stored contiguously as 64 16-byte units,
 * unit l = li + 16 g holding row li, elements [kstep*s + g*c, kstep*s + g*c + c)
 * with c = 8 (bf16) or 4 (fp32).  Rows past V are zero.  w_packed must hold
 * bdd_lmhead_packed_bytes(V, H, dtype) bytes.  Same bytes as w_lm (plus the
 * padding of the last tile); every load of the LM head then reads a
 * contiguous KiB. */
bdd_status bdd_lmhead_pack(const void *w_lm, int32_t V, int32_t H, int32_t dtype, void *w_packed,
                           void *stream);

/* Bytes of n_mats packed 4-bit matrices of rows x cols (0 if invalid: rows a
 * multiple of 16, cols of 128). */
size_t bdd_int4_packed_bytes(int32_t n_mats, int32_t rows, int32_t cols);

/* Packs n_mats 4-bit weight matrices (the BDD_INT4 format) for the 4-bit
 * expert kernels, once, at load time:
 *   codes   device [n_mats][rows][cols/2] uint8 (byte j: columns 2j, 2j + 1)
 *   scales  device [n_mats][rows][cols/128] bf16
 *   packed  device out, bdd_int4_packed_bytes(n_mats, rows, cols) bytes: the
 *           matrices one after the other, each in 16-row tiles with, per
 *           tile and 128-column group, one KiB of codes in the order the MFMA
 *           lanes consume them (lane li + 16 g: row li, dword kk holding the
 *           codes of columns 32 (4 group + kk) + 8 g + e, e = 0..7, code e at
 *           bit 4 (e / 2) + 16 (e % 2)), then the scales as [tile][group][16].
 * Errors: BDD_ERR_INVALID_ARG (NULL pointer, non-positive size),
 * BDD_ERR_UNSUPPORTED (rows not a multiple of 16, cols not of 128). */
bdd_status bdd_pack_int4(const void *codes, const void *scales, int32_t n_mats, int32_t rows, int32_t cols,
                         void *packed, void *stream);

/* Packs a 4-bit weight-only LM head ([P3] 10100.com article on
 * Clover-35B-A3B-Preview, part 03, memory and quantisation: the model is
 * deployed in INT4; the pages give no format, so this one is assumed):
 *   codes   [V][H/2] uint8, device: byte j of row v holds columns 2j (low
 *           nibble) and 2j + 1 (high nibble); a nibble n stands for n - 8
 *   scales  [V][H/128] bf16, device: one scale per row and 128-column group
 *   weight w[v][c] = (n - 8) * scales[v][c / 128].
 * w_packed (device, bdd_lmhead_packed_bytes(V, H, BDD_INT4) bytes) receives,
 * per tile of 16 rows and group of 128 columns, one KiB of codes in the order
 * the LM head's lanes consume them (lane li + 16 g: row li, columns
 * 32 (4 group + kk) + 8 g + e for kk, e in 0..3, 0..7), then after all codes
 * the scales as [tile][group][16] bf16.  Rows past V get zero scales.
 * H must be a multiple of 128.  Runs on `stream`; the caller owns every
 * buffer.  Errors: BDD_ERR_INVALID_ARG (NULL pointer, V or H < 1),
 * BDD_ERR_UNSUPPORTED (H not a multiple of 128, V*H too large). */
bdd_status bdd_lmhead_pack_int4(const void *codes, const void *scales, int32_t V, int32_t H,
                                void *w_packed, void *stream);

/* Workspace bytes bdd_lmhead_confidence_commit needs. */
size_t bdd_lmhead_workspace_bytes(int32_t T, int32_t H, int32_t V);

/* LM head, confidence and LowConfidence commit ([P1] section 三 pseudocode
 * and rules; [P2] decoding-loop steps 2-4).
 *   hhat      [T][H] dtype  normalised final hidden states (bf16 when dtype
 *             is BDD_INT4)
 *   w_packed  the LM-head weight [V][H] (row v = token v) as packed by
 *             bdd_lmhead_pack, or by bdd_lmhead_pack_int4 (dtype BDD_INT4:
 *             logits of the dequantised weight, accumulated in fp32)
 *   For each position: logits z = hhat W_lm^T (never stored), conf = max
 *   softmax probability = 1 / sum_v exp(z_v - max z), choice = argmax (lowest
 *   token id on ties).  Then among positions whose token is MASK: every one
 *   with conf >= threshold is written with its choice; if none qualifies, the
 *   single most confident masked position (lowest index on ties) is written.
 *   Written tokens never change.
 *   tokens     [T] int32 in/out   MASK (-1) = not yet written
 *   conf       [T] fp32 out, choice [T] int32 out (all positions)
 *   round_info [4] int32 out      see BDD_RI_*
 *   threshold in (0, 1]. */
bdd_status bdd_lmhead_confidence_commit(const void *hhat, const void *w_packed, int32_t T,
                                        int32_t H, int32_t V, int32_t dtype,
                                        float threshold, int32_t *tokens, float *conf,
                                        int32_t *choice, int32_t *round_info, void *ws,
                                        size_t ws_bytes, void *stream);

/* Workspace bytes bdd_block_denoise_round needs.  (With wdtype BDD_INT4 the
 * round's LM head is a 4-bit head packed by bdd_lmhead_pack_int4.) */
size_t bdd_round_workspace_bytes(const bdd_moe_dims *d, int32_t V);

/* One full denoising round ([P1] section 三 pseudocode, one pass of the inner
 * loop): the block's hidden states go through n_layers MoE layers with the
 * mixer replaced by identity (h <- h + MoE(RMSNorm(h)), as in
 * bdd_moe_block_forward), a final RMSNorm stored as wdtype, the LM head and
 * the commit (as in bdd_lmhead_confidence_commit).
 *   layers       HOST array [n_layers] of device weight pointers
 *   x_in         [T][H] fp32 hidden states entering layer 0 (read only)
 *   w_packed     LM-head weight [V][H] wdtype, packed by bdd_lmhead_pack
 *   tokens, conf, choice, round_info as in bdd_lmhead_confidence_commit
 *   layer_topk_idx   [n_layers][T][K] int32 out (may be NULL)
 *   layer_n_distinct [n_layers] int32 out (may be NULL)
 *   layer_xhat_out   [n_layers][T][H] wdtype out: each layer's normalised
 *                    input, RMSNorm(h) as the layer consumes it (may be NULL)
 *   hhat_out     [T][H] wdtype out: the LM-head input (may be NULL) */
bdd_status bdd_block_denoise_round(const bdd_moe_dims *d, int32_t n_layers,
                                   const bdd_moe_weights *layers, float coreset_top_p,
                                   const void *w_packed, int32_t V, float threshold,
                                   const float *x_in, int32_t *tokens, float *conf,
                                   int32_t *choice, int32_t *round_info,
                                   int32_t *layer_topk_idx, int32_t *layer_n_distinct,
                                   void *layer_xhat_out, void *hhat_out, void *ws,
                                   size_t ws_bytes, void *stream);

/* The same round for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * arguments and results as bdd_block_denoise_round, without a workspace.
 * The scratch is a static device array of BDD_NOALLOC_SCRATCH_BYTES bytes
 * inside the library, one per GPU, held until the process ends; the call
 * allocates nothing (no hipMalloc, no hipFree).  Dims whose
 * bdd_round_workspace_bytes exceed it are rejected with BDD_ERR_UNSUPPORTED
 * before anything is enqueued.  Every call on a GPU shares that GPU's
 * scratch and leaves its contents behind (the round's kernels clear the
 * counters they need): calls that overlap on one GPU (on different streams
 * or from different threads) race and must not be issued. */
#define BDD_NOALLOC_SCRATCH_BYTES (32u << 20)
bdd_status bdd_block_denoise_round_noalloc(const bdd_moe_dims *d, int32_t n_layers,
                                           const bdd_moe_weights *layers, float coreset_top_p,
                                           const void *w_packed, int32_t V, float threshold,
                                           const float *x_in, int32_t *tokens, float *conf,
                                           int32_t *choice, int32_t *round_info,
                                           int32_t *layer_topk_idx, int32_t *layer_n_distinct,
                                           void *layer_xhat_out, void *hhat_out, void *stream);

/* One denoising round captured as a HIP graph, for callers that replay the
 * same round structure many times (a decode loop): the arguments are those of
 * bdd_block_denoise_round, bound at creation (device pointers, sizes and
 * scalars; the contents of the buffers are read at each launch).  The
 * round's kernels become the graph's nodes, in stream order.
 * Launching enqueues one whole round on `stream`.  The graph holds no
 * memset nodes.  Destroy with bdd_round_graph_destroy. */
typedef struct bdd_round_graph_s *bdd_round_graph;
bdd_status bdd_round_graph_create(const bdd_moe_dims *d, int32_t n_layers,
                                  const bdd_moe_weights *layers, float coreset_top_p,
                                  const void *w_packed, int32_t V, float threshold,
                                  const float *x_in, int32_t *tokens, float *conf,
                                  int32_t *choice, int32_t *round_info,
                                  int32_t *layer_topk_idx, int32_t *layer_n_distinct,
                                  void *layer_xhat_out, void *hhat_out, void *ws,
                                  size_t ws_bytes, bdd_round_graph *out);
bdd_status bdd_round_graph_launch(bdd_round_graph g, void *stream);
void bdd_round_graph_destroy(bdd_round_graph g);

/* Multi-block generation ([P1] section 三, the block_decode pseudocode, and
 * [P2] "How does confidence-threshold block decoding work?" step 6): blocks
 * of T positions start all-MASK and run rounds of bdd_block_denoise_round
 * until every position is committed; a finished block joins the prefix, and
 * generation stops after a block whose last token is eos_token, or once
 * max_new_tokens have been produced (the final block is always resolved
 * whole).  The mixer and its history state are not built: the caller
 * supplies each round's block input (the re-embedding stub).
 *   max_steps      rounds allowed per block (>= 1)
 *   rounds_per_read  how the host learns that a block is resolved.  Every
 *                  round commits at least one masked position, so at most
 *                  min(max_steps, T) rounds run, and each round's kernels
 *                  return at once when an earlier round of the block has
 *                  resolved it.  0: the host stays one round ahead (it
 *                  enqueues round r + 1, then waits for round r's info,
 *                  copied to pinned host memory), so the GPU never waits
 *                  for the host and at most one extra (empty) round runs per
 *                  block; k > 0: k rounds are enqueued back to back, then
 *                  the host reads their info (k >= max_steps: once per
 *                  block).  The library keeps one small pinned host buffer
 *                  and two events per calling thread for mode 0.
 *   prompt_len, max_new_tokens  the request; it is rejected (BDD_ERR_INVALID_ARG,
 *                  nothing enqueued) when prompt_len + max_new_tokens rounded
 *                  up to whole blocks exceeds 131072 tokens ([P2] "What
 *                  generation controls ship by default?"), see bdd_generate_fits
 *   x_rounds       device [n_blocks][max_steps][T][H] fp32: input of round r
 *                  of block b; n_blocks >= ceil(max_new_tokens / T)
 *   out_tokens     device [n_blocks][T] int32 out: the blocks' tokens
 *   block_rounds   HOST [n_blocks] int32 out: rounds each block took
 *   block_fallbacks  HOST [n_blocks] int32 out: its forced (fallback) rounds
 *                  (may be NULL)
 *   result         HOST [3] int32 out: tokens returned (those of the resolved
 *                  blocks, at most max_new_tokens), blocks run, stop (0
 *                  length, 1 eos_token)
 *   ws             bdd_generate_workspace_bytes(d, V) bytes
 * Returns BDD_UNRESOLVED (result filled up to that block, which is counted
 * in blocks run but not in tokens returned) when a block still has masked
 * positions after max_steps rounds. */
int32_t bdd_generate_fits(int32_t prompt_len, int32_t max_new_tokens, int32_t block_size);
size_t bdd_generate_workspace_bytes(const bdd_moe_dims *d, int32_t V);
bdd_status bdd_generate(const bdd_moe_dims *d, int32_t n_layers, const bdd_moe_weights *layers,
                        float coreset_top_p, const void *w_packed, int32_t V, float threshold,
                        int32_t max_steps, int32_t rounds_per_read, int32_t prompt_len,
                        int32_t max_new_tokens, int32_t eos_token, const float *x_rounds,
                        int32_t n_blocks, int32_t *out_tokens, int32_t *block_rounds,
                        int32_t *block_fallbacks, int32_t *result, void *ws, size_t ws_bytes,
                        void *stream);

/* Human-readable name of a status, and the calling thread's last error. */
const char *bdd_status_string(int32_t status);
const char *bdd_last_error(void);

/* Number of compute units of the current HIP device that the kernels size
 * their grids for. */
int32_t bdd_device_cus(void);

/* Kernel timing for measurement tools.  While enabled, every kernel launch of
 * this library whose name contains `filter` (NULL or "": all) is bracketed by
 * a pair of hipEvents recorded on the launching stream.  Kernel names:
 * rmsnorm, router_logits, route_select, coreset, expert_gateup, expert_down,
 * combine, lmhead, commit, pack_lm, block_start.  Not thread-safe. */
bdd_status bdd_timing_enable(int32_t on, const char *filter);

/* Waits for the recorded events, then for up to max_kernels distinct kernel
 * names writes the name (64-byte slots in `names`), the summed duration in ms
 * and the launch count, clears the records and returns the number of distinct
 * names (negative status on failure). */
int32_t bdd_timing_read(int32_t max_kernels, char *names, double *total_ms, int32_t *count);

#ifdef __cplusplus
}
#endif

#endif /* BDD_H */
