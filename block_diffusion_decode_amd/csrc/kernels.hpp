// Kernel launchers of the denoising round (host-callable, enqueue on a stream).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace bdd {

// Per-layer routing results and expert work lists, in the caller's workspace.
struct RouteBufs {
  float *logits;       // [H/128][T][E] router logit slices (bias not added)
  float *prob;         // [T][E]   softmax over all experts
  int32_t *idx;        // [T][K]   picked experts (-1 = unused slot)
  float *wgt;          // [T][K]   their renormalised weights
  int32_t *meta;       // [0] union size, [1] coreset size, [2] token groups, [3] dense experts
  int32_t *union_list; // [E]      union experts, ascending id
  int32_t *glist;      // [expert_groups_max][8] token-group records (see the expert kernels)
  int32_t *dlist;      // [expert_dense_max][kDenseRec] dense-expert records
  uint32_t *cs_bits;   // [8]      coreset membership bitset
  float *mass;         // [E]      block expert mass
  int32_t *n_distinct_out;    // [1] union size copy (may be null)
  int32_t *coreset_size_out;  // [1] coreset size copy (may be null)
  const int32_t *gate;        // block resolved flag (may be null): the layer's kernels return when set
};

// Upper bound of the routed token groups (kTokGroup positions of one expert)
// of a block: sum over union experts of ceil(n_e / kTokGroup).
inline int expert_groups_max(int T, int E, int K) {
  const int picks = T * K;
  return (E < picks ? E : picks) + (picks + kTokGroup - 1) / kTokGroup;
}

// Upper bound of the dense experts (more than kTokGroup positions) of a block,
// and the words of one dense record: expert, positions, 6 spare words, then
// one word per position.
constexpr int kDenseRec = 8 + kMaxT;
inline int expert_dense_max(int T, int E, int K) {
  const int d = T * K / (kTokGroup + 1);
  return d < E ? d : E;
}

// RMSNorm rows of `in` [T][H] into `out` (stored as wdtype); optionally copies
// `in` to `copy_out` and clears `zero_word`.
hipError_t launch_rmsnorm(int wdtype, const float *in, float *copy_out, void *out, void *xpk, int T, int H,
                          int32_t *zero_word, const int32_t *gate, hipStream_t s);

// Router logits from the normalised block, as partial sums over hidden slices
// (part [router_slices(H)][T][E]); clears zero_word.
int router_slices(int H);
hipError_t launch_router(int wdtype, const void *xhat, int32_t *zero_word, const void *w_router,
                         float *part, int T, int H, int E, const int32_t *gate, hipStream_t s);

// Selection: one workgroup per position (logits = slices summed in order +
// bias), then the block-level steps in the last one; workgroups past the
// positions compute the shared expert's gate/up from the packed block `xpk`
// into its packed activation slot `act_shared`.  sorted_ids [T][E] scratch;
// done_count must be zero (the router kernel clears it) and is left zero.
hipError_t launch_route_select(const RouteBufs &r, const float *bias, int T, int H, int E, int K, float top_p,
                               int32_t *sorted_ids, int32_t *done_count, int wdtype, const void *xpk,
                               const void *ws_gate_up, void *act_shared, int Is, hipStream_t s);

hipError_t launch_coreset(const float *prob, const int32_t *idx, int T, int E, int K, float top_p,
                          uint32_t *bits, int32_t *size, float *mass, hipStream_t s);

// Expert FFNs.  Token groups: A [T*K][Imax] fp32 activations (row t*K + k);
// dense experts and the shared expert: packed activation slots in `act`
// (Imax * 128 bytes each; slot 0 the shared expert, slot 1 + d dense record
// d).  P [T*K + T][H] fp32 unweighted outputs (rows t*K + k routed, T*K + t
// shared).
int expert_items_max(int T, int H, int E, int K, int I, int Is, bool gateup);
hipError_t launch_expert_gateup(int wdtype, const void *xhat, const void *xpk, const void *w_gate_up,
                                const RouteBufs &r, float *A, void *act, int T, int H, int I, int Imax, int grid,
                                hipStream_t s);
hipError_t launch_expert_down(int wdtype, const float *A, const void *act, const void *w_down, const void *ws_down,
                              const RouteBufs &r, float *P, int T, int H, int K, int I, int Is, int Imax,
                              int grid, hipStream_t s);

// y_t = sum_k wgt[t*K+k] * P[t*K+k] (slots with idx >= 0) + P_s[t] (if non-null).  Then
// optionally h += y, and optionally out = RMSNorm(h) stored as wdtype (and
// packed into xpk_out when given).
hipError_t launch_combine(int wdtype, const float *P, const float *P_s, const int32_t *idx,
                          const float *wgt, float *h, float *y_out, void *xhat_out, void *xpk_out, int T, int H,
                          int K, const int32_t *gate, hipStream_t s);

// LM head online softmax: per (position, workgroup) partial (max, sum, argmax),
// stored [T][grid].
int lmhead_grid(int cus, int V);
size_t lmhead_packed_bytes(int wdtype, int H, int V);
hipError_t launch_pack_lm(int wdtype, const void *w_lm, int V, int H, void *packed, hipStream_t s);
// 4-bit head (wdtype 2 in the LM-head calls): codes [V][H/2], scales [V][H/128] bf16.
hipError_t launch_pack_lm_int4(const void *codes, const void *scales, int V, int H, void *packed,
                               hipStream_t s);
size_t lmhead_lds_bytes(int wdtype, int T, int H);
// Commit fused into the LM head's last workgroup (done_count must be zero).
struct LmCommit {
  int32_t *done_count;
  float threshold;
  int32_t *tokens;
  float *conf;
  int32_t *choice;
  int32_t *round_info;
  const int32_t *gate;      // block resolved flag (may be null): the head returns at entry when set
  int32_t *resolved_flag;   // set to 1 when the commit resolves the block (may be null)
};
hipError_t launch_lmhead(int wdtype, const void *hhat, const void *w_lm_packed, int T, int H, int V,
                         float *part_m, float *part_s, int32_t *part_i, int grid, const LmCommit *fused,
                         hipStream_t s);

// Start of a block-resident block: tokens [T] = MASK, info [words] = 0, *flag = 0.
hipError_t launch_block_start(int32_t *tokens, int T, int32_t *info, int words, int32_t *flag, hipStream_t s);

hipError_t launch_commit(const float *part_m, const float *part_s, const int32_t *part_i,
                         int nparts, int T, float threshold, int32_t *tokens, float *conf,
                         int32_t *choice, int32_t *round_info, hipStream_t s);

}  // namespace bdd
