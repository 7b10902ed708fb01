// Kernel launchers of the denoising round (host-callable, enqueue on a stream).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace bdd {

// Cross-workgroup state of the selection kernel (one contiguous block of
// sel_sync_bytes(E) in the workspace, cleared by the router kernel).
typedef unsigned long long posmask_t;   // one bit per block position (kMaxT <= 64)
static_assert(kMaxT <= 64, "position masks are 64-bit");
struct SelSync {
  uint32_t *kslot;              // [E][kMaxT / 4] slot of the expert among position t's final picks (byte t % 4)
  unsigned long long *mass_fx;  // [E] block expert mass of the first picks, units of 2^-56
  posmask_t *mask1;             // [E] positions whose first picks include the expert
  posmask_t *mask2;             // [E] positions whose final picks include the expert
  int32_t *words;               // [0] positions counted (coreset)
};
// (the slot words first: 16-byte aligned rows of kMaxT bytes per expert)
inline size_t sel_sync_bytes(int E) { return (size_t)E * (kMaxT + 8 + 8 + 8) + 64; }
inline SelSync sel_sync_at(void *base, int E) {
  char *b = static_cast<char *>(base);
  SelSync s;
  s.kslot = reinterpret_cast<uint32_t *>(b);
  s.mass_fx = reinterpret_cast<unsigned long long *>(b + (size_t)E * kMaxT);
  s.mask1 = reinterpret_cast<posmask_t *>(b + (size_t)E * (kMaxT + 8));
  s.mask2 = reinterpret_cast<posmask_t *>(b + (size_t)E * (kMaxT + 16));
  s.words = reinterpret_cast<int32_t *>(b + (size_t)E * (kMaxT + 24));
  return s;
}

// Per-layer routing results and expert work lists, in the caller's workspace.
struct RouteBufs {
  float *logits;       // [H/128][T][E] router logit slices (bias not added)
  int32_t *idx;        // [T][K]   picked experts (-1 = unused slot)
  float *wgt;          // [T][K]   their renormalised weights
  int32_t *meta;       // [0] union size, [1] coreset size, [4] set if the wait for the positions' counts timed out
  uint32_t *cs_bits;   // [8]      coreset membership bitset
  float *mass;         // [E]      block expert mass (with the coreset)
  SelSync sync;        // selection kernel's cross-workgroup state
  int32_t *n_distinct_out;    // [1] union size copy (may be null)
  int32_t *coreset_size_out;  // [1] coreset size copy (may be null)
  const int32_t *gate;        // block resolved flag (may be null): the layer's kernels return when set
  int coreset;                // the selection took a coreset (else the gate/up kernel reports the union
                              // as the coreset)
};

// Upper bound of the routed token groups of a block: one per expert picked by
// 1 .. kTokGroup positions.
inline int expert_groups_max(int T, int E, int K) {
  const int picks = T * K;
  return E < picks ? E : picks;
}

// Upper bound of the dense experts (more than kTokGroup positions) of a block.
inline int expert_dense_max(int T, int E, int K) {
  const int d = T * K / (kTokGroup + 1);
  return d < E ? d : E;
}

// RMSNorm rows of `in` [T][H] into `out` (stored as wdtype); optionally copies
// `in` to `copy_out` and clears `zero_word`.
hipError_t launch_rmsnorm(int wdtype, const float *in, float *copy_out, void *out, void *xpk, int T, int H,
                          int32_t *zero_word, const int32_t *gate, hipStream_t s);

// Router logits from the normalised block, as partial sums over hidden slices
// (part [router_slices(H)][T][E]); clears zero_words words at zero_base (the
// selection kernel's state).
int router_slices(int H);
hipError_t launch_router(int wdtype, const void *xhat, uint32_t *zero_base, int zero_words, const void *w_router,
                         float *part, int T, int H, int E, const int32_t *gate, hipStream_t s);

// Selection: one workgroup per position (logits = slices summed in order +
// bias) and the coreset (r.sync must have been cleared by the router kernel);
// it leaves the final picks in r.idx / r.wgt and, per expert, the positions
// that picked it (sync.mask2) with the pick slots (sync.kslot), from which
// the expert kernels build their work lists.  Workgroups past the positions
// compute the shared expert's gate/up from the packed block `xpk` into its
// packed activation slot `act_shared`.
hipError_t launch_route_select(const RouteBufs &r, const float *bias, int T, int H, int E, int K, float top_p,
                               int wdtype, const void *xpk, const void *ws_gate_up, void *act_shared, int Is,
                               hipStream_t s);

hipError_t launch_coreset(const float *prob, const int32_t *idx, int T, int E, int K, float top_p,
                          uint32_t *bits, int32_t *size, float *mass, hipStream_t s);

// Expert FFNs.  Token groups: A [T*K][Imax] fp32 activations (row t*K + k);
// dense experts and the shared expert: packed activation slots in `act`
// (Imax * kActSlotPerI bytes each; slot 0 the shared expert, slot 1 + d the
// d-th dense expert in ascending id).  P [T*K + T][H] fp32 unweighted
// outputs (rows t*K + k routed, T*K + t shared).  The gate/up kernel's first
// workgroup reports the union size (and, without a coreset, the union as the
// coreset).
int expert_items_max(int T, int H, int E, int K, int I, int Is, bool gateup, bool int4);
hipError_t launch_expert_gateup(int wdtype, const void *xhat, const void *xpk, const void *w_gate_up,
                                const RouteBufs &r, float *A, void *act, int T, int H, int E, int K, int I,
                                int Imax, int grid, hipStream_t s);
hipError_t launch_expert_down(int wdtype, const float *A, const void *act, const void *w_down, const void *ws_down,
                              const RouteBufs &r, float *P, int T, int H, int E, int K, int I, int Is, int Imax,
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
                         int32_t *choice, int32_t *round_info, hipStream_t s, const int32_t *gate = nullptr,
                         int32_t *resolved_flag = nullptr);

}  // namespace bdd
