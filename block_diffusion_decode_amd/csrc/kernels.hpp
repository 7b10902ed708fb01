// Kernel launchers of the denoising round (host-callable, enqueue on a stream).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace bdd {

// Per-layer routing results and expert work lists, in the caller's workspace.
struct RouteBufs {
  float *logits;       // [T][E]   router logits (bias added)
  float *prob;         // [T][E]   softmax over all experts
  int32_t *idx;        // [T][K]   picked experts (-1 = unused slot)
  float *wgt;          // [T][K]   their renormalised weights
  int32_t *meta;       // [0] union size, [1] coreset size
  int32_t *union_list; // [E]      union experts, ascending id
  int32_t *slot_n;     // [E]      positions routed to each union expert
  int32_t *slot_asg;   // [E][kMaxT] assignment ids t*K+k, ascending t
  uint32_t *cs_bits;   // [8]      coreset membership bitset
  float *mass;         // [E]      block expert mass
  int32_t *n_distinct_out;    // [1] union size copy (may be null)
  int32_t *coreset_size_out;  // [1] coreset size copy (may be null)
};

struct ExpertBufs {
  float *A;    // [T*K][I]   SwiGLU activations of each (position, pick)
  float *A_s;  // [T][I_s]   shared-expert activations
  float *P;    // [T*K][H]   weighted expert outputs of each (position, pick)
  float *P_s;  // [T][H]     shared-expert outputs
};

// RMSNorm rows of `in` [T][H] into `out` (stored as wdtype); optionally copies
// `in` to `copy_out` and clears `zero_word`.
hipError_t launch_rmsnorm(int wdtype, const float *in, float *copy_out, void *out, int T, int H,
                          int32_t *zero_word, hipStream_t s);

// Router logits from the normalised block; clears zero_word.
size_t router_lds_bytes(int wdtype, int T, int H);
hipError_t launch_router(int wdtype, const void *xhat, int32_t *zero_word, const void *w_router,
                         const float *bias, float *logits, int T, int H, int E, hipStream_t s);

// Selection: one workgroup per position, then the block-level steps in the
// last one.  sorted_ids [T][E] scratch; done_count must be zero (the router
// kernel clears it) and is left zero.
hipError_t launch_route_select(const RouteBufs &r, int T, int E, int K, float top_p,
                               int32_t *sorted_ids, int32_t *done_count, hipStream_t s);

hipError_t launch_coreset(const float *prob, const int32_t *idx, int T, int E, int K, float top_p,
                          uint32_t *bits, int32_t *size, float *mass, hipStream_t s);

hipError_t launch_routed_gateup(int wdtype, const void *xhat, const void *w_gate_up,
                                const RouteBufs &r, float *A, int T, int H, int E, int K, int I,
                                int grid, hipStream_t s);

hipError_t launch_routed_down(int wdtype, const float *A, const void *w_down, const RouteBufs &r,
                              float *P, int H, int E, int K, int I, int grid, hipStream_t s);

hipError_t launch_shared_gateup(int wdtype, const void *xhat, const void *ws_gate_up, float *A_s,
                                int T, int H, int I_s, hipStream_t s);

hipError_t launch_shared_down(int wdtype, const float *A_s, const void *ws_down, float *P_s, int T,
                              int H, int I_s, hipStream_t s);

// y_t = sum_k P[t*K+k] (slots with idx >= 0) + P_s[t] (if non-null).  Then
// optionally h += y, and optionally out = RMSNorm(h or y) stored as wdtype.
hipError_t launch_combine(int wdtype, const float *P, const float *P_s, const int32_t *idx,
                          float *h, float *y_out, void *xhat_out, int T, int H, int K,
                          hipStream_t s);

// LM head online softmax: per (position, workgroup) partial (max, sum, argmax),
// stored [T][grid].
int lmhead_grid(int cus);
size_t lmhead_packed_bytes(int wdtype, int H, int V);
hipError_t launch_pack_lm(int wdtype, const void *w_lm, int V, int H, void *packed, hipStream_t s);
size_t lmhead_lds_bytes(int wdtype, int T, int H);
// Commit fused into the LM head's last workgroup (done_count must be zero).
struct LmCommit {
  int32_t *done_count;
  float threshold;
  int32_t *tokens;
  float *conf;
  int32_t *choice;
  int32_t *round_info;
};
hipError_t launch_lmhead(int wdtype, const void *hhat, const void *w_lm_packed, int T, int H, int V,
                         float *part_m, float *part_s, int32_t *part_i, int grid, const LmCommit *fused,
                         hipStream_t s);

hipError_t launch_commit(const float *part_m, const float *part_s, const int32_t *part_i,
                         int nparts, int T, float threshold, int32_t *tokens, float *conf,
                         int32_t *choice, int32_t *round_info, hipStream_t s);

}  // namespace bdd
