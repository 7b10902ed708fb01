// C ABI of the denoising round: argument checks, workspace planning and the
// launch sequences.  Every step runs in the kernels of this library.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/bdd.h"
#include "kernels.hpp"

namespace {

using namespace bdd;

thread_local char g_err[512] = "";

bdd_status fail(bdd_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess) return fail(BDD_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// ----------------------------------------------------------------- kernel timing
// Optional hipEvent pairs around every launch whose name contains the filter
// (measurement tools only; not thread-safe; off by default).
struct TimingRec {
  const char *name;
  hipEvent_t a, b;
};
bool g_timing = false;
std::string g_filter;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t pool_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

bool timing_wants(const char *name) {
  return g_timing && (g_filter.empty() || strstr(name, g_filter.c_str()) != nullptr);
}

#define LAUNCH(name, stream, expr)                                               \
  do {                                                                           \
    const bool rec_ = timing_wants(name);                                        \
    hipEvent_t a_ = nullptr, b_ = nullptr;                                       \
    if (rec_ && (a_ = pool_event()) != nullptr) HIP_TRY(hipEventRecord(a_, stream)); \
    HIP_TRY(expr);                                                               \
    if (a_ && (b_ = pool_event()) != nullptr) {                                  \
      HIP_TRY(hipEventRecord(b_, stream));                                       \
      g_recs.push_back({name, a_, b_});                                          \
    }                                                                            \
  } while (0)

constexpr int kMaxLmGrid = 1024;
constexpr int kGateupWgPerCu = 4;   // persistent workgroups per CU (register budget: 4 waves per SIMD)
constexpr int kDownWgPerCu = 3;     // (3 waves per SIMD)

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }
// bytes of a stored normalised activation (bf16 for the bf16 and 4-bit layers)
int esize(int wdtype) { return wdtype == BDD_F32 ? 4 : 2; }
// dtype of the activations and the router: the 4-bit layers keep both in bf16
int act_dtype(int wdtype) { return wdtype == BDD_INT4 ? BDD_BF16 : wdtype; }

int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

bdd_status check_dims(const bdd_moe_dims *d) {
  if (!d) return fail(BDD_ERR_INVALID_ARG, "dims is NULL");
  if (d->wdtype != BDD_F32 && d->wdtype != BDD_BF16 && d->wdtype != BDD_INT4)
    return fail(BDD_ERR_INVALID_ARG, "wdtype %d is not BDD_F32, BDD_BF16 or BDD_INT4", d->wdtype);
  if (d->T < 1 || d->H < 1 || d->E < 1 || d->K < 1 || d->I < 1 || d->I_shared < 0)
    return fail(BDD_ERR_INVALID_ARG, "non-positive size in dims (T=%d H=%d E=%d K=%d I=%d I_shared=%d)",
                d->T, d->H, d->E, d->K, d->I, d->I_shared);
  if (d->K > d->E) return fail(BDD_ERR_INVALID_ARG, "K=%d exceeds E=%d", d->K, d->E);
  if (d->T > kMaxT) return fail(BDD_ERR_UNSUPPORTED, "T=%d exceeds %d", d->T, kMaxT);
  if (d->E > kMaxE) return fail(BDD_ERR_UNSUPPORTED, "E=%d exceeds %d", d->E, kMaxE);
  if (d->K > 32) return fail(BDD_ERR_UNSUPPORTED, "K=%d exceeds 32", d->K);
  if (d->H % 128 || d->I % 32 || d->I_shared % 32)
    return fail(BDD_ERR_UNSUPPORTED, "H=%d must be a multiple of 128, I=%d and I_shared=%d of 32", d->H,
                d->I, d->I_shared);
  if (d->H > 8192 || d->I > 8192 || d->I_shared > 8192)
    return fail(BDD_ERR_UNSUPPORTED, "H, I, I_shared must be <= 8192");
  if (d->wdtype == BDD_INT4 && (d->I % 128 || d->I_shared % 128))
    return fail(BDD_ERR_UNSUPPORTED, "4-bit experts: I=%d and I_shared=%d must be multiples of 128", d->I,
                d->I_shared);
  return BDD_OK;
}

struct MoePlan {
  size_t logits, idx, wgt, meta, bits, mass, xhat, xpk, A, act, P;
  size_t sync;
  size_t end;
};

MoePlan plan_moe(const bdd_moe_dims &d, size_t base) {
  MoePlan p;
  size_t o = base;
  auto take = [&o](size_t bytes) { size_t at = o; o = a256(o + bytes); return at; };
  const size_t T = d.T, E = d.E, K = d.K, H = d.H, I = d.I, Is = d.I_shared;
  p.logits = take((size_t)router_slices(d.H) * T * E * 4);
  p.idx = take(T * K * 4);
  p.wgt = take(T * K * 4);
  p.meta = take(64);
  p.bits = take(32);
  p.mass = take(E * 4);
  p.xhat = take(T * H * esize(d.wdtype));
  p.xpk = take(T * H * esize(d.wdtype));
  // token-group activations, rows t*K + k
  p.A = take(T * K * (I > Is ? I : Is) * 4);
  // packed activation slots: the shared expert, then the dense experts
  p.act = take((size_t)(expert_dense_max(d.T, d.E, d.K) + 1) * (I > Is ? I : Is) * kActSlotPerI);
  // rows t*K + k of the routed picks, then T*K + t of the shared expert
  p.P = take((T * K + T) * H * 4);
  p.sync = take(sel_sync_bytes(d.E));
  p.end = o;
  return p;
}

struct LmPlan {
  size_t m, s, i, count, end;
};

LmPlan plan_lm(int T, size_t base) {
  LmPlan p;
  size_t o = base;
  auto take = [&o](size_t bytes) { size_t at = o; o = a256(o + bytes); return at; };
  p.m = take((size_t)kMaxLmGrid * T * 4);
  p.s = take((size_t)kMaxLmGrid * T * 4);
  p.i = take((size_t)kMaxLmGrid * T * 4);
  p.count = take(64);
  p.end = o;
  return p;
}

template <typename P>
P *at(void *ws, size_t off) { return reinterpret_cast<P *>(static_cast<char *>(ws) + off); }

bdd_status check_ws(void *ws, size_t have, size_t need) {
  if (need && !ws) return fail(BDD_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (have < need) return fail(BDD_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(BDD_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  return BDD_OK;
}

bdd_status check_weights(const bdd_moe_dims &d, const bdd_moe_weights *w, int layer) {
  if (!w) return fail(BDD_ERR_INVALID_ARG, "weights of layer %d are NULL", layer);
  if (!w->w_router || !w->w_gate_up || !w->w_down)
    return fail(BDD_ERR_INVALID_ARG, "layer %d: w_router, w_gate_up and w_down are required", layer);
  if (d.I_shared > 0 && (!w->ws_gate_up || !w->ws_down))
    return fail(BDD_ERR_INVALID_ARG, "layer %d: shared-expert weights are NULL but I_shared=%d", layer,
                d.I_shared);
  return BDD_OK;
}

bdd_status check_lm(int T, int H, int V, int dtype, float threshold) {
  if (dtype != BDD_F32 && dtype != BDD_BF16 && dtype != BDD_INT4)
    return fail(BDD_ERR_INVALID_ARG, "dtype %d", dtype);
  if (T < 1 || H < 1 || V < 1) return fail(BDD_ERR_INVALID_ARG, "T=%d H=%d V=%d", T, H, V);
  if (T > kMaxT) return fail(BDD_ERR_UNSUPPORTED, "T=%d exceeds %d", T, kMaxT);
  if (H % 32) return fail(BDD_ERR_UNSUPPORTED, "H=%d must be a multiple of 32", H);
  if (dtype == BDD_INT4 && H % 128) return fail(BDD_ERR_UNSUPPORTED, "INT4: H=%d must be a multiple of 128", H);
  if (!(threshold > 0.0f && threshold <= 1.0f))
    return fail(BDD_ERR_INVALID_ARG, "threshold %g outside (0, 1]", (double)threshold);
  if (lmhead_lds_bytes(dtype, T, H) > 144 * 1024)
    return fail(BDD_ERR_UNSUPPORTED, "T=%d, H=%d: block hidden states exceed the LDS budget", T, H);
  if ((long long)V * H >= (1ll << 40)) return fail(BDD_ERR_UNSUPPORTED, "V*H too large");
  return BDD_OK;
}

RouteBufs route_bufs(void *ws, const MoePlan &p) {
  RouteBufs r;
  r.logits = at<float>(ws, p.logits);
  r.idx = at<int32_t>(ws, p.idx);
  r.wgt = at<float>(ws, p.wgt);
  r.meta = at<int32_t>(ws, p.meta);
  r.cs_bits = at<uint32_t>(ws, p.bits);
  r.mass = at<float>(ws, p.mass);
  r.n_distinct_out = nullptr;
  r.coreset_size_out = nullptr;
  r.gate = nullptr;
  r.coreset = 0;
  return r;
}

// One MoE layer.  With h_in given, the layer first normalises it into xhat
// (copying it to h_copy and clearing lm_count when those are given); else
// xhat already holds the normalised block (and the workspace its packed
// copy).  combine: h += y and the next normalisation into xhat_next (and the
// packed copy when xpk_next) when h != nullptr, else y_out = y.
bdd_status moe_layer(const bdd_moe_dims &d, const bdd_moe_weights &w, float top_p, const float *h_in,
                     float *h_copy, void *xhat, RouteBufs r, const MoePlan &p, void *ws, float *h,
                     float *y_out, void *xhat_next, bool xpk_next, int32_t *lm_count, hipStream_t s) {
  const int T = d.T, H = d.H, E = d.E, K = d.K, I = d.I, Is = d.I_shared;
  const int Imax = I > Is ? I : Is;
  const int cus = device_cus();
  float *A = at<float>(ws, p.A), *P = at<float>(ws, p.P);
  void *xpk = at<void>(ws, p.xpk), *act = at<void>(ws, p.act);
  r.sync = sel_sync_at(at<void>(ws, p.sync), E);
  r.coreset = top_p < 1.0f ? 1 : 0;
  const int adt = act_dtype(d.wdtype);
  if (h_in) LAUNCH("rmsnorm", s, launch_rmsnorm(adt, h_in, h_copy, xhat, xpk, T, H, lm_count, r.gate, s));
  LAUNCH("router_logits", s, launch_router(adt, xhat, reinterpret_cast<uint32_t *>(at<void>(ws, p.sync)),
                                           (int)(sel_sync_bytes(E) / 4), w.w_router, r.logits, T, H, E, r.gate, s));
  LAUNCH("route_select", s, launch_route_select(r, w.router_bias, T, H, E, K, top_p, d.wdtype, xpk, w.ws_gate_up,
                                                act, Is, s));
  const bool i4 = d.wdtype == BDD_INT4;
  int g1 = expert_items_max(T, H, E, K, I, Is, true, i4), g2 = expert_items_max(T, H, E, K, I, Is, false, i4);
  g1 = g1 < cus * kGateupWgPerCu ? g1 : cus * kGateupWgPerCu;
  g2 = g2 < cus * kDownWgPerCu ? g2 : cus * kDownWgPerCu;
  LAUNCH("expert_gateup", s, launch_expert_gateup(d.wdtype, xhat, xpk, w.w_gate_up, r, A, act, T, H, E, K, I, Imax,
                                                  g1, s));
  LAUNCH("expert_down", s, launch_expert_down(d.wdtype, A, act, w.w_down, w.ws_down, r, P, T, H, E, K, I, Is, Imax,
                                              g2, s));
  LAUNCH("combine", s, launch_combine(adt, P, Is > 0 ? P + (size_t)T * K * H : nullptr, r.idx, r.wgt, h,
                                      y_out, xhat_next, xpk_next ? xpk : nullptr, T, H, K, r.gate, s));
  return BDD_OK;
}

}  // namespace

extern "C" {

const char *bdd_status_string(int32_t st) {
  switch (st) {
    case BDD_UNRESOLVED: return "BDD_UNRESOLVED";
    case BDD_OK: return "BDD_OK";
    case BDD_ERR_INVALID_ARG: return "BDD_ERR_INVALID_ARG";
    case BDD_ERR_UNSUPPORTED: return "BDD_ERR_UNSUPPORTED";
    case BDD_ERR_WORKSPACE: return "BDD_ERR_WORKSPACE";
    case BDD_ERR_HIP: return "BDD_ERR_HIP";
    default: return "unknown bdd_status";
  }
}

const char *bdd_last_error(void) { return g_err; }

int32_t bdd_device_cus(void) { return device_cus(); }

bdd_status bdd_timing_enable(int32_t on, const char *filter) {
  g_timing = on != 0;
  g_filter = filter ? filter : "";
  return BDD_OK;
}

int32_t bdd_timing_read(int32_t max_kernels, char *names, double *total_ms, int32_t *count) {
  if (max_kernels < 0 || (max_kernels > 0 && (!names || !total_ms || !count)))
    return fail(BDD_ERR_INVALID_ARG, "timing_read: bad output buffers");
  std::vector<std::string> seen;
  std::vector<double> tot;
  std::vector<int> cnt;
  hipError_t err = hipSuccess;
  for (const TimingRec &r : g_recs) {
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventSynchronize(r.b);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, r.a, r.b);
    size_t k = 0;
    while (k < seen.size() && seen[k] != r.name) ++k;
    if (k == seen.size()) { seen.push_back(r.name); tot.push_back(0.0); cnt.push_back(0); }
    tot[k] += ms;
    cnt[k] += 1;
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  if (err != hipSuccess) return fail(BDD_ERR_HIP, "timing_read: %s", hipGetErrorString(err));
  const int n = (int)seen.size() < max_kernels ? (int)seen.size() : max_kernels;
  for (int k = 0; k < n; ++k) {
    snprintf(names + 64 * k, 64, "%s", seen[k].c_str());
    total_ms[k] = tot[k];
    count[k] = cnt[k];
  }
  return (int32_t)seen.size();
}

size_t bdd_moe_workspace_bytes(const bdd_moe_dims *d) {
  if (check_dims(d) != BDD_OK) return 0;
  return plan_moe(*d, 0).end;
}

bdd_status bdd_moe_block_forward(const bdd_moe_dims *d, const bdd_moe_weights *w, const float *h,
                                 float coreset_top_p, float *y, void *xhat_out, int32_t *topk_idx,
                                 float *topk_w, int32_t *n_distinct, uint32_t *coreset_bits,
                                 int32_t *coreset_size, void *ws, size_t ws_bytes, void *stream) {
  bdd_status st = check_dims(d);
  if (st != BDD_OK) return st;
  if ((st = check_weights(*d, w, 0)) != BDD_OK) return st;
  if (!h || !y || !topk_idx || !topk_w || !n_distinct)
    return fail(BDD_ERR_INVALID_ARG, "h, y, topk_idx, topk_w and n_distinct are required");
  if (!(coreset_top_p > 0.0f)) return fail(BDD_ERR_INVALID_ARG, "coreset_top_p %g must be > 0", (double)coreset_top_p);
  const MoePlan p = plan_moe(*d, 0);
  if ((st = check_ws(ws, ws_bytes, p.end)) != BDD_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  RouteBufs r = route_bufs(ws, p);
  r.idx = topk_idx;
  r.wgt = topk_w;
  if (coreset_bits) r.cs_bits = coreset_bits;
  r.n_distinct_out = n_distinct;
  r.coreset_size_out = coreset_size;
  void *xhat = xhat_out ? xhat_out : at<void>(ws, p.xhat);
  return moe_layer(*d, *w, coreset_top_p >= 1.0f ? 1.0f : coreset_top_p, h, nullptr, xhat, r, p, ws,
                   nullptr, y, nullptr, false, nullptr, s);
}

bdd_status bdd_coreset_select(const float *router_prob, const int32_t *topk_idx, int32_t T, int32_t E,
                              int32_t K, float top_p, uint32_t *coreset_bits, int32_t *coreset_size,
                              float *expert_mass, void *stream) {
  if (!router_prob || !topk_idx || !coreset_bits || !coreset_size)
    return fail(BDD_ERR_INVALID_ARG, "router_prob, topk_idx, coreset_bits and coreset_size are required");
  if (T < 1 || E < 1 || K < 1 || K > E) return fail(BDD_ERR_INVALID_ARG, "T=%d E=%d K=%d", T, E, K);
  if (T > kMaxT || E > kMaxE || K > 32) return fail(BDD_ERR_UNSUPPORTED, "T=%d E=%d K=%d", T, E, K);
  if (!(top_p > 0.0f)) return fail(BDD_ERR_INVALID_ARG, "top_p %g must be > 0", (double)top_p);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  LAUNCH("coreset", s, launch_coreset(router_prob, topk_idx, T, E, K, top_p >= 1.0f ? 1.0f : top_p,
                                      coreset_bits, coreset_size, expert_mass, s));
  return BDD_OK;
}

size_t bdd_lmhead_packed_bytes(int32_t V, int32_t H, int32_t dtype) {
  if (V < 1 || H < 1 || H % 32 || (dtype != BDD_F32 && dtype != BDD_BF16 && dtype != BDD_INT4)) return 0;
  if (dtype == BDD_INT4 && H % 128) return 0;
  return lmhead_packed_bytes(dtype, H, V);
}

bdd_status bdd_lmhead_pack_int4(const void *codes, const void *scales, int32_t V, int32_t H, void *w_packed,
                                void *stream) {
  if (!codes || !scales || !w_packed) return fail(BDD_ERR_INVALID_ARG, "codes, scales and w_packed are required");
  if (V < 1 || H < 1) return fail(BDD_ERR_INVALID_ARG, "V=%d H=%d", V, H);
  if (H % 128) return fail(BDD_ERR_UNSUPPORTED, "H=%d must be a multiple of 128", H);
  if ((long long)V * H >= (1ll << 40)) return fail(BDD_ERR_UNSUPPORTED, "V*H too large");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  LAUNCH("pack_lm", s, launch_pack_lm_int4(codes, scales, V, H, w_packed, s));
  return BDD_OK;
}

size_t bdd_int4_packed_bytes(int32_t n_mats, int32_t rows, int32_t cols) {
  if (n_mats < 1 || rows < 1 || cols < 1 || rows % 16 || cols % 128) return 0;
  return (size_t)n_mats * lmhead_packed_bytes(BDD_INT4, cols, rows);
}

bdd_status bdd_pack_int4(const void *codes, const void *scales, int32_t n_mats, int32_t rows, int32_t cols,
                         void *packed, void *stream) {
  if (!codes || !scales || !packed) return fail(BDD_ERR_INVALID_ARG, "codes, scales and packed are required");
  if (n_mats < 1 || rows < 1 || cols < 1)
    return fail(BDD_ERR_INVALID_ARG, "n_mats=%d rows=%d cols=%d", n_mats, rows, cols);
  if (rows % 16 || cols % 128)
    return fail(BDD_ERR_UNSUPPORTED, "rows=%d must be a multiple of 16 and cols=%d of 128", rows, cols);
  if ((long long)rows * cols >= (1ll << 31)) return fail(BDD_ERR_UNSUPPORTED, "rows*cols too large");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t mb = lmhead_packed_bytes(BDD_INT4, cols, rows);
  const size_t cb = (size_t)rows * (cols / 2), sb = (size_t)rows * (cols / 128) * 2;
  for (int m = 0; m < n_mats; ++m)
    LAUNCH("pack_lm", s, launch_pack_lm_int4(static_cast<const char *>(codes) + m * cb,
                                             static_cast<const char *>(scales) + m * sb, rows, cols,
                                             static_cast<char *>(packed) + m * mb, s));
  return BDD_OK;
}

bdd_status bdd_lmhead_pack(const void *w_lm, int32_t V, int32_t H, int32_t dtype, void *w_packed,
                           void *stream) {
  if (!w_lm || !w_packed) return fail(BDD_ERR_INVALID_ARG, "w_lm and w_packed are required");
  if (dtype != BDD_F32 && dtype != BDD_BF16) return fail(BDD_ERR_INVALID_ARG, "dtype %d", dtype);
  if (V < 1 || H < 1) return fail(BDD_ERR_INVALID_ARG, "V=%d H=%d", V, H);
  if (H % 32) return fail(BDD_ERR_UNSUPPORTED, "H=%d must be a multiple of 32", H);
  if ((long long)V * H >= (1ll << 40)) return fail(BDD_ERR_UNSUPPORTED, "V*H too large");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  LAUNCH("pack_lm", s, launch_pack_lm(dtype, w_lm, V, H, w_packed, s));
  return BDD_OK;
}

size_t bdd_lmhead_workspace_bytes(int32_t T, int32_t H, int32_t V) {
  if (T < 1 || T > kMaxT || H < 1 || V < 1) return 0;
  return plan_lm(T, 0).end;
}

bdd_status bdd_lmhead_confidence_commit(const void *hhat, const void *w_lm, int32_t T, int32_t H,
                                        int32_t V, int32_t dtype, float threshold, int32_t *tokens,
                                        float *conf, int32_t *choice, int32_t *round_info, void *ws,
                                        size_t ws_bytes, void *stream) {
  bdd_status st = check_lm(T, H, V, dtype, threshold);
  if (st != BDD_OK) return st;
  if (!hhat || !w_lm || !tokens || !conf || !choice || !round_info)
    return fail(BDD_ERR_INVALID_ARG, "hhat, w_lm, tokens, conf, choice and round_info are required");
  const LmPlan p = plan_lm(T, 0);
  if ((st = check_ws(ws, ws_bytes, p.end)) != BDD_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int cus = device_cus();
  const int grid = lmhead_grid(cus, V) < kMaxLmGrid ? lmhead_grid(cus, V) : kMaxLmGrid;
  float *pm = at<float>(ws, p.m), *ps = at<float>(ws, p.s);
  int32_t *pi = at<int32_t>(ws, p.i);
  LAUNCH("lmhead", s, launch_lmhead(dtype, hhat, w_lm, T, H, V, pm, ps, pi, grid, nullptr, s));
  LAUNCH("commit", s, launch_commit(pm, ps, pi, grid, T, threshold, tokens, conf, choice, round_info, s));
  return BDD_OK;
}

size_t bdd_round_workspace_bytes(const bdd_moe_dims *d, int32_t V) {
  if (check_dims(d) != BDD_OK || V < 1) return 0;
  const MoePlan m = plan_moe(*d, 0);
  const size_t h_off = m.end;
  const LmPlan l = plan_lm(d->T, a256(h_off + (size_t)d->T * d->H * 4));
  return l.end;
}

}  // extern "C"

namespace {

// One round (the body of bdd_block_denoise_round and of its no-allocation
// variant): host checks first, then the launches on `stream`.
// With `gate` given, every kernel of the round returns at entry while *gate
// is set, and the commit sets *resolved_flag when it resolves the block.
bdd_status round_impl(const bdd_moe_dims *d, int32_t n_layers, const bdd_moe_weights *layers,
                      float coreset_top_p, const void *w_lm, int32_t V, float threshold, const float *x_in,
                      int32_t *tokens, float *conf, int32_t *choice, int32_t *round_info, int32_t *layer_topk_idx,
                      int32_t *layer_n_distinct, void *layer_xhat_out, void *hhat_out, void *ws, size_t ws_bytes,
                      void *stream, const int32_t *gate = nullptr, int32_t *resolved_flag = nullptr) {
  bdd_status st = check_dims(d);
  if (st != BDD_OK) return st;
  if (n_layers < 0) return fail(BDD_ERR_INVALID_ARG, "n_layers=%d", n_layers);
  if (n_layers > 0 && !layers) return fail(BDD_ERR_INVALID_ARG, "layers is NULL");
  for (int l = 0; l < n_layers; ++l)
    if ((st = check_weights(*d, &layers[l], l)) != BDD_OK) return st;
  if ((st = check_lm(d->T, d->H, V, d->wdtype, threshold)) != BDD_OK) return st;
  if (!w_lm || !x_in || !tokens || !conf || !choice || !round_info)
    return fail(BDD_ERR_INVALID_ARG, "w_lm, x_in, tokens, conf, choice and round_info are required");
  if (!(coreset_top_p > 0.0f)) return fail(BDD_ERR_INVALID_ARG, "coreset_top_p %g must be > 0", (double)coreset_top_p);
  const MoePlan p = plan_moe(*d, 0);
  const size_t h_off = p.end;
  const LmPlan lp = plan_lm(d->T, a256(h_off + (size_t)d->T * d->H * 4));
  if ((st = check_ws(ws, ws_bytes, lp.end)) != BDD_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int T = d->T, H = d->H, K = d->K;
  float *h = at<float>(ws, h_off);
  void *xhat = at<void>(ws, p.xhat);
  void *hhat = hhat_out ? hhat_out : xhat;
  const float tp = coreset_top_p >= 1.0f ? 1.0f : coreset_top_p;
  int32_t *count = at<int32_t>(ws, lp.count);
  if (n_layers == 0) {
    // the LM head reads RMSNorm(x_in); the norm kernel clears the counter
    LAUNCH("rmsnorm", s, launch_rmsnorm(act_dtype(d->wdtype), x_in, h, hhat, nullptr, T, H, count, gate, s));
  }
  // layer l's normalised input: the caller's buffer slot, else the workspace
  const size_t xbytes = (size_t)T * H * esize(d->wdtype);
  auto xin = [&](int l) -> void * {
    return layer_xhat_out ? static_cast<void *>(static_cast<char *>(layer_xhat_out) + (size_t)l * xbytes) : xhat;
  };
  for (int l = 0; l < n_layers; ++l) {
    RouteBufs r = route_bufs(ws, p);
    r.gate = gate;
    if (layer_topk_idx) r.idx = layer_topk_idx + (size_t)l * T * K;
    if (layer_n_distinct) r.n_distinct_out = layer_n_distinct + l;
    void *next = l + 1 == n_layers ? hhat : xin(l + 1);
    // layer 0 normalises x_in and keeps x_in as the residual
    if ((st = moe_layer(*d, layers[l], tp, l == 0 ? x_in : nullptr, l == 0 ? h : nullptr, xin(l), r, p, ws, h,
                        nullptr, next, l + 1 < n_layers, l == 0 ? count : nullptr, s)) != BDD_OK)
      return st;
  }
  const int cus = device_cus();
  const int grid = lmhead_grid(cus, V) < kMaxLmGrid ? lmhead_grid(cus, V) : kMaxLmGrid;
  float *pm = at<float>(ws, lp.m), *ps = at<float>(ws, lp.s);
  int32_t *pi = at<int32_t>(ws, lp.i);
  const LmCommit fused = {count, threshold, tokens, conf, choice, round_info, gate, resolved_flag};
  LAUNCH("lmhead", s, launch_lmhead(d->wdtype, hhat, w_lm, T, H, V, pm, ps, pi, grid, &fused, s));
  return BDD_OK;
}

// ----------------------------------------------------------------- no-allocation round
// Scratch of bdd_block_denoise_round_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): the device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and is kept here.
static __device__ __align__(256) unsigned char scratch[BDD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

bdd_status scratch_address(void **out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(BDD_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr) return fail(BDD_ERR_HIP, "hipGetSymbolAddress returned no address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BDD_OK;
}

}  // namespace

extern "C" {

bdd_status bdd_block_denoise_round(const bdd_moe_dims *d, int32_t n_layers,
                                   const bdd_moe_weights *layers, float coreset_top_p,
                                   const void *w_lm, int32_t V, float threshold, const float *x_in,
                                   int32_t *tokens, float *conf, int32_t *choice, int32_t *round_info,
                                   int32_t *layer_topk_idx, int32_t *layer_n_distinct,
                                   void *layer_xhat_out, void *hhat_out, void *ws, size_t ws_bytes,
                                   void *stream) {
  return round_impl(d, n_layers, layers, coreset_top_p, w_lm, V, threshold, x_in, tokens, conf, choice, round_info,
                    layer_topk_idx, layer_n_distinct, layer_xhat_out, hhat_out, ws, ws_bytes, stream);
}

bdd_status bdd_block_denoise_round_noalloc(const bdd_moe_dims *d, int32_t n_layers,
                                           const bdd_moe_weights *layers, float coreset_top_p,
                                           const void *w_lm, int32_t V, float threshold, const float *x_in,
                                           int32_t *tokens, float *conf, int32_t *choice,
                                           int32_t *round_info, int32_t *layer_topk_idx,
                                           int32_t *layer_n_distinct, void *layer_xhat_out, void *hhat_out,
                                           void *stream) {
  const size_t need = bdd_round_workspace_bytes(d, V);
  if (need == 0)   // invalid dims or V: the round's own checks name the problem
    return round_impl(d, n_layers, layers, coreset_top_p, w_lm, V, threshold, x_in, tokens, conf, choice,
                      round_info, layer_topk_idx, layer_n_distinct, layer_xhat_out, hhat_out, nullptr, 0, stream);
  if (need > (size_t)BDD_NOALLOC_SCRATCH_BYTES)
    return fail(BDD_ERR_UNSUPPORTED, "these dims need %zu bytes of scratch; the static scratch holds %zu", need,
                (size_t)BDD_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  const bdd_status st = scratch_address(&ws);
  if (st != BDD_OK) return st;
  return round_impl(d, n_layers, layers, coreset_top_p, w_lm, V, threshold, x_in, tokens, conf, choice, round_info,
                    layer_topk_idx, layer_n_distinct, layer_xhat_out, hhat_out, ws, BDD_NOALLOC_SCRATCH_BYTES,
                    stream);
}

// ----------------------------------------------------------------- generation
// The request bound of the generation controls: prompt plus generated tokens,
// counting the whole final block, at most this many.
constexpr long long kMaxRequestTokens = 131072;

int32_t bdd_generate_fits(int32_t prompt_len, int32_t max_new_tokens, int32_t block_size) {
  if (prompt_len < 0 || max_new_tokens < 1 || block_size < 1) return 0;
  const long long blocks = ((long long)max_new_tokens + block_size - 1) / block_size;
  return (long long)prompt_len + blocks * block_size <= kMaxRequestTokens ? 1 : 0;
}

size_t bdd_generate_workspace_bytes(const bdd_moe_dims *d, int32_t V) {
  const size_t r = bdd_round_workspace_bytes(d, V);
  if (r == 0) return 0;
  // after the round's workspace: conf [T] f32 and choice [T] i32, one
  // round_info slot [4] i32 per round of a block (at most kMaxT rounds), the
  // block's resolved flag
  return a256(r) + a256((size_t)d->T * 8) + a256((size_t)kMaxT * 16) + 256;
}

bdd_status bdd_generate(const bdd_moe_dims *d, int32_t n_layers, const bdd_moe_weights *layers,
                        float coreset_top_p, const void *w_lm, int32_t V, float threshold, int32_t max_steps,
                        int32_t rounds_per_read, int32_t prompt_len, int32_t max_new_tokens, int32_t eos_token,
                        const float *x_rounds, int32_t n_blocks, int32_t *out_tokens, int32_t *block_rounds,
                        int32_t *block_fallbacks, int32_t *result, void *ws, size_t ws_bytes, void *stream) {
  bdd_status st = check_dims(d);
  if (st != BDD_OK) return st;
  if (!bdd_generate_fits(prompt_len, max_new_tokens, d->T))
    return fail(BDD_ERR_INVALID_ARG,
                "request of %d prompt tokens + %d new tokens (whole blocks of %d) exceeds %lld tokens", prompt_len,
                max_new_tokens, d->T, kMaxRequestTokens);
  if (max_steps < 1) return fail(BDD_ERR_INVALID_ARG, "max_steps=%d", max_steps);
  if (rounds_per_read < 0) return fail(BDD_ERR_INVALID_ARG, "rounds_per_read=%d", rounds_per_read);
  const int T = d->T, H = d->H;
  const int need_blocks = (max_new_tokens + T - 1) / T;
  if (n_blocks < need_blocks)
    return fail(BDD_ERR_INVALID_ARG, "%d blocks of round inputs given, %d needed for %d new tokens", n_blocks,
                need_blocks, max_new_tokens);
  if (!x_rounds || !out_tokens || !block_rounds || !result)
    return fail(BDD_ERR_INVALID_ARG, "x_rounds, out_tokens, block_rounds and result are required");
  const size_t r_bytes = bdd_round_workspace_bytes(d, V);
  if (r_bytes == 0) return fail(BDD_ERR_INVALID_ARG, "bad dims or V");
  if ((st = check_ws(ws, ws_bytes, bdd_generate_workspace_bytes(d, V))) != BDD_OK) return st;
  char *tail = static_cast<char *>(ws) + a256(r_bytes);
  float *conf = reinterpret_cast<float *>(tail);
  int32_t *choice = reinterpret_cast<int32_t *>(tail + (size_t)T * 4);
  int32_t *slots = reinterpret_cast<int32_t *>(tail + a256((size_t)T * 8));
  int32_t *flag = reinterpret_cast<int32_t *>(tail + a256((size_t)T * 8) + a256((size_t)kMaxT * 16));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Every round commits at least one masked position, so a block resolves
  // within T rounds: at most min(max_steps, T) rounds run.  Each round is
  // gated on the block's resolved flag, so a round enqueued after the
  // resolving one returns at once.
  const int R = max_steps < T ? max_steps : T;
  result[0] = result[1] = result[2] = 0;
  // rounds_per_read == 0: the host keeps one round ahead of the one whose
  // info it reads (copied to pinned host memory, waited for on an event), so
  // the GPU runs back to back and at most one gated round per block is spent
  thread_local int32_t *pinned = nullptr;
  thread_local hipEvent_t evs[2] = {nullptr, nullptr};
  if (rounds_per_read == 0) {
    if (!pinned) HIP_TRY(hipHostMalloc(reinterpret_cast<void **>(&pinned), (size_t)kMaxT * 16));
    for (hipEvent_t &e : evs)
      if (!e) HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  }
  int produced = 0;
  for (int b = 0; b < need_blocks; ++b) {
    int32_t *tok = out_tokens + (size_t)b * T;
    LAUNCH("block_start", s, launch_block_start(tok, T, slots, 4 * R, flag, s));
    auto enqueue = [&](int r) -> bdd_status {
      const float *x = x_rounds + ((size_t)b * max_steps + r) * T * H;
      return round_impl(d, n_layers, layers, coreset_top_p, w_lm, V, threshold, x, tok, conf, choice, slots + 4 * r,
                        nullptr, nullptr, nullptr, nullptr, ws, r_bytes, stream, flag, flag);
    };
    int32_t info[kMaxT][4];
    int32_t last = 0;
    int rounds = 0, fallbacks = 0;
    bool resolved = false;
    if (rounds_per_read == 0) {
      auto enqueue_and_copy = [&](int r) -> bdd_status {
        const bdd_status st2 = enqueue(r);
        if (st2 != BDD_OK) return st2;
        HIP_TRY(hipMemcpyAsync(pinned + 4 * r, slots + 4 * r, 16, hipMemcpyDeviceToHost, s));
        HIP_TRY(hipEventRecord(evs[r & 1], s));
        return BDD_OK;
      };
      if ((st = enqueue_and_copy(0)) != BDD_OK) return st;
      for (int r = 0; r < R && !resolved; ++r) {
        if (r + 1 < R && (st = enqueue_and_copy(r + 1)) != BDD_OK) return st;
        HIP_TRY(hipEventSynchronize(evs[r & 1]));
        rounds = r + 1;
        fallbacks += pinned[4 * r + 1];
        resolved = pinned[4 * r + 3] != 0;
      }
      HIP_TRY(hipMemcpyAsync(&last, tok + T - 1, 4, hipMemcpyDeviceToHost, s));
      HIP_TRY(hipStreamSynchronize(s));
    } else {
      for (int r0 = 0; r0 < R && !resolved; r0 += rounds_per_read) {
        const int r1 = r0 + rounds_per_read < R ? r0 + rounds_per_read : R;
        for (int r = r0; r < r1; ++r)
          if ((st = enqueue(r)) != BDD_OK) return st;
        HIP_TRY(hipMemcpyAsync(info[0], slots, (size_t)r1 * 16, hipMemcpyDeviceToHost, s));
        HIP_TRY(hipMemcpyAsync(&last, tok + T - 1, 4, hipMemcpyDeviceToHost, s));
        HIP_TRY(hipStreamSynchronize(s));
        for (int r = r0; r < r1 && !resolved; ++r) {
          rounds = r + 1;
          fallbacks += info[r][1];
          resolved = info[r][3] != 0;
        }
      }
    }
    block_rounds[b] = rounds;
    if (block_fallbacks) block_fallbacks[b] = fallbacks;
    result[1] = b + 1;
    if (!resolved) return fail(BDD_UNRESOLVED, "block %d still has masked positions after %d rounds", b, R);
    produced += T;
    result[0] = produced < max_new_tokens ? produced : max_new_tokens;
    if (last == eos_token) {
      result[2] = 1;
      return BDD_OK;
    }
  }
  result[2] = 0;
  return BDD_OK;
}

struct bdd_round_graph_s {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

bdd_status bdd_round_graph_create(const bdd_moe_dims *d, int32_t n_layers, const bdd_moe_weights *layers,
                                  float coreset_top_p, const void *w_packed, int32_t V, float threshold,
                                  const float *x_in, int32_t *tokens, float *conf, int32_t *choice,
                                  int32_t *round_info, int32_t *layer_topk_idx, int32_t *layer_n_distinct,
                                  void *layer_xhat_out, void *hhat_out, void *ws, size_t ws_bytes,
                                  bdd_round_graph *out) {
  if (!out) return fail(BDD_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  hipStream_t cs = nullptr;
  HIP_TRY(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  const bool timing = g_timing;
  g_timing = false;
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) {
    g_timing = timing;
    (void)hipStreamDestroy(cs);
    return fail(BDD_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
  }
  const bdd_status st = bdd_block_denoise_round(d, n_layers, layers, coreset_top_p, w_packed, V, threshold,
                                                x_in, tokens, conf, choice, round_info, layer_topk_idx,
                                                layer_n_distinct, layer_xhat_out, hhat_out, ws, ws_bytes, cs);
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(cs, &graph);
  g_timing = timing;
  (void)hipStreamDestroy(cs);
  if (st != BDD_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  if (e != hipSuccess) return fail(BDD_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return fail(BDD_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
  }
  *out = new bdd_round_graph_s{graph, exec};
  return BDD_OK;
}

bdd_status bdd_round_graph_launch(bdd_round_graph g, void *stream) {
  if (!g || !g->exec) return fail(BDD_ERR_INVALID_ARG, "graph is NULL");
  HIP_TRY(hipGraphLaunch(g->exec, reinterpret_cast<hipStream_t>(stream)));
  return BDD_OK;
}

void bdd_round_graph_destroy(bdd_round_graph g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  delete g;
}

}  // extern "C"
