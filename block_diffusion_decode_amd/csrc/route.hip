// Normalisation, router, top-K selection, block coreset and expert work lists.
//
// Pages: [P1] aitujian.cn article on Clover-35B-A3B-Preview, section 四 (256
// routed experts, top-8, one shared expert) and section 五 (a block of 32
// positions touches a union of experts); [P2] goremy.ai "What Is
// Clover-35B-A3B? Block Diffusion on a Qwen3.6 MoE", section "What is the MoE
// coreset and why does it matter?" (aggregate each position's top-8 scores,
// rank experts, keep enough to cover top_p of the mass).
#include <float.h>
#include <limits.h>

#include "dense.hpp"
#include "kernels.hpp"

namespace bdd {

constexpr int kMaxK = 32;

// ------------------------------------------------------------------ RMSNorm
constexpr int kRowThreads = 512;
constexpr int kRowVec = 4;  // float4 per thread: H <= 4 * 4 * 512 = 8192

__device__ __forceinline__ float block_sum_512(float v, float *red8) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) red8[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kRowThreads / 64; ++w) t += red8[w];
  __syncthreads();
  return t;
}

template <typename OT>
__device__ __forceinline__ void store4(OT *out, size_t i, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float *out, size_t i, float4 v) {
  *reinterpret_cast<float4 *>(out + i) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *out, size_t i, float4 v) {
  *reinterpret_cast<uint2 *>(out + i) = make_uint2(pack2(f2bf(v.x), f2bf(v.y)), pack2(f2bf(v.z), f2bf(v.w)));
}

// x_hat = h / sqrt(mean(h^2) + eps), unit gain, one workgroup per position.
template <typename OT>
__global__ __launch_bounds__(kRowThreads) void rmsnorm_kernel(const float *__restrict__ in,
                                                              float *__restrict__ copy_out,
                                                              OT *__restrict__ out, int H, float eps) {
  __shared__ float red[kRowThreads / 64];
  const size_t base = (size_t)blockIdx.x * H;
  const int H4 = H / 4;
  float4 v[kRowVec];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < kRowVec; ++q) {
    const int j = threadIdx.x + q * kRowThreads;
    v[q] = j < H4 ? reinterpret_cast<const float4 *>(in + base)[j] : make_float4(0, 0, 0, 0);
    ss += v[q].x * v[q].x + v[q].y * v[q].y + v[q].z * v[q].z + v[q].w * v[q].w;
  }
  ss = block_sum_512(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int q = 0; q < kRowVec; ++q) {
    const int j = threadIdx.x + q * kRowThreads;
    if (j < H4) {
      if (copy_out) reinterpret_cast<float4 *>(copy_out + base)[j] = v[q];
      store4<OT>(out, base + 4 * (size_t)j,
                 make_float4(v[q].x * inv, v[q].y * inv, v[q].z * inv, v[q].w * inv));
    }
  }
}

// ------------------------------------------------------------------ router logits
// logits[t][e] = xhat_t . W_r[e] + b_e.  One workgroup per 16 experts; its
// waves split the hidden dimension and sum through LDS.
template <class W, int NT>
__global__ __launch_bounds__(512) void router_logits_kernel(const typename W::T *__restrict__ xhat,
                                                            const typename W::T *__restrict__ wr,
                                                            const float *__restrict__ bias,
                                                            float *__restrict__ logits, int T, int H,
                                                            int E) {
  __shared__ float red[8 * NT * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int row0 = blockIdx.x * 16;
  const int row = row0 + (lane & 15);
  const bool ok = row < E;
  int k0, k1;
  k_slice(H, mfma_kstep<W>(), wave, nw, k0, k1);
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  dense_acc_global<W, typename W::T, NT>(wr + (size_t)(ok ? row : 0) * H, ok, xhat, H, T, k0, k1,
                                         lane, acc);
  splitk_sum<NT>(acc, red, wave, nw, lane);
  if (wave == 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = row0 + 4 * (lane >> 4) + r;
        const int t = n * 16 + (lane & 15);
        if (e < E && t < T) logits[(size_t)t * E + e] = acc[n][r] + (bias ? bias[e] : 0.f);
      }
  }
}

// ------------------------------------------------------------------ selection helpers

// Wave-wide best (largest value, lowest id on ties).
__device__ __forceinline__ void wave_argbest(float &v, int &id) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const float v2 = __shfl_xor(v, s);
    const int i2 = __shfl_xor(id, s);
    if (v2 > v || (v2 == v && i2 < id)) { v = v2; id = i2; }
  }
}

// One wave picks up to K experts for each of its NQ positions by descending
// logit (ties to the lower id) among those allowed (allowed == nullptr: all);
// the positions' selections run interleaved.  lv / pv hold the lane's logits
// and softmax scores for experts lane + 64j.  Writes the picks and their
// scores to idx_row[q] / psel_row[q] (-1 / 0 where fewer than K are allowed);
// rows with live[q] false are skipped.  All lanes take part.
template <int NQ>
__device__ void wave_topk(const float (&lv)[NQ][4], const float (&pv)[NQ][4], const bool (&live)[NQ],
                          int E, int K, const int32_t *allowed, int lane, int32_t *const (&idx_row)[NQ],
                          float *const (&psel_row)[NQ]) {
  bool avail[NQ][4];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      avail[q][j] = live[q] && e < E && (allowed == nullptr || allowed[e] != 0);
    }
  for (int k = 0; k < K; ++k) {
    float bv[NQ];
    int be[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      bv[q] = -FLT_MAX;
      be[q] = INT_MAX;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        if (avail[q][j] && (be[q] == INT_MAX || lv[q][j] > bv[q])) { bv[q] = lv[q][j]; be[q] = e; }
      }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const float v2 = __shfl_xor(bv[q], s);
        const int i2 = __shfl_xor(be[q], s);
        if (v2 > bv[q] || (v2 == bv[q] && i2 < be[q])) { bv[q] = v2; be[q] = i2; }
      }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (!live[q]) continue;
      float ps = 0.f;
      if (be[q] != INT_MAX) {
        const int j = be[q] >> 6;                      // uniform across the wave
        const float pj = j == 0 ? pv[q][0] : j == 1 ? pv[q][1] : j == 2 ? pv[q][2] : pv[q][3];
        ps = __shfl(pj, be[q] & 63);
        if ((be[q] & 63) == lane) avail[q][j] = false;
      }
      if (lane == 0) {
        idx_row[q][k] = be[q] == INT_MAX ? -1 : be[q];
        psel_row[q][k] = ps;
      }
    }
  }
}

struct SelShared {
  int32_t idx[kMaxT][kMaxK];    // picks of each position (-1: unused slot)
  float psel[kMaxT][kMaxK];     // their softmax scores
  uint32_t tokmask[kMaxE];      // positions that picked each expert
  uint8_t kslot[kMaxT][kMaxE];  // slot k of expert e among position t's picks
  double mass[kMaxE];           // block expert mass
  int32_t ulist[kMaxE];         // experts with a pick, ascending id
  double umass[kMaxE];          // their mass, in ulist order
  int32_t rank[kMaxE];          // rank of each ulist entry
  int32_t sorted[kMaxE];        // ulist ranked by (mass desc, id asc)
  double cum[kMaxE];            // prefix sums of ranked mass
  int32_t member[kMaxE];        // coreset membership
  int32_t wtot[16];
  double wtotd[16];
  int32_t nu, csize, below;
};

// Rebuilds tokmask / kslot from sh.idx (all threads; ends with a barrier).
__device__ void build_masks(SelShared &sh, int T, int E, int K) {
  const int tid = threadIdx.x;
  if (tid < E) sh.tokmask[tid] = 0u;
  __syncthreads();
  for (int i = tid; i < T * K; i += blockDim.x) {
    const int t = i / K, k = i - t * K;
    const int e = sh.idx[t][k];
    if (e >= 0) {
      atomicOr(&sh.tokmask[e], 1u << t);
      sh.kslot[t][e] = (uint8_t)k;
    }
  }
  __syncthreads();
}

// Union of experts, ascending id, into sh.ulist / sh.nu (all threads, >= E
// threads; ends with a barrier).  Returns the caller's slot (or -1).
__device__ int union_scan(SelShared &sh, int E) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int flag = (tid < E && sh.tokmask[tid] != 0u) ? 1 : 0;
  int incl = flag;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const int o = __shfl_up(incl, s);
    if (lane >= s) incl += o;
  }
  if (lane == 63) sh.wtot[wave] = incl;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += sh.wtot[w];
  const int slot = flag ? off + incl - 1 : -1;
  if (flag) sh.ulist[slot] = tid;
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < nw; ++w) tot += sh.wtot[w];
    sh.nu = tot;
  }
  __syncthreads();
  return slot;
}

// Block expert mass, ranking and coreset cut ([P2] coreset section): mass_e
// sums the softmax scores of the positions that picked e (ascending position
// order); experts are ranked by (mass desc, id asc); the coreset is the
// shortest ranked prefix whose cumulative mass reaches top_p of the total
// (top_p >= 1: every expert with positive mass).  Needs sh.idx / sh.psel.
// Fills sh.mass, sh.member, sh.csize (all threads, >= E threads).
__device__ void coreset_core(SelShared &sh, int T, int E, int K, float top_p) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  build_masks(sh, T, E, K);
  if (tid < E) {
    double m = 0.0;
    uint32_t bits = sh.tokmask[tid];
    while (bits) {
      const int t = __ffs(bits) - 1;
      bits &= bits - 1u;
      m += (double)sh.psel[t][sh.kslot[t][tid]];
    }
    sh.mass[tid] = m;
    sh.member[tid] = 0;
  }
  union_scan(sh, E);
  const int nu = sh.nu;
  if (tid < nu) {
    sh.umass[tid] = sh.mass[sh.ulist[tid]];
    sh.rank[tid] = 0;
  }
  __syncthreads();
  {
    // rank of union entry j = number of entries before it in (mass desc, id
    // asc) order; the block's threads split each entry's count into parts
    const int parts = (int)blockDim.x / kMaxE;
    const int j = tid % kMaxE, part = tid / kMaxE;
    if (j < nu) {
      const double m = sh.umass[j];
      const int e = sh.ulist[j];
      const int lo = part * nu / parts, hi = (part + 1) * nu / parts;
      int r = 0;
#pragma unroll 8
      for (int i = lo; i < hi; ++i) {
        const double o = sh.umass[i];
        r += (o > m) || (o == m && sh.ulist[i] < e);
      }
      atomicAdd(&sh.rank[j], r);
    }
  }
  if (tid == 0) sh.below = 0;
  __syncthreads();
  if (tid < nu) {
    sh.sorted[sh.rank[tid]] = sh.ulist[tid];
    sh.cum[sh.rank[tid]] = sh.umass[tid];
  }
  __syncthreads();
  int k = nu;
  if (top_p < 1.0f && nu > 0) {
    // inclusive prefix sum of the ranked masses (fp64), one wave per 64 ranks
    double v = tid < nu ? sh.cum[tid] : 0.0;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const double o = __shfl_up(v, s);
      if (lane >= s) v += o;
    }
    if (lane == 63) sh.wtotd[wave] = v;
    __syncthreads();
    double off = 0.0;
    for (int w = 0; w < wave; ++w) off += sh.wtotd[w];
    v += off;
    if (tid < nu) sh.cum[tid] = v;
    __syncthreads();
    const double target = (double)top_p * sh.cum[nu - 1];
    // the prefix with cumulative mass below the target, plus one
    const unsigned long long b = __ballot(tid < nu && v < target);
    if (lane == 0 && b) atomicAdd(&sh.below, (int)__popcll(b));
    __syncthreads();
    k = max(1, min(sh.below + 1, nu));
  }
  if (tid < k) sh.member[sh.sorted[tid]] = 1;
  if (tid == 0) sh.csize = k;
  __syncthreads();
}

__device__ void write_bits(const SelShared &sh, int E, uint32_t *bits) {
  const int tid = threadIdx.x;
  if (tid < (E + 31) / 32) {
    uint32_t b = 0;
    for (int j = 0; j < 32; ++j) {
      const int e = tid * 32 + j;
      if (e < E && sh.member[e]) b |= 1u << j;
    }
    bits[tid] = b;
  }
}

// ------------------------------------------------------------------ route + select
// One workgroup of 1024 threads: per-position softmax and top-K, optional
// coreset and re-routing, then the union of experts and each union expert's
// list of (position, pick) assignments.
__global__ __launch_bounds__(1024) void route_select_kernel(RouteBufs r, int T, int E, int K,
                                                            float top_p) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  constexpr int kTokPerWave = kMaxT / 16;
  float lv[kTokPerWave][4], pv[kTokPerWave][4];

  // softmax over all experts and top-K by logit
  bool live[kTokPerWave];
  int32_t *idx_rows[kTokPerWave];
  float *psel_rows[kTokPerWave];
#pragma unroll
  for (int q = 0; q < kTokPerWave; ++q) {
    const int t = wave + q * nw;
    live[q] = t < T;
    idx_rows[q] = sh.idx[live[q] ? t : 0];
    psel_rows[q] = sh.psel[live[q] ? t : 0];
    float m = -FLT_MAX;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      lv[q][j] = (live[q] && e < E) ? r.logits[(size_t)t * E + e] : -FLT_MAX;
      m = fmaxf(m, lv[q][j]);
    }
    m = wave_max(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      pv[q][j] = (live[q] && e < E) ? expf(lv[q][j] - m) : 0.f;
      s += pv[q][j];
    }
    s = wave_sum(s);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      pv[q][j] = live[q] ? pv[q][j] / s : 0.f;
      if (live[q] && e < E) r.prob[(size_t)t * E + e] = pv[q][j];
    }
  }
  wave_topk<kTokPerWave>(lv, pv, live, E, K, nullptr, lane, idx_rows, psel_rows);
  __syncthreads();

  // block mass and coreset (also run without coreset: it reports the union)
  coreset_core(sh, T, E, K, top_p);
  if (tid < E) r.mass[tid] = (float)sh.mass[tid];
  write_bits(sh, E, r.cs_bits);
  if (top_p < 1.0f) {
    const int kk = min(K, sh.csize);
    wave_topk<kTokPerWave>(lv, pv, live, E, kk, sh.member, lane, idx_rows, psel_rows);
#pragma unroll
    for (int q = 0; q < kTokPerWave; ++q)
      if (live[q] && lane == 0)
        for (int k = kk; k < K; ++k) { idx_rows[q][k] = -1; psel_rows[q][k] = 0.f; }
    __syncthreads();
    build_masks(sh, T, E, K);
  }

  // renormalised weights, outputs
  if (tid < T * K) {
    const int t = tid / K, k = tid % K;
    float s = 0.f;
    for (int j = 0; j < K; ++j) s += sh.psel[t][j];
    const int e = sh.idx[t][k];
    r.idx[tid] = e;
    r.wgt[tid] = e >= 0 ? sh.psel[t][k] / s : 0.f;
  }

  // union of experts read and each one's assignment list (t*K + k, ascending t)
  const int slot = union_scan(sh, E);
  if (slot >= 0) {
    uint32_t bits = sh.tokmask[tid];
    r.union_list[slot] = tid;
    r.slot_n[slot] = __popc(bits);
    int j = 0;
    while (bits) {
      const int t = __ffs(bits) - 1;
      bits &= bits - 1u;
      r.slot_asg[slot * kMaxT + j++] = t * K + sh.kslot[t][tid];
    }
  }
  if (tid == 0) {
    r.meta[0] = sh.nu;
    r.meta[1] = sh.csize;
    if (r.n_distinct_out) *r.n_distinct_out = sh.nu;
    if (r.coreset_size_out) *r.coreset_size_out = sh.csize;
  }
}

// ------------------------------------------------------------------ coreset alone
__global__ __launch_bounds__(256) void coreset_kernel(const float *__restrict__ prob,
                                                      const int32_t *__restrict__ idx, int T,
                                                      int E, int K, float top_p,
                                                      uint32_t *__restrict__ bits,
                                                      int32_t *__restrict__ size,
                                                      float *__restrict__ mass) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  for (int i = tid; i < T * K; i += blockDim.x) {
    const int t = i / K, k = i % K;
    const int e = idx[i];
    const bool ok = e >= 0 && e < E;
    sh.idx[t][k] = ok ? e : -1;
    sh.psel[t][k] = ok ? prob[(size_t)t * E + e] : 0.f;
  }
  __syncthreads();
  coreset_core(sh, T, E, K, top_p);
  write_bits(sh, E, bits);
  if (tid == 0) *size = sh.csize;
  if (mass && tid < E) mass[tid] = (float)sh.mass[tid];
}

// ------------------------------------------------------------------ combine
// y_t = sum_k P[t*K+k] (live slots, in slot order) + P_s[t]; then h += y and
// xhat = RMSNorm(h), one workgroup per position.
template <typename OT>
__global__ __launch_bounds__(kRowThreads) void combine_kernel(const float *__restrict__ P,
                                                              const float *__restrict__ P_s,
                                                              const int32_t *__restrict__ idx,
                                                              float *__restrict__ h,
                                                              float *__restrict__ y_out,
                                                              OT *__restrict__ xhat_out, int H, int K,
                                                              float eps) {
  __shared__ float red[kRowThreads / 64];
  const int t = blockIdx.x;
  uint32_t live = 0;
  for (int k = 0; k < K; ++k) live |= (idx[t * K + k] >= 0 ? 1u : 0u) << k;
  const size_t base = (size_t)t * H;
  const int H4 = H / 4;
  float4 hv[kRowVec];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < kRowVec; ++q) {
    const int j = threadIdx.x + q * kRowThreads;
    if (j >= H4) continue;
    float4 y = make_float4(0, 0, 0, 0);
#pragma unroll 8
    for (int k = 0; k < K; ++k) {
      if (live >> k & 1u) {
        const float4 p = reinterpret_cast<const float4 *>(P + ((size_t)t * K + k) * H)[j];
        y.x += p.x; y.y += p.y; y.z += p.z; y.w += p.w;
      }
    }
    if (P_s) {
      const float4 p = reinterpret_cast<const float4 *>(P_s + base)[j];
      y.x += p.x; y.y += p.y; y.z += p.z; y.w += p.w;
    }
    if (y_out) reinterpret_cast<float4 *>(y_out + base)[j] = y;
    if (h) {
      float4 v = reinterpret_cast<float4 *>(h + base)[j];
      v.x += y.x; v.y += y.y; v.z += y.z; v.w += y.w;
      reinterpret_cast<float4 *>(h + base)[j] = v;
      hv[q] = v;
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  }
  if (h && xhat_out) {
    ss = block_sum_512(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
    for (int q = 0; q < kRowVec; ++q) {
      const int j = threadIdx.x + q * kRowThreads;
      if (j < H4)
        store4<OT>(xhat_out, base + 4 * (size_t)j,
                   make_float4(hv[q].x * inv, hv[q].y * inv, hv[q].z * inv, hv[q].w * inv));
    }
  }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_rmsnorm(int wdtype, const float *in, float *copy_out, void *out, int T, int H,
                          hipStream_t s) {
  if (wdtype == 1)
    rmsnorm_kernel<bf16_t><<<T, kRowThreads, 0, s>>>(in, copy_out, (bf16_t *)out, H, 1e-6f);
  else
    rmsnorm_kernel<float><<<T, kRowThreads, 0, s>>>(in, copy_out, (float *)out, H, 1e-6f);
  return hipGetLastError();
}

hipError_t launch_router_logits(int wdtype, const void *xhat, const void *w_router,
                                const float *bias, float *logits, int T, int H, int E,
                                hipStream_t s) {
  const int grid = (E + 15) / 16;
  if (wdtype == 1) {
    if (T <= 16)
      router_logits_kernel<WBf16, 1><<<grid, 512, 0, s>>>((const bf16_t *)xhat,
                                                           (const bf16_t *)w_router, bias, logits,
                                                           T, H, E);
    else
      router_logits_kernel<WBf16, 2><<<grid, 512, 0, s>>>((const bf16_t *)xhat,
                                                           (const bf16_t *)w_router, bias, logits,
                                                           T, H, E);
  } else {
    if (T <= 16)
      router_logits_kernel<WF32, 1><<<grid, 512, 0, s>>>((const float *)xhat,
                                                          (const float *)w_router, bias, logits, T,
                                                          H, E);
    else
      router_logits_kernel<WF32, 2><<<grid, 512, 0, s>>>((const float *)xhat,
                                                          (const float *)w_router, bias, logits, T,
                                                          H, E);
  }
  return hipGetLastError();
}

hipError_t launch_route_select(const RouteBufs &r, int T, int E, int K, float top_p,
                               hipStream_t s) {
  route_select_kernel<<<1, 1024, 0, s>>>(r, T, E, K, top_p);
  return hipGetLastError();
}

hipError_t launch_coreset(const float *prob, const int32_t *idx, int T, int E, int K, float top_p,
                          uint32_t *bits, int32_t *size, float *mass, hipStream_t s) {
  coreset_kernel<<<1, 256, 0, s>>>(prob, idx, T, E, K, top_p, bits, size, mass);
  return hipGetLastError();
}

hipError_t launch_combine(int wdtype, const float *P, const float *P_s, const int32_t *idx,
                          float *h, float *y_out, void *xhat_out, int T, int H, int K,
                          hipStream_t s) {
  if (wdtype == 1)
    combine_kernel<bf16_t><<<T, kRowThreads, 0, s>>>(P, P_s, idx, h, y_out, (bf16_t *)xhat_out, H, K,
                                             1e-6f);
  else
    combine_kernel<float><<<T, kRowThreads, 0, s>>>(P, P_s, idx, h, y_out, (float *)xhat_out, H, K,
                                            1e-6f);
  return hipGetLastError();
}

}  // namespace bdd
