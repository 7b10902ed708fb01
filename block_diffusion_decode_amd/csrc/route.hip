// Normalisation, router, top-K selection and block coreset.
//
// Pages: [P1] aitujian.cn article on Clover-35B-A3B-Preview, section 四 (256
// routed experts, top-8, one shared expert) and section 五 (a block of 32
// positions touches a union of experts); [P2] goremy.ai "What Is
// Clover-35B-A3B? Block Diffusion on a Qwen3.6 MoE", section "What is the MoE
// coreset and why does it matter?" (aggregate each position's top-8 scores,
// rank experts, keep enough to cover top_p of the mass).
#include <float.h>
#include <limits.h>

#include <type_traits>

#include "int4.hpp"
#include "kernels.hpp"
#include "stream.hpp"

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

// Elements k .. k + 3 of position t into the packed block (see xpack_unit).
template <typename OT>
__device__ __forceinline__ void store4_packed(OT *xpk, int t, int T, int k, float4 v) {
  constexpr int CH = 16 / (int)sizeof(OT);
  store4<OT>(xpk, (size_t)xpack_unit(k / CH, t, T) * CH + k % CH, v);
}

// x_hat = h / sqrt(mean(h^2) + eps), unit gain, one workgroup per position;
// also into the packed block `xpk` when given.
template <typename OT>
__global__ __launch_bounds__(kRowThreads) void rmsnorm_kernel(const float *__restrict__ in,
                                                              float *__restrict__ copy_out,
                                                              OT *__restrict__ out, OT *__restrict__ xpk, int H,
                                                              float eps, int32_t *__restrict__ zero_word,
                                                              const int32_t *__restrict__ gate) {
  __shared__ float red[kRowThreads / 64];
  if (gated_off(gate)) return;
  if (blockIdx.x == 0 && threadIdx.x == 0 && zero_word) *zero_word = 0;
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
      const float4 o = make_float4(v[q].x * inv, v[q].y * inv, v[q].z * inv, v[q].w * inv);
      store4<OT>(out, base + 4 * (size_t)j, o);
      if (xpk) store4_packed<OT>(xpk, blockIdx.x, gridDim.x, 4 * j, o);
    }
  }
}

// ------------------------------------------------------------------ router logits
// Partial router logits over hidden slices of kRouterSlice elements:
// part[ks][t][e] = xhat_t[slice ks] . W_r[e][slice ks].  One wave per
// (16 experts, slice): 16x16 MFMA tiles with the experts as rows and the
// positions as columns, both operands loaded straight from memory (the block
// is L2-resident), so the 1 MiB of router weights is spread over ~256
// workgroups.  The selection kernel sums the slices in slice order and adds
// the bias.  The workgroups also clear the selection kernel's state.
constexpr int kRouterSlice = 128;
constexpr uint32_t kRouterOut = 0x7ff00000u;  // out-of-range buffer offset: loads return zeros

template <class W, int NT>
__global__ __launch_bounds__(64) void router_kernel(const typename W::T *__restrict__ xhat,
                                                    uint32_t *__restrict__ zero_base, int zero_words,
                                                    const typename W::T *__restrict__ wr,
                                                    float *__restrict__ part, int T, int H, int E,
                                                    const int32_t *__restrict__ gate) {
  typedef typename W::T WT;
  constexpr int CH = W::kChunk;
  constexpr int NCS = kRouterSlice / CH;  // 16-byte chunks per slice
  if (gated_off(gate)) return;
  constexpr int NS = NCS / 4;             // MFMA k-steps per slice (4 chunks each)
  const int lane = threadIdx.x, li = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16, ks = blockIdx.y;
  {
    const int nthr = (int)(gridDim.x * gridDim.y) * 64;
    for (int i = (int)(blockIdx.y * gridDim.x + blockIdx.x) * 64 + lane; i < zero_words; i += nthr) zero_base[i] = 0u;
  }
  const rsrc_t rw = make_rsrc(wr, (uint32_t)(E * H) * sizeof(WT));
  const rsrc_t rx = make_rsrc(xhat, (uint32_t)(T * H) * sizeof(WT));
  const int e_row = row0 + li;
  uint4 a[NS], b[NS][NT];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int c = ks * NCS + 4 * j + g;
    a[j] = buf_ld16(rw, e_row < E ? (uint32_t)(e_row * H + c * CH) * sizeof(WT) : kRouterOut, 0);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int t = n * 16 + li;
      b[j][n] = buf_ld16(rx, t < T ? (uint32_t)(t * H + c * CH) * sizeof(WT) : kRouterOut, 0);
    }
  }
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if constexpr (std::is_same<W, WBf16>::value) {
        acc[n] = mfma_bf16(a[j], b[j][n], acc[n]);
      } else {
        acc[n] = mfma_f32(__uint_as_float(a[j].x), __uint_as_float(b[j][n].x), acc[n]);
        acc[n] = mfma_f32(__uint_as_float(a[j].y), __uint_as_float(b[j][n].y), acc[n]);
        acc[n] = mfma_f32(__uint_as_float(a[j].z), __uint_as_float(b[j][n].z), acc[n]);
        acc[n] = mfma_f32(__uint_as_float(a[j].w), __uint_as_float(b[j][n].w), acc[n]);
      }
    }
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = row0 + 4 * g + r;
      const int t = n * 16 + li;
      if (e < E && t < T) part[((size_t)ks * T + t) * E + e] = acc[n][r];
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

struct SelShared {
  int32_t idx[kMaxT][kMaxK];    // picks of each position (-1: unused slot)
  float psel[kMaxT][kMaxK];     // their softmax scores
  posmask_t tokmask[kMaxE];     // positions that picked each expert
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
  if (tid < E) sh.tokmask[tid] = 0ull;
  __syncthreads();
  for (int i = tid; i < T * K; i += blockDim.x) {
    const int t = i / K, k = i - t * K;
    const int e = sh.idx[t][k];
    if (e >= 0) {
      atomicOr(&sh.tokmask[e], 1ull << t);
      sh.kslot[t][e] = (uint8_t)k;
    }
  }
  __syncthreads();
}

// Union of experts, ascending id, into sh.ulist / sh.nu (all threads, >= E
// threads; ends with a barrier).  Returns the caller's slot (or -1).
__device__ int union_scan(SelShared &sh, int E) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int flag = (tid < E && sh.tokmask[tid] != 0ull) ? 1 : 0;
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
    // ascending positions, eight at a time (their slot reads are independent)
    double m = 0.0;
    posmask_t bits = sh.tokmask[tid];
    while (bits) {
      int tt[8], kq[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        tt[j] = bits ? __ffsll((long long)bits) - 1 : -1;
        bits &= bits - 1ull;
      }
      // unconditional reads (row 0 stands in for a missing position, whose
      // term is then +0.0), so the sixteen reads are not serialised by branches
#pragma unroll
      for (int j = 0; j < 8; ++j) kq[j] = sh.kslot[tt[j] >= 0 ? tt[j] : 0][tid];
      float pq[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pq[j] = sh.psel[tt[j] >= 0 ? tt[j] : 0][kq[j] & (kMaxK - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j) m += tt[j] >= 0 ? (double)pq[j] : 0.0;
    }
    sh.mass[tid] = m;
    sh.member[tid] = 0;
  }
  union_scan(sh, E);
  const int nu = sh.nu;
  if (top_p >= 1.0f) {
    // no coreset: every expert with a pick (positive mass) is kept
    if (tid < nu) sh.member[sh.ulist[tid]] = 1;
    if (tid == 0) sh.csize = nu;
    __syncthreads();
    return;
  }
  if (nu <= 64) {
    // one wave: lane j holds union entry j; its rank counts the entries
    // before it in (mass desc, id asc) order, read from LDS eight at a time
    // (broadcast reads, all in flight together); the ranked masses' prefix
    // sum comes from a shuffle scan and the cut from a ballot
    if (tid < nu) sh.umass[tid] = sh.mass[sh.ulist[tid]];
    __syncthreads();
    if (wave == 0) {
      const bool live = lane < nu;
      const int e = live ? sh.ulist[lane] : 0;
      const double m = live ? sh.umass[lane] : 0.0;
      int r = 0;
      for (int i0 = 0; i0 < nu; i0 += 8) {
        double mi[8];
        int ei[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = min(i0 + j, nu - 1);
          mi[j] = sh.umass[i];
          ei[j] = sh.ulist[i];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)   // bitwise, so no branches per comparison
          r += (int)(i0 + j < nu) & ((int)(mi[j] > m) | ((int)(mi[j] == m) & (int)(ei[j] < e)));
      }
      if (live) {
        sh.sorted[r] = e;
        sh.cum[r] = m;
      }
      double v = live ? sh.cum[lane] : 0.0;
#pragma unroll
      for (int s = 1; s < 64; s <<= 1) {
        const double o = __shfl_up(v, s);
        if (lane >= s) v += o;
      }
      const long long tb = __double_as_longlong(v);
      const double total = __longlong_as_double(
          ((long long)__builtin_amdgcn_readlane((int)(tb >> 32), nu - 1) << 32) |
          (long long)(uint32_t)__builtin_amdgcn_readlane((int)tb, nu - 1));
      const double target = (double)top_p * total;
      const int below = (int)__popcll(__ballot(live && v < target));
      const int k = max(1, min(below + 1, nu));
      if (live) sh.cum[lane] = v;
      if (lane < k) sh.member[sh.sorted[lane]] = 1;
      if (lane == 0) sh.csize = k;
    }
    __syncthreads();
    return;
  }
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
        const int oe = sh.ulist[i];
        r += (int)(o > m) | ((int)(o == m) & (int)(oe < e));
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
  if (nu > 0) {
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

// Coreset membership bitset from a ballot per wave (>= E threads).
__device__ void write_bits(const SelShared &sh, int E, uint32_t *bits) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const unsigned long long b = __ballot(tid < E && sh.member[tid] != 0);
  if (lane == 0 && 64 * w < E) bits[2 * w] = (uint32_t)b;
  if (lane == 32 && 64 * w + 32 < E) bits[2 * w + 1] = (uint32_t)(b >> 32);
}

// ------------------------------------------------------------------ route + select
// One workgroup of kSelThreads per position: softmax over the position's E
// router logits and its expert order (logit desc, expert id asc), the rank of
// each expert counted over all keys, so its top-K are ranks 0 .. K-1.  The
// block-level steps run in these workgroups, in parallel:
//   - with the coreset, each adds its first picks' softmax scores to the block
//     mass (64-bit fixed-point atomics: the sums are exact, so their order
//     does not matter) and its bit to each picked expert's position mask,
//     counts itself, and waits until all T positions are counted; then each
//     ranks the experts and cuts the coreset itself (the same exact sums give
//     every workgroup the same coreset, so nothing is handed back) and
//     re-takes its position's first min(K, |C|) coreset members in its own
//     order;
//   - each writes its final picks and weights, and adds its bit and pick slot
//     to each picked expert's mask and slot word.  The expert kernels build
//     the union and their work lists from these (after the kernel boundary).
// The wait is for the other positions' workgroups, which the dispatcher
// starts first (T <= 64 of them, far fewer than the device runs at once).  It
// is bounded all the same (every wave leaves it), and a timeout is reported in
// meta[4].
// Workgroups past the T positions compute the shared expert's gate/up (it
// needs only the normalised block), so its weights stream while selection
// runs: workgroup T + j takes intermediate units 16 j .. 16 j + 15.
constexpr int kSelThreads = 256;
static_assert(kSelThreads == 256, "the shared gate/up item runs on four waves");
static_assert(kSelThreads >= kMaxE, "one thread per expert in the block steps");
constexpr int kSelSpinMax = 1 << 17;          // bound of the wait for the positions' counts: polls of ~1 us, ~0.1-0.2 s
constexpr double kMassScale = 72057594037927936.0;   // 2^56: fixed-point unit of the block mass

// Shared-expert operands for the workgroups past the positions.
template <class W>
struct SharedGU {
  const typename W::T *xpk;    // packed normalised block
  const typename W::T *wsgu;   // [2 I_s][H]
  char *act;                   // its packed activation slot (entry t = position t)
  int H, Is;
};

__device__ __forceinline__ uint32_t order_key(float v) {
  // larger float -> smaller key (ascending sort = descending logits)
  const uint32_t u = __float_as_uint(v);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

// Exclusive prefix over the workgroup of flags (0/1), via ballots; returns
// this thread's prefix and leaves the total in *total.  Ends with a barrier.
__device__ __forceinline__ int block_flag_scan(bool flag, int *s_wave, int *total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long b = __ballot(flag);
  if (lane == 0) s_wave[wave] = __popcll(b);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    off += w < wave ? s_wave[w] : 0;
    tot += s_wave[w];
  }
  *total = tot;
  __syncthreads();
  return off + __popcll(b & lanes_below(lane));
}

// The coreset step ([P2] coreset section), in every position's workgroup
// once all positions are counted: experts with a first pick, ranked by (mass
// desc, id asc) from the exact fixed-point masses; the shortest ranked prefix
// whose cumulative mass reaches top_p of the total.  The masses are exact
// integer sums, so every workgroup finds the same coreset; it is left in
// s_cb / *s_csize, and the workgroup with `report` also writes the bitset,
// the masses and the size out.  It runs after the workgroup's acquire (the
// count and a barrier), so the other workgroups' atomics are visible to plain
// loads, all issued at once.
__device__ void coreset_step(const RouteBufs &r, int E, float top_p, int *s_wave, uint32_t *s_cb, int *s_csize,
                             bool report) {
  __shared__ unsigned long long s_um[kMaxE];
  __shared__ int s_ue[kMaxE], s_rank[kMaxE], s_sorted[kMaxE];
  __shared__ unsigned long long s_cum[kMaxE];
  __shared__ unsigned long long s_wtot[kSelThreads / 64];
  __shared__ int s_below;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int te = min(tid, E - 1);
  const unsigned long long m_all = r.sync.mass_fx[te];
  const posmask_t msk_all = r.sync.mask1[te];
  const unsigned long long m = tid < E ? m_all : 0ull;
  const posmask_t msk = tid < E ? msk_all : 0ull;
  if (tid < kMaxE / 32) s_cb[tid] = 0u;
  if (tid == 0) s_below = 0;
  int nu = 0;
  const int slot = block_flag_scan(msk != 0ull, s_wave, &nu);
  if (msk != 0ull) {
    s_um[slot] = m;
    s_ue[slot] = tid;
  }
  if (tid < kMaxE) s_rank[tid] = 0;
  __syncthreads();
  {
    // rank of entry j = entries before it in (mass desc, id asc) order; the
    // threads split each entry's comparisons into `parts` ranges
    const int parts = nu <= 64 ? 4 : nu <= 128 ? 2 : 1;
    const int span = parts == 4 ? 64 : parts == 2 ? 128 : 256;
    const int j = tid % span, part = tid / span;
    if (j < nu && part < parts) {
      const unsigned long long mj = s_um[j];
      const int ej = s_ue[j];
      const int lo = part * nu / parts, hi = (part + 1) * nu / parts;
      int rk = 0;
      for (int i0 = lo; i0 < hi; i0 += 8) {
        unsigned long long mi[8];
        int ei[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int i = min(i0 + q, hi - 1);
          mi[q] = s_um[i];
          ei[q] = s_ue[i];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
          rk += (int)(i0 + q < hi) & ((int)(mi[q] > mj) | ((int)(mi[q] == mj) & (int)(ei[q] < ej)));
      }
      atomicAdd(&s_rank[j], rk);
    }
  }
  __syncthreads();
  if (tid < nu) {
    s_sorted[s_rank[tid]] = s_ue[tid];
    s_cum[s_rank[tid]] = s_um[tid];
  }
  __syncthreads();
  // inclusive prefix of the ranked masses (exact integer sums)
  unsigned long long v = tid < nu ? s_cum[tid] : 0ull;
#pragma unroll
  for (int sft = 1; sft < 64; sft <<= 1) {
    const unsigned long long o = __shfl_up(v, sft);
    if (lane >= sft) v += o;
  }
  if (lane == 63) s_wtot[wave] = v;
  __syncthreads();
  unsigned long long off = 0ull, tot = 0ull;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    off += w < wave ? s_wtot[w] : 0ull;
    tot += s_wtot[w];
  }
  v += off;
  // the prefix whose cumulative mass stays below top_p of the total, plus one
  const double target = (double)top_p * (double)tot;
  const unsigned long long b = __ballot(tid < nu && (double)v < target);
  if (lane == 0 && b) atomicAdd(&s_below, (int)__popcll(b));
  __syncthreads();
  const int k = max(1, min(s_below + 1, nu));
  if (tid < k) atomicOr(&s_cb[s_sorted[tid] >> 5], 1u << (s_sorted[tid] & 31));
  if (tid == 0) *s_csize = k;
  __syncthreads();
  if (report) {
    if (tid < (E + 31) / 32) r.cs_bits[tid] = s_cb[tid];
    if (tid < E) r.mass[tid] = (float)((double)m / kMassScale);
    if (tid == 0) {
      r.meta[1] = k;
      if (r.coreset_size_out) *r.coreset_size_out = k;
    }
  }
}

template <class W, int NT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(RouteBufs r, const float *__restrict__ bias,
                                                             int KS, int T, int E, int K, float top_p,
                                                             SharedGU<W> sg) {
  __shared__ __align__(16) unsigned long long s_key[kSelThreads];
  __shared__ int s_order[kSelThreads];
  __shared__ float s_p[kSelThreads];
  __shared__ float s_red[kSelThreads / 64];
  __shared__ int s_wave[kSelThreads / 64];
  __shared__ int s_pick[kMaxK];
  __shared__ uint32_t s_cb[kMaxE / 32];
  __shared__ int s_csize;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  if (gated_off(r.gate)) return;
  if (t >= T) {
    __shared__ f32x4 red[4 * 2 * NT * 64];
    // column entry j is position j
    int pos[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int j = n * 16 + (lane & 15);
      pos[n] = j < T ? j : -1;
    }
    if constexpr (std::is_same<W, WI4>::value)
      i4_gateup_item<NT>(i4_mat(sg.wsgu, 2 * sg.Is, sg.H), sg.Is, sg.xpk, T, pos, (t - T) * 16, wave, lane, sg.act,
                         nullptr, nullptr, 0, red);
    else
      dense_gateup_item<W, kSgSteps, NT>(sg.wsgu, sg.Is, sg.xpk, T, sg.H, pos, t - T, (t - T) * 16, wave, lane, sg.act,
                                     red);
    return;
  }
  // ---- this position: logit = router slices in slice order + bias
  float l = -FLT_MAX;
  if (tid < E) {
    float acc = 0.f;
#pragma unroll 16
    for (int ks = 0; ks < KS; ++ks) acc += r.logits[((size_t)ks * T + t) * E + tid];
    l = acc + (bias ? bias[tid] : 0.f);
  }
  float m = wave_max_dpp(l);
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  const float ex = tid < E ? expf(l - m) : 0.f;
  float sum = wave_sum_dpp(ex);
  if (lane == 0) s_red[wave] = sum;
  __syncthreads();
  sum = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  s_p[tid] = ex / sum;
  // the position's expert order, ascending on (order_key(logit), id): each
  // expert's rank is the number of keys below its own (the keys are distinct),
  // counted over the keys in LDS with broadcast reads
  const unsigned long long key = tid < E ? (((unsigned long long)order_key(l) << 32) | (uint32_t)tid) : ~0ull;
  s_key[tid] = key;
  __syncthreads();
  int rank = tid;   // (padding past E keeps its own slot)
  if (tid < E) {
    const ulonglong2 *kp = reinterpret_cast<const ulonglong2 *>(s_key);
    int below = 0;
#pragma unroll 8
    for (int j = 0; j < (E + 1) / 2; ++j) {   // (an odd E reads padding key E, which is never below)
      const ulonglong2 v = kp[j];
      below += (int)(v.x < key) + (int)(v.y < key);
    }
    rank = below;
  }
  s_order[rank] = tid;
  __syncthreads();
  const int e_sorted = tid < E ? s_order[tid] : -1;   // the expert of rank tid
  const bool coreset = top_p < 1.0f;
  int kk = K;
  if (coreset) {
    // contribute the first picks to the block mass and the position masks
    if (tid < K) {
      atomicAdd(r.sync.mass_fx + e_sorted, (unsigned long long)((double)s_p[e_sorted] * kMassScale));
      atomicOr(r.sync.mask1 + e_sorted, 1ull << t);
    }
    __syncthreads();
    // the positions' timeout is reported, and the wait ends
    if (tid == 0 && !count_and_wait_all(r.sync.words, T, kSelSpinMax)) r.meta[4] = 1;
    __syncthreads();
    coreset_step(r, E, top_p, s_wave, s_cb, &s_csize, t == 0);
    // re-routing: the first min(K, |C|) coreset members in this position's order
    const int es = e_sorted & (kMaxE - 1);   // (padding lanes past E hold no expert)
    const bool member = tid < E && ((s_cb[es >> 5] >> (es & 31)) & 1u);
    int nmem = 0;
    const int before = block_flag_scan(member, s_wave, &nmem);
    kk = min(min(K, s_csize), nmem);
    if (member && before < kk) s_pick[before] = e_sorted;
    __syncthreads();
  } else {
    if (tid < K) s_pick[tid] = e_sorted;
    __syncthreads();
  }
  // ---- final picks: weights renormalised over the picks (slot order)
  if (tid < K) {
    const int e = tid < kk ? s_pick[tid] : -1;
    float ssum = 0.f;
    for (int j = 0; j < kk; ++j) ssum += s_p[s_pick[j]];
    r.idx[(size_t)t * K + tid] = e;
    r.wgt[(size_t)t * K + tid] = e >= 0 ? s_p[e] / ssum : 0.f;
    if (e >= 0) {
      atomicOr(r.sync.mask2 + e, 1ull << t);
      atomicOr(r.sync.kslot + e * (kMaxT / 4) + (t >> 2), (uint32_t)tid << (8 * (t & 3)));
    }
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
// y_t = sum_k w[t*K+k] * P[t*K+k] (live slots, in slot order) + P_s[t]; then h += y and
// xhat = RMSNorm(h) (also packed into xpk_out when given), one workgroup per position.
template <typename OT>
__global__ __launch_bounds__(kRowThreads) void combine_kernel(const float *__restrict__ P,
                                                              const float *__restrict__ P_s,
                                                              const int32_t *__restrict__ idx,
                                                              const float *__restrict__ wgt,
                                                              float *__restrict__ h,
                                                              float *__restrict__ y_out,
                                                              OT *__restrict__ xhat_out,
                                                              OT *__restrict__ xpk_out, int H, int K,
                                                              float eps, const int32_t *__restrict__ gate) {
  __shared__ float red[kRowThreads / 64];
  const int t = blockIdx.x;
  if (gated_off(gate)) return;
  const size_t base = (size_t)t * H;
  const int H4 = H / 4;
  float4 hv[kRowVec];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < kRowVec; ++q) {
    const int j = threadIdx.x + q * kRowThreads;
    if (j >= H4) continue;
    float4 y = make_float4(0, 0, 0, 0);
    for (int k0 = 0; k0 < K; k0 += 8) {
      // eight slots' pick, weight and row loads in flight together (rows of
      // unused slots are read but never summed: they may hold stale values)
      int iv[8];
      float gv[8];
      float4 pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = min(k0 + u, K - 1);
        iv[u] = idx[t * K + k];
        gv[u] = wgt[t * K + k];
        pv[u] = reinterpret_cast<const float4 *>(P + ((size_t)t * K + k) * H)[j];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (k0 + u < K && iv[u] >= 0) {
          y.x = fmaf(gv[u], pv[u].x, y.x); y.y = fmaf(gv[u], pv[u].y, y.y);
          y.z = fmaf(gv[u], pv[u].z, y.z); y.w = fmaf(gv[u], pv[u].w, y.w);
        }
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
      if (j < H4) {
        const float4 o = make_float4(hv[q].x * inv, hv[q].y * inv, hv[q].z * inv, hv[q].w * inv);
        store4<OT>(xhat_out, base + 4 * (size_t)j, o);
        if (xpk_out) store4_packed<OT>(xpk_out, t, gridDim.x, 4 * j, o);
      }
    }
  }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_rmsnorm(int wdtype, const float *in, float *copy_out, void *out, void *xpk, int T, int H,
                          int32_t *zero_word, const int32_t *gate, hipStream_t s) {
  if (wdtype == 1)
    rmsnorm_kernel<bf16_t><<<T, kRowThreads, 0, s>>>(in, copy_out, (bf16_t *)out, (bf16_t *)xpk, H, 1e-6f,
                                                     zero_word, gate);
  else
    rmsnorm_kernel<float><<<T, kRowThreads, 0, s>>>(in, copy_out, (float *)out, (float *)xpk, H, 1e-6f,
                                                    zero_word, gate);
  return hipGetLastError();
}

int router_slices(int H) { return H / kRouterSlice; }

template <class W, int NT>
static hipError_t router_launch(const void *xhat, uint32_t *zero_base, int zero_words, const void *w_router,
                                float *part, int T, int H, int E, const int32_t *gate, hipStream_t s) {
  typedef typename W::T WT;
  const dim3 grid((E + 15) / 16, router_slices(H));
  router_kernel<W, NT><<<grid, 64, 0, s>>>((const WT *)xhat, zero_base, zero_words, (const WT *)w_router, part, T,
                                           H, E, gate);
  return hipGetLastError();
}

hipError_t launch_router(int wdtype, const void *xhat, uint32_t *zero_base, int zero_words, const void *w_router,
                         float *part, int T, int H, int E, const int32_t *gate, hipStream_t s) {
  if (wdtype == 1)
    return T <= 16   ? router_launch<WBf16, 1>(xhat, zero_base, zero_words, w_router, part, T, H, E, gate, s)
           : T <= 32 ? router_launch<WBf16, 2>(xhat, zero_base, zero_words, w_router, part, T, H, E, gate, s)
                     : router_launch<WBf16, 4>(xhat, zero_base, zero_words, w_router, part, T, H, E, gate, s);
  return T <= 16   ? router_launch<WF32, 1>(xhat, zero_base, zero_words, w_router, part, T, H, E, gate, s)
         : T <= 32 ? router_launch<WF32, 2>(xhat, zero_base, zero_words, w_router, part, T, H, E, gate, s)
                   : router_launch<WF32, 4>(xhat, zero_base, zero_words, w_router, part, T, H, E, gate, s);
}

template <int NT>
static hipError_t select_launch(const RouteBufs &r, const float *bias, int T, int H, int E, int K, float top_p,
                                int wdtype, const void *xpk, const void *ws_gate_up, void *act_shared, int Is,
                                hipStream_t s) {
  const int grid = T + Is / 16;
  if (wdtype == 2) {
    // 4-bit shared expert: the packed matrix behind a bf16-typed pointer
    const SharedGU<WI4> sg = {(const bf16_t *)xpk, (const bf16_t *)ws_gate_up, (char *)act_shared, H, Is};
    select_kernel<WI4, NT><<<grid, kSelThreads, 0, s>>>(r, bias, router_slices(H), T, E, K, top_p, sg);
  } else if (wdtype == 1) {
    const SharedGU<WBf16> sg = {(const bf16_t *)xpk, (const bf16_t *)ws_gate_up, (char *)act_shared, H, Is};
    select_kernel<WBf16, NT><<<grid, kSelThreads, 0, s>>>(r, bias, router_slices(H), T, E, K, top_p, sg);
  } else {
    const SharedGU<WF32> sg = {(const float *)xpk, (const float *)ws_gate_up, (char *)act_shared, H, Is};
    select_kernel<WF32, NT><<<grid, kSelThreads, 0, s>>>(r, bias, router_slices(H), T, E, K, top_p, sg);
  }
  return hipGetLastError();
}

hipError_t launch_route_select(const RouteBufs &r, const float *bias, int T, int H, int E, int K, float top_p,
                               int wdtype, const void *xpk, const void *ws_gate_up, void *act_shared, int Is,
                               hipStream_t s) {
  // the shared expert's items cover the block in 16-entry column tiles
  return T > 32 ? select_launch<4>(r, bias, T, H, E, K, top_p, wdtype, xpk, ws_gate_up, act_shared, Is, s)
                : select_launch<2>(r, bias, T, H, E, K, top_p, wdtype, xpk, ws_gate_up, act_shared, Is, s);
}

hipError_t launch_coreset(const float *prob, const int32_t *idx, int T, int E, int K, float top_p,
                          uint32_t *bits, int32_t *size, float *mass, hipStream_t s) {
  coreset_kernel<<<1, 256, 0, s>>>(prob, idx, T, E, K, top_p, bits, size, mass);
  return hipGetLastError();
}

hipError_t launch_combine(int wdtype, const float *P, const float *P_s, const int32_t *idx,
                          const float *wgt, float *h, float *y_out, void *xhat_out, void *xpk_out, int T, int H,
                          int K, const int32_t *gate, hipStream_t s) {
  if (wdtype == 1)
    combine_kernel<bf16_t><<<T, kRowThreads, 0, s>>>(P, P_s, idx, wgt, h, y_out, (bf16_t *)xhat_out,
                                                     (bf16_t *)xpk_out, H, K, 1e-6f, gate);
  else
    combine_kernel<float><<<T, kRowThreads, 0, s>>>(P, P_s, idx, wgt, h, y_out, (float *)xhat_out,
                                                    (float *)xpk_out, H, K, 1e-6f, gate);
  return hipGetLastError();
}

}  // namespace bdd
