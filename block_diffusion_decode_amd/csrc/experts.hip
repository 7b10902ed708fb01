// Expert FFNs of one MoE layer: the routed experts of the block's union and
// the shared expert, as one work list per projection.  Each routed expert's
// weights stream from HBM once per block for every position routed to it.
//
// Pages: [P1] aitujian.cn article on Clover-35B-A3B-Preview, section 五 (the 32
// positions of a block reach a union of experts far larger than 8; the bytes
// read grow much less than the tokens produced because the same weights serve
// many positions) and section 四 (one shared expert per layer).  The expert
// activation (SwiGLU) is not on the pages; it is the reading this library
// documents in its header.
//
// A routed expert sees ~1.6 positions on average at the Clover shape (at most
// 32), so its contraction is a matrix-vector product: VALU dot products on
// weights streamed with 16-byte buffer loads.  Work items are (token group,
// row tile); a token group is up to kTokGroup positions of one expert (the
// selection kernel lists them), and the shared expert contributes the first
// ceil(T / kTokGroup) groups, covering every position.  A wave owns 8 weight
// rows of its item; lane l covers 16-byte chunks l, l + 64, ... of every row,
// so a load instruction reads one contiguous 1 KiB segment of a row.  The
// positions' activations are read per chunk straight from L2 next to the
// weights, so the four waves of a workgroup never synchronise.
#include <type_traits>

#include "kernels.hpp"

namespace bdd {

// A buffer offset past every descriptor used here: such a load returns zeros
// without a memory access.  It pads the last prefetch of a stream and masks
// positions beyond a group.
constexpr uint32_t kOutOfRange = 0x7ff00000u;

template <class W>
__device__ __forceinline__ void chunk_to_f32(const uint4 &v, float (&f)[W::kChunk]);
template <>
__device__ __forceinline__ void chunk_to_f32<WBf16>(const uint4 &v, float (&f)[8]) { unpack8(v, f); }
template <>
__device__ __forceinline__ void chunk_to_f32<WF32>(const uint4 &v, float (&f)[4]) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// a.lo * b.lo + a.hi * b.hi + c for two bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}
__device__ __forceinline__ float dot8bf(const uint4 &w, const uint4 &x, float c) {
  c = dot2bf(w.x, x.x, c);
  c = dot2bf(w.y, x.y, c);
  c = dot2bf(w.z, x.z, c);
  return dot2bf(w.w, x.w, c);
}

// Token group of one work item (wave-uniform).  Assignment rows index A and
// P: routed (position t, pick k) -> t * K + k, shared expert position t ->
// T * K + t.
struct Group {
  const void *w;           // the expert's weights
  int ie;                  // its intermediate size
  int ng;                  // positions in the group, 1..kTokGroup
  const int32_t *asg;      // routed: the group's assignment rows; shared: null
  int base;                // shared: first position of the group
  int TK;                  // T * K
  int K;
  // assignment row and block position of the group's t-th position
  __device__ __forceinline__ int row(int t) const { return asg ? asg[t] : TK + base + t; }
  __device__ __forceinline__ int pos(int t) const { return asg ? asg[t] / K : base + t; }
};

// Resolves work item `item` of a list made of `s_items` shared-expert items
// (ceil(T / kTokGroup) groups x tiles_s) followed by the routed groups of the
// selection kernel (r.glist) x tiles.  Items of one group and different tiles
// are `tiles` apart, so on a grid that is a multiple of 8 they run on one XCD
// and a group's repeated weight reads stay in that XCD's L2.
__device__ __forceinline__ Group resolve(int item, int s_items, int tiles_s, int tiles, const RouteBufs &r,
                                         const void *w_routed, const void *w_shared, size_t expert_bytes,
                                         int I, int Is, int T, int K, int &tile) {
  Group g;
  g.TK = T * K;
  g.K = K;
  if (item < s_items) {
    const int grp = item / tiles_s;
    tile = item - grp * tiles_s;
    g.w = w_shared;
    g.ie = Is;
    g.base = grp * kTokGroup;
    g.ng = min(kTokGroup, T - g.base);
    g.asg = nullptr;
  } else {
    const int j = item - s_items;
    const int gi = j / tiles;
    tile = j - gi * tiles;
    const int v = uniform(r.glist[gi]);
    const int u = v >> 8, g0 = v & 255;
    const int e = uniform(r.union_list[u]);
    const int n = uniform(r.slot_n[u]);
    g.w = static_cast<const char *>(w_routed) + (size_t)e * expert_bytes;
    g.ie = I;
    g.base = 0;
    g.ng = min(kTokGroup, n - g0);
    g.asg = r.slot_asg + u * kMaxT + g0;
  }
  return g;
}

// Two-deep streaming loop: step s's loads are issued before step s-1's
// arithmetic.  The prefetch past the last step is an out-of-range load, so the
// loop always has the same loads in flight and the compiler's in-order wait
// counts stay exact (a conditional prefetch makes it drain every load).
template <class Bufs, class Load, class Step>
__device__ __forceinline__ void pipeline(int steps, Bufs &b0, Bufs &b1, Load load, Step step) {
  load(0, b0);
  for (int s = 0; s < steps; s += 2) {
    load(s + 1, b1);
    step(s, b0);
    if (s + 1 >= steps) break;
    load(s + 2, b0);
    step(s + 1, b1);
  }
}

template <int NT>
struct GuBufs {
  uint4 w[8];
  uint4 x[NT];
};

// Gate/up of one (group, tile) item for this wave: gate rows i0 + r and the
// matching up rows ie + i0 + r (r = 0..3), read in full, against the group's
// normalised positions.  A[row][i] = silu(gate) * up.
template <class W, int NT>
__device__ __forceinline__ void gateup_group(const Group &g, const typename W::T *__restrict__ xhat,
                                             uint32_t x_bytes, int H, int Imax, int i0, int lane,
                                             float *__restrict__ A) {
  typedef typename W::T WT;
  constexpr int CH = W::kChunk;
  const int NC = H / CH, nq = (NC + 63) / 64;
  const uint32_t rowb = (uint32_t)H * sizeof(WT);
  const rsrc_t rw = make_rsrc(g.w, 2u * (uint32_t)g.ie * rowb);
  const rsrc_t rx = make_rsrc(xhat, x_bytes);
  uint32_t xoff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) xoff[t] = t < g.ng ? (uint32_t)uniform(g.pos(t)) * rowb : kOutOfRange;
  // the lane's output: value index q = r * NT + t after the wave reduction
  constexpr int shift = 6 - log2i<8 * NT>();
  const int my_t = (lane >> shift) % NT;
  const int my_row = my_t < g.ng ? g.row(my_t) : 0;
  float acc[8][NT];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;
  auto load = [&](int s, GuBufs<NT> &b) {
    const int c = lane + 64 * s;
    const bool live = s < nq && c < NC;
    const uint32_t vo = live ? (uint32_t)c * 16u : kOutOfRange;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      b.w[r] = buf_ld16(rw, vo, (uint32_t)(r < 4 ? i0 + r : g.ie + i0 + r - 4) * rowb);
#pragma unroll
    for (int t = 0; t < NT; ++t) b.x[t] = buf_ld16(rx, live ? xoff[t] + vo : kOutOfRange, 0);
  };
  auto step = [&](int, const GuBufs<NT> &b) {
    if constexpr (std::is_same<W, WBf16>::value) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[r][t] = dot8bf(b.w[r], b.x[t], acc[r][t]);
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float wf[4];
        chunk_to_f32<W>(b.w[r], wf);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float xf[4];
          chunk_to_f32<W>(b.x[t], xf);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r][t] = fmaf(wf[j], xf[j], acc[r][t]);
        }
      }
    }
  };
  GuBufs<NT> b0, b1;
  pipeline(nq, b0, b1, load, step);
  float v[8 * NT];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) v[r * NT + t] = acc[r][t];
  const float tot = reduce_scatter<8 * NT>(v, lane);
  // q < 4 * NT: gate rows; lane ^ 32 holds the matching up row (q + 4 * NT)
  const float up = __shfl_xor(tot, 32);
  if ((lane & 32) == 0 && (lane & ((1 << shift) - 1)) == 0 && my_t < g.ng) {
    const int r = (lane >> shift) / NT;
    A[(size_t)my_row * Imax + i0 + r] = silu(tot) * up;
  }
}

template <class W>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void expert_gateup_kernel(const typename W::T *__restrict__ xhat,
                                                            const typename W::T *__restrict__ wgu,
                                                            const typename W::T *__restrict__ wsgu,
                                                            RouteBufs r, float *__restrict__ A, int T,
                                                            int H, int K, int I, int Is, int Imax) {
  typedef typename W::T WT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tiles_s = Is / 16, tiles = I / 16;
  const int s_items = Is > 0 ? (T + kTokGroup - 1) / kTokGroup * tiles_s : 0;
  const int items = s_items + uniform(r.meta[2]) * tiles;
  const uint32_t x_bytes = (uint32_t)(T * H) * sizeof(WT);
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    int tile;
    const Group g = resolve(item, s_items, tiles_s, tiles, r, wgu, wsgu, (size_t)2 * I * H * sizeof(WT),
                            I, Is, T, K, tile);
    const int i0 = uniform(tile * 16 + wave * 4);
    if (g.ng <= 1)      gateup_group<W, 1>(g, xhat, x_bytes, H, Imax, i0, lane, A);
    else if (g.ng <= 2) gateup_group<W, 2>(g, xhat, x_bytes, H, Imax, i0, lane, A);
    else                gateup_group<W, 4>(g, xhat, x_bytes, H, Imax, i0, lane, A);
  }
}

constexpr int kDownRowsPerWave = 32;  // 128 rows per item
constexpr int kDownSub = 2;           // positions per pass of the down projection

template <int NX>
struct DnBufs {
  uint4 w[8];
  uint4 x[NX];
};

// Down projection of positions [sub0, sub0 + NT) of a group for this wave's
// rows h0 .. h0 + 31 of W_d [H][ie].  Lane l works on rows h0 + (l >> 4) + 4i
// (i = 0..7) and, at step s, on chunk (l & 15) + 16 s of those rows: a load
// instruction reads four 256-byte row segments, and a row's partial sums meet
// in one 16-lane group, reduced once per item.  The fp32 activations meet
// bf16 weights as a bf16 high part plus a bf16 residual (two dot passes).
// P[row][h] = A_row . W_d[h] (the routing weight is applied by the combine).
template <class W, int NT>
__device__ __forceinline__ void down_group(const Group &g, int sub0, const float *__restrict__ A,
                                           uint32_t a_bytes, int H, int Imax, int h0, int lane,
                                           float *__restrict__ P) {
  typedef typename W::T WT;
  constexpr int CH = W::kChunk;
  constexpr int NXP = CH / 4;  // 16-byte activation loads per position and chunk
  const int NC = g.ie / CH, steps = (NC + 15) / 16;
  const int lg = lane >> 4, lc = lane & 15;
  const int ngs = min(NT, g.ng - sub0);
  const uint32_t rowb = (uint32_t)g.ie * sizeof(WT);
  const rsrc_t rw = make_rsrc(g.w, (uint32_t)H * rowb);
  const rsrc_t ra = make_rsrc(A, a_bytes);
  uint32_t aoff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    aoff[t] = t < ngs ? (uint32_t)uniform(g.row(sub0 + t)) * (uint32_t)Imax * 4u : kOutOfRange;
  // after the 16-lane reduction lane l holds value q = i * NT + t
  constexpr int shift = 4 - log2i<8 * NT>();
  const int my_q = lc >> shift;
  const int my_t = my_q % NT;
  const int my_row = my_t < ngs ? g.row(sub0 + my_t) : 0;
  float acc[8][NT];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = 0.f;
  auto load = [&](int s, DnBufs<NT * NXP> &b) {
    const int c = lc + 16 * s;
    const bool live = s < steps && c < NC;
    const uint32_t vo = live ? (uint32_t)lg * rowb + (uint32_t)c * 16u : kOutOfRange;
#pragma unroll
    for (int i = 0; i < 8; ++i) b.w[i] = buf_ld16(rw, vo, (uint32_t)(h0 + 4 * i) * rowb);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < NXP; ++j)
        b.x[t * NXP + j] = buf_ld16(ra, live ? aoff[t] + (uint32_t)(c * CH * 4 + 16 * j) : kOutOfRange, 0);
  };
  auto step = [&](int, const DnBufs<NT * NXP> &b) {
    if constexpr (std::is_same<W, WBf16>::value) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float x[8];
        x[0] = __uint_as_float(b.x[2 * t].x); x[1] = __uint_as_float(b.x[2 * t].y);
        x[2] = __uint_as_float(b.x[2 * t].z); x[3] = __uint_as_float(b.x[2 * t].w);
        x[4] = __uint_as_float(b.x[2 * t + 1].x); x[5] = __uint_as_float(b.x[2 * t + 1].y);
        x[6] = __uint_as_float(b.x[2 * t + 1].z); x[7] = __uint_as_float(b.x[2 * t + 1].w);
        uint4 hi, lo;
        split_hi_lo(x, hi, lo);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i][t] = dot8bf(b.w[i], lo, dot8bf(b.w[i], hi, acc[i][t]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float wf[4];
        chunk_to_f32<W>(b.w[i], wf);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float xf[4];
          chunk_to_f32<W>(b.x[t], xf);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][t] = fmaf(wf[j], xf[j], acc[i][t]);
        }
      }
    }
  };
  DnBufs<NT * NXP> b0, b1;
  pipeline(steps, b0, b1, load, step);
  float v[8 * NT];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) v[i * NT + t] = acc[i][t];
  reduce_scatter_step<8 * NT, 8>(v, lane);
  if ((lc & ((1 << shift) - 1)) == 0 && my_t < ngs) {
    const int i = my_q / NT;
    P[(size_t)my_row * H + h0 + lg + 4 * i] = v[0];
  }
}

template <class W>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void expert_down_kernel(const float *__restrict__ A,
                                                          const typename W::T *__restrict__ wd,
                                                          const typename W::T *__restrict__ wsd,
                                                          RouteBufs r, float *__restrict__ P, int T,
                                                          int H, int K, int I, int Is, int Imax) {
  typedef typename W::T WT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tiles = H / (4 * kDownRowsPerWave);
  const int s_items = Is > 0 ? (T + kTokGroup - 1) / kTokGroup * tiles : 0;
  const int items = s_items + uniform(r.meta[2]) * tiles;
  const uint32_t a_bytes = (uint32_t)(T * K + T) * (uint32_t)Imax * 4u;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    int tile;
    const Group g = resolve(item, s_items, tiles, tiles, r, wd, wsd, (size_t)H * I * sizeof(WT), I, Is,
                            T, K, tile);
    const int h0 = uniform(tile * 4 * kDownRowsPerWave + wave * kDownRowsPerWave);
    for (int sub0 = 0; sub0 < g.ng; sub0 += kDownSub) {
      if (g.ng - sub0 <= 1) down_group<W, 1>(g, sub0, A, a_bytes, H, Imax, h0, lane, P);
      else                  down_group<W, kDownSub>(g, sub0, A, a_bytes, H, Imax, h0, lane, P);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

int expert_items_max(int T, int H, int E, int K, int I, int Is, bool gateup) {
  const int groups = expert_groups_max(T, E, K);
  const int s_groups = Is > 0 ? (T + kTokGroup - 1) / kTokGroup : 0;
  if (gateup) return s_groups * (Is / 16) + groups * (I / 16);
  return (s_groups + groups) * (H / (4 * kDownRowsPerWave));
}

hipError_t launch_expert_gateup(int wdtype, const void *xhat, const void *w_gate_up, const void *ws_gate_up,
                                const RouteBufs &r, float *A, int T, int H, int K, int I, int Is, int Imax,
                                int grid, hipStream_t s) {
  if (wdtype == 1)
    expert_gateup_kernel<WBf16><<<grid, 256, 0, s>>>((const bf16_t *)xhat, (const bf16_t *)w_gate_up,
                                                     (const bf16_t *)ws_gate_up, r, A, T, H, K, I, Is, Imax);
  else
    expert_gateup_kernel<WF32><<<grid, 256, 0, s>>>((const float *)xhat, (const float *)w_gate_up,
                                                    (const float *)ws_gate_up, r, A, T, H, K, I, Is, Imax);
  return hipGetLastError();
}

hipError_t launch_expert_down(int wdtype, const float *A, const void *w_down, const void *ws_down,
                              const RouteBufs &r, float *P, int T, int H, int K, int I, int Is, int Imax,
                              int grid, hipStream_t s) {
  if (wdtype == 1)
    expert_down_kernel<WBf16><<<grid, 256, 0, s>>>(A, (const bf16_t *)w_down, (const bf16_t *)ws_down, r, P,
                                                   T, H, K, I, Is, Imax);
  else
    expert_down_kernel<WF32><<<grid, 256, 0, s>>>(A, (const float *)w_down, (const float *)ws_down, r, P, T,
                                                  H, K, I, Is, Imax);
  return hipGetLastError();
}

}  // namespace bdd
