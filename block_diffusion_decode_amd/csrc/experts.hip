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
#include "stream.hpp"

namespace bdd {

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

// Routed token group of one work item (wave-uniform): one record of the
// selection kernel's list, [expert, positions, (row | position << 16) x
// kTokGroup, 0, 0], where the row of (position t, pick k) in A and P is
// t * K + k.
struct Group {
  const void *w;           // the expert's weights
  int ie;                  // its intermediate size
  int ng;                  // positions in the group, 1..kTokGroup
  int p[kTokGroup];        // row | position << 16 of the group's positions
  const int32_t *rec;      // the record (for per-lane reads)
  __device__ __forceinline__ int row(int t) const { return p[t] & 0xffff; }
  __device__ __forceinline__ int pos(int t) const { return p[t] >> 16; }
  // row of position t where t differs between lanes
  __device__ __forceinline__ int lane_row(int t) const { return rec[2 + t] & 0xffff; }
};

// Resolves routed item j = group * tiles + tile.  Items of one group and
// different tiles are `tiles` apart, so on a grid that is a multiple of 8
// they run on one XCD.  Only scalar loads with no dependence between them, so
// the next item's record can be fetched while the current item streams.
__device__ __forceinline__ Group resolve(int j, int tiles, const RouteBufs &r, const void *w_routed,
                                         size_t expert_bytes, int I, int &tile) {
  Group g;
  const int gi = j / tiles;
  tile = j - gi * tiles;
  const int32_t *rec = r.glist + gi * 8;
  const int e = uniform(rec[0]);
  g.w = static_cast<const char *>(w_routed) + (size_t)e * expert_bytes;
  g.ie = I;
  g.ng = uniform(rec[1]);
#pragma unroll
  for (int t = 0; t < kTokGroup; ++t) g.p[t] = uniform(rec[2 + t]);
  g.rec = rec;
  return g;
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
  const int my_row = my_t < g.ng ? g.lane_row(my_t) : 0;
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
  // q < 4 * NT: gate rows (lanes 0..31); lane + 32 holds the matching up row
  // (q + 4 * NT), which the swap hands to the lower lanes as its second result
  const float up = __uint_as_float(
      __builtin_amdgcn_permlane32_swap(__float_as_uint(tot), __float_as_uint(tot), false, false)[1]);
  if ((lane & 32) == 0 && (lane & ((1 << shift) - 1)) == 0 && my_t < g.ng) {
    const int r = (lane >> shift) / NT;
    A[(size_t)my_row * Imax + i0 + r] = silu(tot) * up;
  }
}

constexpr int kSdSteps = 4;   // k-steps per load batch of the shared down projection

// Down projection of the shared expert for rows h0 .. h0 + 31 (two row tiles)
// and every position.  The four waves split the intermediate dimension; each
// issues all loads of a batch of kSdSteps k-steps at once, and the partial
// tiles are added in LDS (`red`, 16 KiB).  fp32 activations meet bf16 weights
// as a bf16 high part plus a bf16 residual.  P[T*K + t][h].
template <class W>
__device__ __forceinline__ void shared_down_item(const typename W::T *__restrict__ wsd,
                                                 const float *__restrict__ A, int T, int H, int Is, int TK,
                                                 int Imax, int h0, int wave, int lane, float *__restrict__ P,
                                                 f32x4 *red) {
  typedef typename W::T WT;
  constexpr bool BF = std::is_same<W, WBf16>::value;
  constexpr int CH = W::kChunk;
  constexpr int NXP = CH / 4;
  const int li = lane & 15, g = lane >> 4;
  const int ncw = Is / CH / 4;            // chunks of this wave's quarter of I_s
  const int cw0 = wave * ncw;
  const int ksteps = (ncw + 3) / 4;
  const rsrc_t rw = make_rsrc(wsd, (uint32_t)(H * Is) * sizeof(WT));
  const rsrc_t ra = make_rsrc(A + (size_t)TK * Imax, (uint32_t)(T * Imax) * 4u);
  uint32_t rowa[2], rowx[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) rowa[m] = (uint32_t)((h0 + 16 * m + li) * Is) * sizeof(WT);
#pragma unroll
  for (int n = 0; n < 2; ++n) rowx[n] = n * 16 + li < T ? (uint32_t)((n * 16 + li) * Imax) * 4u : kOutOfRange;
  f32x4 acc[2][2];   // [row tile][column tile]
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < ksteps; k0 += kSdSteps) {
    uint4 wa[kSdSteps][2], xa[kSdSteps][2][NXP];
#pragma unroll
    for (int j = 0; j < kSdSteps; ++j) {
      const int c = 4 * (k0 + j) + g;
      const bool live = k0 + j < ksteps && c < ncw;
      const uint32_t cb = (uint32_t)(cw0 + c);
#pragma unroll
      for (int m = 0; m < 2; ++m)
        wa[j][m] = buf_ld16(rw, live ? rowa[m] + cb * CH * sizeof(WT) : kOutOfRange, 0);
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int q = 0; q < NXP; ++q)
          xa[j][n][q] = buf_ld16(ra, live ? rowx[n] + cb * CH * 4u + 16u * q : kOutOfRange, 0);
    }
#pragma unroll
    for (int j = 0; j < kSdSteps; ++j)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        if constexpr (BF) {
          float f[8];
          f[0] = __uint_as_float(xa[j][n][0].x); f[1] = __uint_as_float(xa[j][n][0].y);
          f[2] = __uint_as_float(xa[j][n][0].z); f[3] = __uint_as_float(xa[j][n][0].w);
          f[4] = __uint_as_float(xa[j][n][1].x); f[5] = __uint_as_float(xa[j][n][1].y);
          f[6] = __uint_as_float(xa[j][n][1].z); f[7] = __uint_as_float(xa[j][n][1].w);
          uint4 hi, lo;
          split_hi_lo(f, hi, lo);
#pragma unroll
          for (int m = 0; m < 2; ++m) acc[m][n] = mfma_bf16(wa[j][m], lo, mfma_bf16(wa[j][m], hi, acc[m][n]));
        } else {
#pragma unroll
          for (int m = 0; m < 2; ++m) acc[m][n] = mfma_chunk<W>(wa[j][m], xa[j][n][0], acc[m][n]);
        }
      }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) red[((wave * 2 + m) * 2 + n) * 64 + lane] = acc[m][n];
  __syncthreads();
  {
    // wave w finishes row tile w >> 1, column tile w & 1
    const int m = wave >> 1, n = wave & 1;
    f32x4 v = red[(m * 2 + n) * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[((w * 2 + m) * 2 + n) * 64 + lane];
    const int t = n * 16 + li;
    if (t < T)
      *reinterpret_cast<float4 *>(P + (size_t)(TK + t) * H + h0 + 16 * m + 4 * g) =
          make_float4(v[0], v[1], v[2], v[3]);
  }
  __syncthreads();  // `red` is free for the next item
}

template <class W>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void expert_gateup_kernel(
    const typename W::T *__restrict__ xhat, const typename W::T *__restrict__ wgu, RouteBufs r,
    float *__restrict__ A, int T, int H, int I, int Imax) {
  typedef typename W::T WT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tiles = I / 16;
  const int items = uniform(r.meta[2]) * tiles;
  const uint32_t x_bytes = (uint32_t)(T * H) * sizeof(WT);
  const size_t eb = (size_t)2 * I * H * sizeof(WT);
  int item = blockIdx.x, tile_next = 0;
  Group next;
  if (item < items) next = resolve(item, tiles, r, wgu, eb, I, tile_next);
  for (; item < items; item += gridDim.x) {
    const Group g = next;
    const int tile = tile_next;
    const int nitem = item + (int)gridDim.x;
    if (nitem < items) next = resolve(nitem, tiles, r, wgu, eb, I, tile_next);
    const int i0 = uniform(tile * 16 + wave * 4);
    if (g.ng <= 1)      gateup_group<W, 1>(g, xhat, x_bytes, H, Imax, i0, lane, A);
    else if (g.ng <= 2) gateup_group<W, 2>(g, xhat, x_bytes, H, Imax, i0, lane, A);
    else                gateup_group<W, 4>(g, xhat, x_bytes, H, Imax, i0, lane, A);
  }
}

constexpr int kDownRowsPerWave = 32;  // four batches of 8 rows (128 rows per item)
constexpr int kDownSub = 2;           // positions per pass when activations reload per step

template <int NX>
struct DnBufs {
  uint4 w[8];
  uint4 x[NX];
};

// Down projection of positions [sub0, sub0 + NT) of a group for this wave's
// rows h0 + 8b + r (b = 0..3, r = 0..7) of W_d [H][ie]: lane l covers chunks
// l, l + 64, ... of each row, so a load reads one contiguous 1 KiB row
// segment.  With a single chunk per lane (ONCE: ie <= 64 chunks) the lane's
// activation chunks are read and split once per pass, else with every step.
// The fp32 activations meet bf16 weights as a bf16 high part plus a bf16
// residual (two dot passes).  P[row][h] = A_row . W_d[h] (the routing weight
// is applied by the combine).
template <class W, int NT, int sub0, bool ONCE>
__device__ __forceinline__ void down_group(const Group &g, const float *__restrict__ A,
                                           uint32_t a_bytes, int H, int Imax, int h0, int lane,
                                           float *__restrict__ P) {
  typedef typename W::T WT;
  constexpr bool BF = std::is_same<W, WBf16>::value;
  constexpr int CH = W::kChunk;
  constexpr int NXP = CH / 4;  // 16-byte activation loads per position and chunk
  const int NC = g.ie / CH, nq = ONCE ? 1 : (NC + 63) / 64;
  const int nb = kDownRowsPerWave / 8;
  const int ngs = min(NT, g.ng - sub0);
  const uint32_t rowb = (uint32_t)g.ie * sizeof(WT);
  const rsrc_t rw = make_rsrc(g.w, (uint32_t)H * rowb);
  const rsrc_t ra = make_rsrc(A, a_bytes);
  uint32_t aoff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    aoff[t] = t < ngs ? (uint32_t)uniform(g.row(sub0 + t)) * (uint32_t)Imax * 4u : kOutOfRange;
  constexpr int shift = 6 - log2i<8 * NT>();
  const int my_t = (lane >> shift) % NT;
  const int my_row = my_t < ngs ? g.lane_row(sub0 + my_t) : 0;
  auto load_act = [&](int c, bool live, uint4 *x) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < NXP; ++j)
        x[t * NXP + j] = buf_ld16(ra, live ? aoff[t] + (uint32_t)(c * CH * 4 + 16 * j) : kOutOfRange, 0);
  };
  // activation operands of one chunk: bf16 weights take (high, residual)
  // pairs, fp32 weights the fp32 values
  uint4 xop[NT][2];
  auto prep = [&](const uint4 *x) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (BF) {
        float f[8];
        f[0] = __uint_as_float(x[2 * t].x); f[1] = __uint_as_float(x[2 * t].y);
        f[2] = __uint_as_float(x[2 * t].z); f[3] = __uint_as_float(x[2 * t].w);
        f[4] = __uint_as_float(x[2 * t + 1].x); f[5] = __uint_as_float(x[2 * t + 1].y);
        f[6] = __uint_as_float(x[2 * t + 1].z); f[7] = __uint_as_float(x[2 * t + 1].w);
        split_hi_lo(f, xop[t][0], xop[t][1]);
      } else {
        xop[t][0] = x[t];
      }
    }
  };
  if constexpr (ONCE) {
    uint4 x[NT * NXP];
    load_act(lane, lane < NC, x);
    prep(x);
  }
  float acc[8][NT];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;
  constexpr int NX = ONCE ? 1 : NT * NXP;
  auto load = [&](int s, DnBufs<NX> &b) {
    const int bb = s / nq, q = s - bb * nq;
    const int c = lane + 64 * q;
    const bool live = bb < nb && c < NC;
    const uint32_t vo = live ? (uint32_t)c * 16u : kOutOfRange;
#pragma unroll
    for (int r = 0; r < 8; ++r) b.w[r] = buf_ld16(rw, vo, (uint32_t)(h0 + 8 * min(bb, nb - 1) + r) * rowb);
    if constexpr (!ONCE) load_act(c, live, b.x);
  };
  auto step = [&](int s, const DnBufs<NX> &b) {
    if constexpr (!ONCE) prep(b.x);
    if constexpr (BF) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[r][t] = dot8bf(b.w[r], xop[t][1], dot8bf(b.w[r], xop[t][0], acc[r][t]));
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float wf[4];
        chunk_to_f32<W>(b.w[r], wf);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float xf[4];
          chunk_to_f32<W>(xop[t][0], xf);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r][t] = fmaf(wf[j], xf[j], acc[r][t]);
        }
      }
    }
  };
  // end of a batch of 8 rows: reduce over the wave and store
  auto post = [&](int s) {
    const int bb = s / nq;
    if (s - bb * nq == nq - 1) {
      float v[8 * NT];
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) { v[r * NT + t] = acc[r][t]; acc[r][t] = 0.f; }
      const float tot = reduce_scatter<8 * NT>(v, lane);
      if ((lane & ((1 << shift) - 1)) == 0 && my_t < ngs) {
        const int r = (lane >> shift) / NT;
        P[(size_t)my_row * H + h0 + 8 * bb + r] = tot;
      }
    }
  };
  DnBufs<NX> b0, b1;
  if constexpr (NT >= 4 || !ONCE) {
    // with four positions, or activations reloaded per step, the registers
    // do not hold the epilogue's state beside two full buffers: the epilogue
    // runs with one batch in flight
    pipeline(nb * nq, b0, b1, load, [&](int s, const DnBufs<NX> &b) { step(s, b); post(s); });
  } else {
    pipeline_post(nb * nq, b0, b1, load, step, post);
  }
}

template <class W, int sub0, bool ONCE>
__device__ __forceinline__ void down_pass(const Group &g, const float *__restrict__ A, uint32_t a_bytes, int H,
                                          int Imax, int h0, int lane, float *__restrict__ P) {
  if (g.ng - sub0 <= 1) down_group<W, 1, sub0, ONCE>(g, A, a_bytes, H, Imax, h0, lane, P);
  else                  down_group<W, kDownSub, sub0, ONCE>(g, A, a_bytes, H, Imax, h0, lane, P);
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
  const int s_items = Is > 0 ? H / 32 : 0;   // shared expert: 32 rows x every position per item
  __shared__ f32x4 red[4 * 2 * 2 * 64];
  const int items = s_items + uniform(r.meta[2]) * tiles;
  const uint32_t a_bytes = (uint32_t)(T * K + T) * (uint32_t)Imax * 4u;
  const size_t eb = (size_t)H * I * sizeof(WT);
  const int stride = gridDim.x;
  int item = blockIdx.x, tile_next = 0;
  Group next;
  if (item < items && item >= s_items) next = resolve(item - s_items, tiles, r, wd, eb, I, tile_next);
  for (; item < items; item += stride) {
    const int nitem = item + stride;
    if (item < s_items) {
      if (nitem < items && nitem >= s_items) next = resolve(nitem - s_items, tiles, r, wd, eb, I, tile_next);
      shared_down_item<W>(wsd, A, T, H, Is, T * K, Imax, item * 32, wave, lane, P, red);
      continue;
    }
    const Group g = next;
    const int tile = tile_next;
    if (nitem < items) next = resolve(nitem - s_items, tiles, r, wd, eb, I, tile_next);
    const int h0 = uniform(tile * 4 * kDownRowsPerWave + wave * kDownRowsPerWave);
    if (g.ie <= 64 * W::kChunk) {
      // one pass over the whole group: the activations sit in registers
      static_assert(kTokGroup == 4, "token groups of at most 4 positions");
      if (g.ng <= 1)      down_group<W, 1, 0, true>(g, A, a_bytes, H, Imax, h0, lane, P);
      else if (g.ng <= 2) down_group<W, 2, 0, true>(g, A, a_bytes, H, Imax, h0, lane, P);
      else                down_group<W, 4, 0, true>(g, A, a_bytes, H, Imax, h0, lane, P);
    } else {
      // passes of kDownSub positions (group rows are picked with constant indices)
      static_assert(kTokGroup == 2 * kDownSub, "two down passes per token group");
      down_pass<W, 0, false>(g, A, a_bytes, H, Imax, h0, lane, P);
      if (g.ng > kDownSub) down_pass<W, kDownSub, false>(g, A, a_bytes, H, Imax, h0, lane, P);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

int expert_items_max(int T, int H, int E, int K, int I, int Is, bool gateup) {
  (void)T;
  const int groups = expert_groups_max(T, E, K);
  if (gateup) return groups * (I / 16);
  return (Is > 0 ? H / 32 : 0) + groups * (H / (4 * kDownRowsPerWave));
}

hipError_t launch_expert_gateup(int wdtype, const void *xhat, const void *w_gate_up, const RouteBufs &r, float *A,
                                int T, int H, int I, int Imax, int grid, hipStream_t s) {
  if (wdtype == 1)
    expert_gateup_kernel<WBf16><<<grid, 256, 0, s>>>((const bf16_t *)xhat, (const bf16_t *)w_gate_up, r, A, T, H, I,
                                                     Imax);
  else
    expert_gateup_kernel<WF32><<<grid, 256, 0, s>>>((const float *)xhat, (const float *)w_gate_up, r, A, T, H, I,
                                                    Imax);
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
