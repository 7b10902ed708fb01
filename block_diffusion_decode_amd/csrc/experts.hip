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
// A routed expert sees ~1.6 positions on average at the Clover shape under
// flat routing, so its contraction is a matrix-vector product: VALU dot
// products on weights streamed with 16-byte buffer loads.  Work items are
// (token group, row tile); a token group is up to kTokGroup positions of one
// expert (see the work lists below).  A wave owns 8 weight rows of its
// item; lane l covers 16-byte chunks l, l + 64, ... of every row, so a load
// instruction reads one contiguous 1 KiB segment of a row.  The positions'
// activations are read per chunk straight from L2 next to the weights, so the
// four waves of a workgroup never synchronise.
//
// An expert with more positions than a token group holds (skewed routing
// sends most of a block to a few experts) and the shared expert (every
// position) run as dense items instead: MFMA tiles over all their positions
// at once, so their weights stream once per block rather than once per group.
#include <type_traits>

#include "int4.hpp"
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

// ---------------------------------------------------------------------------
// Work lists.  The selection leaves, per expert, the mask of the positions
// whose final picks include it (sync.mask2) and each such pick's slot k
// (sync.kslot); the row of (position t, slot k) in A and P is t * K + k.
// Every workgroup of an expert kernel rebuilds the block's lists from the
// masks in LDS: the experts with more than kTokGroup positions (dense, in
// ascending id), then those with 1 .. kTokGroup (one token group each, in
// ascending id).  An expert's entry j is its j-th position in ascending order.
// ---------------------------------------------------------------------------
struct ListShared {
  posmask_t msk[kMaxE];   // position masks: dense experts, then token groups
  int32_t exp[kMaxE];     // their expert ids
  int wsum[4];            // per-wave counts (dense | groups << 16)
};

// Builds the lists (all 256 threads; ends with a barrier) and returns the
// number of dense experts | token groups << 16.  With `report` (one
// workgroup of the layer) it also writes the union size and, without a
// coreset, the union as the coreset.
__device__ __forceinline__ int build_lists(const RouteBufs &r, int E, ListShared &L, bool report) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const posmask_t m = tid < E ? r.sync.mask2[tid] : 0ull;
  const int npos = __popcll(m);
  const bool dense = npos > kTokGroup, grp = npos > 0 && !dense;
  const unsigned long long bd = __ballot(dense), bg = __ballot(grp);
  if (lane == 0) L.wsum[wave] = __popcll(bd) | __popcll(bg) << 16;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int v = L.wsum[w];
    pre += w < wave ? v : 0;
    tot += v;
  }
  const int nd = tot & 0xffff;
  const unsigned long long below = lanes_below(lane);
  if (dense) {
    const int at = (pre & 0xffff) + __popcll(bd & below);
    L.exp[at] = tid;
    L.msk[at] = m;
  }
  if (grp) {
    const int at = nd + (pre >> 16) + __popcll(bg & below);
    L.exp[at] = tid;
    L.msk[at] = m;
  }
  if (report) {
    const int nu = nd + (tot >> 16);
    if (tid == 0) {
      r.meta[0] = nu;
      if (r.n_distinct_out) *r.n_distinct_out = nu;
      if (!r.coreset) {
        r.meta[1] = nu;
        if (r.coreset_size_out) *r.coreset_size_out = nu;
      }
    }
    // without a coreset every expert with a pick is reported as its member
    if (!r.coreset && lane == 0 && 64 * wave < E) r.cs_bits[2 * wave] = (uint32_t)(bd | bg);
    if (!r.coreset && lane == 32 && 64 * wave + 32 < E) r.cs_bits[2 * wave + 1] = (uint32_t)((bd | bg) >> 32);
  }
  __syncthreads();
  return tot;
}

// The pick slot of expert e in position t's final picks.
__device__ __forceinline__ int pick_slot(const RouteBufs &r, int e, int t) {
  return (int)((r.sync.kslot[e * (kMaxT / 4) + (t >> 2)] >> (8 * (t & 3))) & 0xffu);
}

// Routed token group of one work item (wave-uniform): up to kTokGroup
// positions of one expert and the expert's slot words (lane l < kMaxT / 4
// holds word l).  A row is formed only where it is used, so the slot load of
// a prefetched group stays in flight until then.
struct Group {
  const void *w;             // the expert's weights
  int ie;                    // its intermediate size
  int ng;                    // positions in the group, 1..kTokGroup
  int K;                     // picks per position
  int pp[kTokGroup];         // positions, ascending (0 past the group)
  uint32_t wv;               // this lane's slot word of the expert
  __device__ __forceinline__ int pos(int t) const { return pp[t]; }
  __device__ __forceinline__ int row(int t) const {
    const uint32_t word = (uint32_t)__builtin_amdgcn_readlane((int)wv, pp[t] >> 2);
    return pp[t] * K + (int)((word >> (8 * (pp[t] & 3))) & 0xffu);
  }
  // row of entry t where t differs between lanes (value arithmetic: a
  // runtime index would leave the arrays in memory)
  __device__ __forceinline__ int lane_row(int t) const {
    int v = row(0);
#pragma unroll
    for (int j = 1; j < kTokGroup; ++j) v = t == j ? row(j) : v;
    return v;
  }
};

// Resolves routed item j = group * tiles + tile.  Items of one group and
// different tiles are `tiles` apart, so on a grid that is a multiple of 8
// they run on one XCD.  The group's mask comes from LDS and its slot words
// from one vector load (a load at a wave-uniform address would be moved to a
// scalar register at once, waiting for it there), so the next item's group
// can be fetched while the current item streams.
__device__ __forceinline__ Group resolve(int j, int tiles, const RouteBufs &r, const ListShared &L, int nd, int K,
                                         const void *w_routed, size_t expert_bytes, int I, int &tile) {
  Group g;
  const int gi = j / tiles;
  tile = j - gi * tiles;
  const int e = uniform(L.exp[nd + gi]);
  posmask_t m = uniform64(L.msk[nd + gi]);
  g.w = static_cast<const char *>(w_routed) + (size_t)e * expert_bytes;
  g.ie = I;
  g.ng = __popcll(m);
  g.K = K;
#pragma unroll
  for (int t = 0; t < kTokGroup; ++t) {
    const int pt = m ? __ffsll((long long)m) - 1 : 0;
    m &= m - 1ull;
    g.pp[t] = pt;
  }
  g.wv = r.sync.kslot[e * (kMaxT / 4) + (__lane_id() & (kMaxT / 4 - 1))];
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

constexpr int kDenseRowTiles = 2;   // 16-row tiles per dense down item (32 rows)
// k-steps per load batch of a dense down projection: all of a wave's quarter
// of I = 512 in one batch at two row tiles
template <int MT>
constexpr int dense_down_batch() { return MT <= 2 ? 4 : 2; }

// Down projection of one dense expert, W_d [H][ie], for rows h0 .. h0 + 16 MT - 1
// (MT row tiles) and up to 16 NT column entries, from the expert's packed
// activation slot (see act_unit).  Lane (li, g) names entries li + 16 n:
// live[n] < 0 where there is no entry, and row[n] is the entry's row in P
// (read only at the end, so it may still be in flight when the item
// starts).  The four waves split the intermediate dimension; each issues the
// loads of a batch of k-steps at once, stages its weights through its own
// span of `red` (MT * 2 KiB), and the partial tiles are then added through
// all of it.  With bf16
// weights the activations enter as bf16 high parts and residuals (two MFMA
// passes); every activation load serves MT weight tiles.
// P[row][h] = A_entry . W_d[h].
template <class W, int MT, int NT>
__device__ __forceinline__ void dense_down_item(const typename W::T *__restrict__ w, int ie,
                                                const char *__restrict__ act, int H, const int (&live)[NT],
                                                const int (&row)[NT], int h0, int wave, int lane,
                                                float *__restrict__ P, f32x4 *red) {
  typedef typename W::T WT;
  constexpr bool BF = std::is_same<W, WBf16>::value;
  constexpr int CH = W::kChunk;
  constexpr int NP = act_planes<W>();
  const int li = lane & 15, g = lane >> 4;
  const int ncw = ie / CH / 4;            // chunks of this wave's quarter of ie
  const int cw0 = wave * ncw;
  const rsrc_t rw = make_rsrc(w, (uint32_t)(H * ie) * sizeof(WT));
  const rsrc_t ra = make_rsrc(act, (uint32_t)ie * kActSlotPerI);
  f32x4 acc[MT][NT];   // [row tile][column tile]
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int kSdSteps = dense_down_batch<MT>();
  static_assert(kSdSteps % 2 == 0, "the dense down item streams whole units of 2 k-steps");
  constexpr int UB = kSdSteps / 2;          // units per load batch
  const int nunits = (ncw + 7) / 8;
  // weights staged as in the dense gate/up item: a load reads 128 bytes of
  // each of 8 rows (rows 8j + sr, the row offsets wave-uniform), and the wave
  // passes each unit through its own MT * 2 KiB of `red`
  const int sr = lane >> 3, sc = lane & 7;
  const uint32_t rowa = (uint32_t)((h0 + sr) * ie) * sizeof(WT), rows8 = (uint32_t)(8 * ie) * sizeof(WT);
  // (inside the span the wave's partial tiles take afterwards, MT * NT * 64)
  f32x4 *stage = red + wave * MT * NT * 64;
  for (int u0 = 0; u0 < nunits; u0 += UB) {
    uint4 wa[UB][2 * MT], xa[2 * UB][NT][NP];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const bool live_u = u0 + u < nunits;
      const int cs = 8 * (u0 + u) + sc;
      const uint32_t vo = live_u && cs < ncw ? rowa + (uint32_t)((cw0 + cs) * CH) * sizeof(WT) : kOutOfRange;
#pragma unroll
      for (int j = 0; j < 2 * MT; ++j) wa[u][j] = buf_ld16(rw, vo, (uint32_t)j * rows8);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 8 * (u0 + u) + 4 * h + g;
        const bool live_c = live_u && c < ncw;
        const int C = cw0 + c;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int q = 0; q < NP; ++q)
            xa[2 * u + h][n][q] =
                buf_ld16(ra, live_c && live[n] >= 0 ? act_unit(C, q, 16 * n + li, NP) * 16u : kOutOfRange, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      // lanes read rows other lanes wrote: in-order LDS, fenced against the compiler
#pragma unroll
      for (int j = 0; j < 2 * MT; ++j)
        stage[stage_slot(j >> 1, 8 * (j & 1) + sr, sc)] = __builtin_bit_cast(f32x4, wa[u][j]);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      uint4 a[2][MT];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int m = 0; m < MT; ++m) a[h][m] = __builtin_bit_cast(uint4, stage[stage_slot(m, li, 4 * h + g)]);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            const uint4 *x = xa[2 * u + h][n];
            if constexpr (BF) acc[m][n] = mfma_bf16(a[h][m], x[1], mfma_bf16(a[h][m], x[0], acc[m][n]));
            else acc[m][n] = mfma_chunk<W>(a[h][m], x[0], acc[m][n]);
          }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) red[((wave * MT + m) * NT + n) * 64 + lane] = acc[m][n];
  __syncthreads();
  // wave v finishes output tiles v, v + 4, ... (tile q: row tile q / NT, column tile q % NT)
#pragma unroll
  for (int q0 = 0; q0 < NT * MT; q0 += 4) {
    const int q = q0 + wave, m = q / NT, n = q % NT;
    f32x4 v = red[q * 64 + lane];
#pragma unroll
    for (int u = 1; u < 4; ++u) v += red[(u * MT * NT + q) * 64 + lane];
    const int rw_ = pick_n<NT>(row, n);
    if (rw_ >= 0)
      *reinterpret_cast<float4 *>(P + (size_t)rw_ * H + h0 + 16 * m + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
  }
  __syncthreads();  // `red` is free for the next item
}

// Per-lane column entries of a dense expert with position mask m: entries
// li + 16 c, c < NT, as positions (-1 past the expert's positions).
template <int NT>
__device__ __forceinline__ void dense_positions(posmask_t m, int lane, int (&pos)[NT]) {
  const int n = __popcll(m);
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const int j = 16 * c + (lane & 15);
    pos[c] = j < n ? nth_bit(m, j) : -1;
  }
}

// The same entries as positions and as rows t * K + k of P (-1 past the
// expert's positions); the rows wait on a load of the pick slots.
template <int NT>
__device__ __forceinline__ void dense_rows(const RouteBufs &r, int e, posmask_t m, int K, int lane, int (&pos)[NT],
                                           int (&row)[NT]) {
  dense_positions<NT>(m, lane, pos);
#pragma unroll
  for (int c = 0; c < NT; ++c) row[c] = pos[c] >= 0 ? pos[c] * K + pick_slot(r, e, max(pos[c], 0)) : -1;
}

// Work list: the dense experts' items (expert, 16-row tile), then the token
// groups' items (group, 16-row tile).
// (four column tiles double the dense items' operands: fewer waves per SIMD,
// so they stay in registers)
template <class W, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT > 2 ? 2 : 4))) void expert_gateup_kernel(
    const typename W::T *__restrict__ xhat, const typename W::T *__restrict__ xpk,
    const typename W::T *__restrict__ wgu, RouteBufs r, float *__restrict__ A, char *__restrict__ act, int T,
    int H, int E, int K, int I, int Imax) {
  typedef typename W::T WT;
  if (gated_off(r.gate)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ ListShared L;
  const int cnt = build_lists(r, E, L, blockIdx.x == 0);
  const int nd = cnt & 0xffff;
  const int tiles = I / 16;
  const int d_items = nd * tiles;
  const int items = d_items + (cnt >> 16) * tiles;
  const uint32_t x_bytes = (uint32_t)(T * H) * sizeof(WT);
  const size_t eb = (size_t)2 * I * H * sizeof(WT);
  __shared__ f32x4 red[4 * 2 * NT * 64];
  int item = blockIdx.x;
  for (; item < d_items; item += gridDim.x) {
    const int di = item / tiles, tile = item - di * tiles;
    const int e = uniform(L.exp[di]);
    int pos[NT];
    dense_positions<NT>(uniform64(L.msk[di]), lane, pos);
    // slot 0 holds the shared expert
    dense_gateup_item<W, 2, NT>(wgu + (size_t)e * 2 * I * H, I, xpk, T, H, pos, item, tile * 16, wave, lane,
                            act + (size_t)(1 + di) * Imax * kActSlotPerI, red);
  }
  int tile_next = 0;
  Group next;
  if (item < items) next = resolve(item - d_items, tiles, r, L, nd, K, wgu, eb, I, tile_next);
  for (; item < items; item += gridDim.x) {
    const int nitem = item + (int)gridDim.x;
    const Group g = next;
    const int tile = tile_next;
    if (nitem < items) next = resolve(nitem - d_items, tiles, r, L, nd, K, wgu, eb, I, tile_next);
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

// Work list: the shared expert's items (32 rows each), the dense experts'
// items (expert, 32 rows), then the token groups' items (group, 128 rows).
template <class W, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT > 2 ? 2 : 3))) void expert_down_kernel(const float *__restrict__ A,
                                                          const char *__restrict__ act,
                                                          const typename W::T *__restrict__ wd,
                                                          const typename W::T *__restrict__ wsd,
                                                          RouteBufs r, float *__restrict__ P, int T,
                                                          int H, int E, int K, int I, int Is, int Imax) {
  typedef typename W::T WT;
  if (gated_off(r.gate)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ ListShared L;
  const int cnt = build_lists(r, E, L, false);
  const int nd = cnt & 0xffff;
  constexpr int DR = 16 * kDenseRowTiles;   // rows per dense item
  const int tiles = H / (4 * kDownRowsPerWave), dtiles = H / DR;
  const int s_items = Is > 0 ? dtiles : 0;
  const int d_end = s_items + nd * dtiles;
  __shared__ f32x4 red[4 * kDenseRowTiles * NT * 64];
  const int items = d_end + (cnt >> 16) * tiles;
  const uint32_t a_bytes = (uint32_t)(T * K) * (uint32_t)Imax * 4u;
  const size_t eb = (size_t)H * I * sizeof(WT);
  const int stride = gridDim.x;
  int item = blockIdx.x;
  for (; item < d_end; item += stride) {
    int live[NT], row[NT];
    const WT *w;
    int ie, h0, slot;
    if (item < s_items) {
      // the shared expert (slot 0): column entry j is position j, row T*K + j
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        const int j = c * 16 + (lane & 15);
        row[c] = j < T ? T * K + j : -1;
        live[c] = row[c];
      }
      w = wsd;
      ie = Is;
      h0 = item * DR;
      slot = 0;
    } else {
      const int di = (item - s_items) / dtiles;
      const int e = uniform(L.exp[di]);
      dense_rows<NT>(r, e, uniform64(L.msk[di]), K, lane, live, row);
      w = wd + (size_t)e * H * I;
      ie = I;
      h0 = (item - s_items - di * dtiles) * DR;
      slot = 1 + di;
    }
    dense_down_item<W, kDenseRowTiles, NT>(w, ie, act + (size_t)slot * Imax * kActSlotPerI, H, live, row, h0, wave,
                                           lane, P, red);
  }
  int tile_next = 0;
  Group next;
  if (item < items) next = resolve(item - d_end, tiles, r, L, nd, K, wd, eb, I, tile_next);
  for (; item < items; item += stride) {
    const int nitem = item + stride;
    const Group g = next;
    const int tile = tile_next;
    if (nitem < items) next = resolve(nitem - d_end, tiles, r, L, nd, K, wd, eb, I, tile_next);
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
// 4-bit expert weights: every item on MFMA (see int4.hpp).  w_gate_up and
// w_down are stacks of E packed matrices ([2I][H] and [H][I]), the shared
// expert's one matrix each.
// ---------------------------------------------------------------------------

constexpr int kI4GroupDownTiles = 4;   // 16-row tiles per token-group down item (64 rows)

// Per-lane entry of token group gi: entry li (< positions) of the group, as
// (row t*K + k, position t); -1, -1 past the group.  Returns the expert.
__device__ __forceinline__ int group_entry(const RouteBufs &r, const ListShared &L, int nd, int gi, int K, int lane,
                                           int &row, int &pos) {
  const int e = uniform(L.exp[nd + gi]);
  const posmask_t m = uniform64(L.msk[nd + gi]);
  const int li = lane & 15;
  pos = li < __popcll(m) ? nth_bit(m, li) : -1;
  row = pos >= 0 ? pos * K + pick_slot(r, e, max(pos, 0)) : -1;
  return e;
}

template <int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT > 2 ? 1 : 2))) void expert_gateup_i4_kernel(
    const bf16_t *__restrict__ xpk, const char *__restrict__ wgu, RouteBufs r, float *__restrict__ A,
    char *__restrict__ act, int T, int H, int E, int K, int I, int Imax) {
  if (gated_off(r.gate)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ ListShared L;
  const int cnt = build_lists(r, E, L, blockIdx.x == 0);
  const int nd = cnt & 0xffff;
  const int tiles = I / 16;
  const int d_items = nd * tiles;
  const int items = d_items + (cnt >> 16) * tiles;
  const size_t mb = i4_mat_bytes(2 * I, H);
  __shared__ f32x4 red[4 * 2 * NT * 64];
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    if (item < d_items) {
      const int di = item / tiles, tile = item - di * tiles;
      const int e = uniform(L.exp[di]);
      int pos[NT];
      dense_positions<NT>(uniform64(L.msk[di]), lane, pos);
      const I4Mat w = i4_mat(wgu + (size_t)e * mb, 2 * I, H);
      i4_gateup_item<NT>(w, I, xpk, T, pos, tile * 16, wave, lane, act + (size_t)(1 + di) * Imax * kActSlotPerI,
                        nullptr, nullptr, Imax, red);
    } else {
      const int j = item - d_items;
      const int gi = j / tiles, tile = j - gi * tiles;
      int row[1], pos[1];
      const int e = group_entry(r, L, nd, gi, K, lane, row[0], pos[0]);
      const I4Mat w = i4_mat(wgu + (size_t)e * mb, 2 * I, H);
      i4_gateup_item<1>(w, I, xpk, T, pos, tile * 16, wave, lane, nullptr, A, row, Imax, red);
    }
  }
}

template <int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT > 2 ? 2 : 3))) void expert_down_i4_kernel(
    const float *__restrict__ A, const char *__restrict__ act, const char *__restrict__ wd,
    const char *__restrict__ wsd, RouteBufs r, float *__restrict__ P, int T, int H, int E, int K, int I, int Is,
    int Imax) {
  if (gated_off(r.gate)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ ListShared L;
  const int cnt = build_lists(r, E, L, false);
  const int nd = cnt & 0xffff;
  constexpr int DR = 16 * kDenseRowTiles;              // rows per dense item
  constexpr int GR = 16 * kI4GroupDownTiles;           // rows per token-group item
  const int dtiles = H / DR, gtiles = H / GR;
  const int s_items = Is > 0 ? dtiles : 0;
  const int d_end = s_items + nd * dtiles;
  const int items = d_end + (cnt >> 16) * gtiles;
  const uint32_t a_bytes = (uint32_t)(T * K) * (uint32_t)Imax * 4u;
  const size_t mb = i4_mat_bytes(H, I);
  static_assert(kI4GroupDownTiles * 2 >= kDenseRowTiles * 4, "`red` holds a dense item's tiles for four column tiles");
  __shared__ f32x4 red[4 * kI4GroupDownTiles * 2 * 64];
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    if (item < d_end) {
      int live[NT], prow[NT];
      I4Mat w;
      int ie, h0, slot;
      if (item < s_items) {
        // the shared expert (slot 0): column entry j is position j, row T*K + j
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const int j = c * 16 + (lane & 15);
          prow[c] = j < T ? T * K + j : -1;
          live[c] = prow[c];
        }
        w = i4_mat(wsd, H, Is);
        ie = Is;
        h0 = item * DR;
        slot = 0;
      } else {
        const int di = (item - s_items) / dtiles;
        const int e = uniform(L.exp[di]);
        dense_rows<NT>(r, e, uniform64(L.msk[di]), K, lane, live, prow);
        w = i4_mat(wd + (size_t)e * mb, H, I);
        ie = I;
        h0 = (item - s_items - di * dtiles) * DR;
        slot = 1 + di;
      }
      i4_down_item<kDenseRowTiles, NT>(w, ie, act + (size_t)slot * Imax * kActSlotPerI, nullptr, nullptr, 0, Imax, H,
                                      live, prow, h0, wave, lane, P, red);
    } else {
      const int j = item - d_end;
      const int gi = j / gtiles, tile = j - gi * gtiles;
      int row[1], pos[1];
      const int e = group_entry(r, L, nd, gi, K, lane, row[0], pos[0]);
      const I4Mat w = i4_mat(wd + (size_t)e * mb, H, I);
      i4_down_item<kI4GroupDownTiles, 1>(w, I, nullptr, A, row, a_bytes, Imax, H, row, row, tile * GR, wave, lane,
                                         P, red);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

int expert_items_max(int T, int H, int E, int K, int I, int Is, bool gateup, bool int4) {
  const int groups = expert_groups_max(T, E, K), dense = expert_dense_max(T, E, K);
  if (gateup) return (groups + dense) * (I / 16);
  const int dtiles = H / (16 * kDenseRowTiles);
  const int gtiles = int4 ? H / (16 * kI4GroupDownTiles) : H / (4 * kDownRowsPerWave);
  return (Is > 0 ? dtiles : 0) + dense * dtiles + groups * gtiles;
}

template <int NT>
static hipError_t gateup_launch(int wdtype, const void *xhat, const void *xpk, const void *w_gate_up,
                                const RouteBufs &r, float *A, void *act, int T, int H, int E, int K, int I, int Imax,
                                int grid, hipStream_t s) {
  if (wdtype == 2)
    expert_gateup_i4_kernel<NT><<<grid, 256, 0, s>>>((const bf16_t *)xpk, (const char *)w_gate_up, r, A,
                                                     (char *)act, T, H, E, K, I, Imax);
  else if (wdtype == 1)
    expert_gateup_kernel<WBf16, NT><<<grid, 256, 0, s>>>((const bf16_t *)xhat, (const bf16_t *)xpk,
                                                         (const bf16_t *)w_gate_up, r, A, (char *)act, T, H, E, K, I,
                                                         Imax);
  else
    expert_gateup_kernel<WF32, NT><<<grid, 256, 0, s>>>((const float *)xhat, (const float *)xpk,
                                                        (const float *)w_gate_up, r, A, (char *)act, T, H, E, K, I,
                                                        Imax);
  return hipGetLastError();
}

hipError_t launch_expert_gateup(int wdtype, const void *xhat, const void *xpk, const void *w_gate_up,
                                const RouteBufs &r, float *A, void *act, int T, int H, int E, int K, int I,
                                int Imax, int grid, hipStream_t s) {
  // two 16-entry column tiles cover a block of up to 32 positions, four up to 64
  return T > 32 ? gateup_launch<4>(wdtype, xhat, xpk, w_gate_up, r, A, act, T, H, E, K, I, Imax, grid, s)
                : gateup_launch<2>(wdtype, xhat, xpk, w_gate_up, r, A, act, T, H, E, K, I, Imax, grid, s);
}

template <int NT>
static hipError_t down_launch(int wdtype, const float *A, const void *act, const void *w_down, const void *ws_down,
                              const RouteBufs &r, float *P, int T, int H, int E, int K, int I, int Is, int Imax,
                              int grid, hipStream_t s) {
  if (wdtype == 2)
    expert_down_i4_kernel<NT><<<grid, 256, 0, s>>>(A, (const char *)act, (const char *)w_down, (const char *)ws_down,
                                                   r, P, T, H, E, K, I, Is, Imax);
  else if (wdtype == 1)
    expert_down_kernel<WBf16, NT><<<grid, 256, 0, s>>>(A, (const char *)act, (const bf16_t *)w_down,
                                                       (const bf16_t *)ws_down, r, P, T, H, E, K, I, Is, Imax);
  else
    expert_down_kernel<WF32, NT><<<grid, 256, 0, s>>>(A, (const char *)act, (const float *)w_down,
                                                      (const float *)ws_down, r, P, T, H, E, K, I, Is, Imax);
  return hipGetLastError();
}

hipError_t launch_expert_down(int wdtype, const float *A, const void *act, const void *w_down, const void *ws_down,
                              const RouteBufs &r, float *P, int T, int H, int E, int K, int I, int Is, int Imax,
                              int grid, hipStream_t s) {
  return T > 32 ? down_launch<4>(wdtype, A, act, w_down, ws_down, r, P, T, H, E, K, I, Is, Imax, grid, s)
                : down_launch<2>(wdtype, A, act, w_down, ws_down, r, P, T, H, E, K, I, Is, Imax, grid, s);
}

}  // namespace bdd
