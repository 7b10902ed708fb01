// Expert FFNs of one MoE layer: routed experts grouped by expert (each union
// expert's weights stream from HBM once per block, for every position routed
// to it) and the dense shared expert.
//
// Pages: [P1] aitujian.cn article on Clover-35B-A3B-Preview, section 五 (the 32
// positions of a block reach a union of experts far larger than 8; the bytes
// read grow much less than the tokens produced because the same weights serve
// many positions) and section 四 (one shared expert per layer).  The expert
// activation (SwiGLU) is not on the pages; it is the reading this library
// documents in its header.
#include <type_traits>

#include "dense.hpp"
#include "kernels.hpp"

namespace bdd {

// ---------------------------------------------------------------------------
// Routed experts, VALU.  A routed expert sees ~1.6 positions on average at the
// Clover shape (at most 32), so its contraction is a matrix-vector product:
// fp32 FMAs on weights streamed with 16-byte loads, positions' activations
// staged in LDS.  A wave owns 8 weight rows; lane l covers 16-byte chunks
// l, l+64, ... of every row, so a load instruction reads one contiguous
// 1 KiB segment of a row.  Per-lane partial dot products are summed across
// the wave by a halving exchange at the end of the item.
// ---------------------------------------------------------------------------

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

// Streams the rows of one wave in batches of 8 through a buffer descriptor.
// Step s covers batch b = s / nq and chunk q = s % nq: the 16-byte chunk
// c = lane + 64 q of each of the batch's 8 rows (lanes past the row end read
// the last chunk, and the activation chunk they see is zero).  The next
// step's 8 loads are issued before the current step's arithmetic (two
// buffers), and the first step's loads before `ready()` (the caller's LDS
// staging and barrier), so weight latency overlaps staging, arithmetic and
// the per-batch epilogue.
//   rowoff(b, r): wave-uniform byte offset of row r of batch b in `rs`
//   fma(c, w[8], acc): accumulates chunk c of the 8 rows into acc[8][NT]
//   batch_end(b, acc): consumes a finished batch (acc is then cleared)
template <class W, int NT, class RowOff, class Ready, class Fma, class BatchEnd>
__device__ __forceinline__ void stream_rows(rsrc_t rs, int nb, int nq, int NC, int lane,
                                            RowOff rowoff, Ready ready, Fma fma,
                                            BatchEnd batch_end) {
  float acc[8][NT];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;
  const int steps = nb * nq;
  uint4 w0[8], w1[8];
  auto load = [&](int s, uint4(&w)[8]) {
    const int b = s / nq;
    const uint32_t voff = (uint32_t)min(lane + 64 * (s - b * nq), NC - 1) * 16u;
#pragma unroll
    for (int r = 0; r < 8; ++r) w[r] = buf_ld16(rs, voff, rowoff(b, r));
  };
  auto step = [&](int s, const uint4(&w)[8]) {
    const int b = s / nq, q = s - b * nq;
    fma(lane + 64 * q, w, acc);
    if (q == nq - 1) {
      batch_end(b, acc);
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;
    }
  };
  if (steps > 0) load(0, w0);
  ready();
  for (int s = 0; s < steps; s += 2) {
    if (s + 1 < steps) load(s + 1, w1);
    step(s, w0);
    if (s + 1 >= steps) break;
    if (s + 2 < steps) load(s + 2, w0);
    step(s + 1, w1);
  }
}

// Sums acc[8][NT] over the wave; returns the lane's total and its value index
// q = r * NT + t (see reduce_scatter).
template <int NT>
__device__ __forceinline__ float wave_reduce_rows(float (&acc)[8][NT], int lane) {
  constexpr int N = 8 * NT;
  float v[N];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) v[r * NT + t] = acc[r][t];
  return reduce_scatter<N>(v, lane);
}

// Gate/up of one work item (expert e, tile j): wave w owns gate rows
// j*16 + 4w + r and the matching up rows I + j*16 + 4w + r (r = 0..3), read in
// full; xs holds the token group's activations as [chunk][kTokGroup] 16-byte
// entries.  A[asg][i] = silu(gate) * up.
template <class W, int NT, class Ready>
__device__ __forceinline__ void gateup_item(const typename W::T *__restrict__ wgu_e, const uint4 *xs,
                                            int H, int I, int i0, int lane,
                                            const int32_t *__restrict__ asg, int ng,
                                            float *__restrict__ A, Ready ready) {
  constexpr int CH = W::kChunk;
  const int NC = H / CH;
  const int nq = (NC + 63) / 64;
  const rsrc_t rs = make_rsrc(wgu_e, (uint32_t)(2 * I * H * sizeof(typename W::T)));
  auto rowoff = [&](int, int r) {
    return (uint32_t)((r < 4 ? i0 + r : I + i0 + r - 4) * H * (int)sizeof(typename W::T));
  };
  auto fma = [&](int c, const uint4(&w)[8], float(&acc)[8][NT]) {
    uint4 xv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) xv[t] = c < NC ? xs[c * kTokGroup + t] : make_uint4(0, 0, 0, 0);
    if constexpr (std::is_same<W, WBf16>::value) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float a = acc[r][t];
          a = dot2bf(w[r].x, xv[t].x, a);
          a = dot2bf(w[r].y, xv[t].y, a);
          a = dot2bf(w[r].z, xv[t].z, a);
          a = dot2bf(w[r].w, xv[t].w, a);
          acc[r][t] = a;
        }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float wf[4];
        chunk_to_f32<W>(w[r], wf);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float xf[4];
          chunk_to_f32<W>(xv[t], xf);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[r][t] = fmaf(wf[j], xf[j], acc[r][t]);
        }
      }
    }
  };
  auto batch_end = [&](int, float(&acc)[8][NT]) {
    const float tot = wave_reduce_rows<NT>(acc, lane);
    // q < 4*NT: gate rows; lane ^ 32 holds the matching up row (q + 4*NT)
    const float up = __shfl_xor(tot, 32);
    constexpr int shift = 6 - log2i<8 * NT>();
    if ((lane & 32) == 0 && (lane & ((1 << shift) - 1)) == 0) {
      const int q = lane >> shift;
      const int r = q / NT, t = q % NT;
      if (t < ng) A[(size_t)asg[t] * I + i0 + r] = silu(tot) * up;
    }
  };
  stream_rows<W, NT>(rs, 1, nq, NC, lane, rowoff, ready, fma, batch_end);
}

template <class W>
__global__ __launch_bounds__(256) void routed_gateup_kernel(const typename W::T *__restrict__ xhat,
                                                            const typename W::T *__restrict__ wgu,
                                                            RouteBufs r, float *__restrict__ A,
                                                            int H, int K, int I) {
  extern __shared__ uint4 xs[];  // [H / kChunk][kTokGroup]
  constexpr int CH = W::kChunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NC = H / CH;
  const int tiles = I / 16;
  const int items = uniform(r.meta[0]) * tiles;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int u = item / tiles, tile = item - u * tiles;
    const int e = uniform(r.union_list[u]);
    const int n = uniform(r.slot_n[u]);
    const typename W::T *wgu_e = wgu + (size_t)e * 2 * I * H;
    const int32_t *asg_all = r.slot_asg + u * kMaxT;
    const int i0 = uniform(tile * 16 + wave * 4);
    for (int g0 = 0; g0 < n; g0 += kTokGroup) {
      const int ng = min(kTokGroup, n - g0);
      auto ready = [&]() {
        // position rows of the group (wave-uniform scalar loads), then the
        // group's chunk loads, independent of each other
        const typename W::T *xrow[kTokGroup];
#pragma unroll
        for (int t = 0; t < kTokGroup; ++t)
          xrow[t] = t < ng ? xhat + (size_t)(asg_all[g0 + t] / K) * H : nullptr;
        __syncthreads();  // previous group's readers are done with xs
        for (int c = tid; c < NC; c += 256) {
          uint4 val[kTokGroup];
#pragma unroll
          for (int t = 0; t < kTokGroup; ++t)
            val[t] = xrow[t] ? ld16(xrow[t] + (size_t)c * CH) : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int t = 0; t < kTokGroup; ++t) xs[c * kTokGroup + t] = val[t];
        }
        __syncthreads();
      };
      const int32_t *asg = asg_all + g0;
      if (ng <= 1)      gateup_item<W, 1>(wgu_e, xs, H, I, i0, lane, asg, ng, A, ready);
      else if (ng <= 2) gateup_item<W, 2>(wgu_e, xs, H, I, i0, lane, asg, ng, A, ready);
      else              gateup_item<W, 4>(wgu_e, xs, H, I, i0, lane, asg, ng, A, ready);
    }
  }
}

constexpr int kDownRowsPerWave = 32;  // four batches of 8 rows (128 rows per item)

// Down projection of one work item (expert e, 128 output rows): wave w owns
// rows h0 + 8b + r (b = 0..3, r = 0..7) of W_d[e] [H][I]; xs holds the token
// group's fp32 activations as [chunk][kTokGroup][kChunk].
// P[asg][h] = w_asg * (A_asg . W_d[h]).
template <class W, int NT, class Ready>
__device__ __forceinline__ void down_item(const typename W::T *__restrict__ wd_e, const void *xs,
                                          int H, int I, int h0, int lane,
                                          const int32_t *__restrict__ asg,
                                          const float *__restrict__ wgt, int ng,
                                          float *__restrict__ P, Ready ready) {
  constexpr int CH = W::kChunk;
  const int NC = I / CH;
  const int nq = (NC + 63) / 64;
  const int nb = kDownRowsPerWave / 8;
  const rsrc_t rs = make_rsrc(wd_e, (uint32_t)(H * I * sizeof(typename W::T)));
  auto rowoff = [&](int b, int r) { return (uint32_t)((h0 + 8 * b + r) * I * (int)sizeof(typename W::T)); };
  auto fma = [&](int c, const uint4(&w)[8], float(&acc)[8][NT]) {
    if constexpr (std::is_same<W, WBf16>::value) {
      // activations as bf16 (high, residual) pairs: two dot2 passes
      const uint4 *xp = static_cast<const uint4 *>(xs);
      uint4 xh[NT], xl[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        xh[t] = c < NC ? xp[(c * kTokGroup + t) * 2] : make_uint4(0, 0, 0, 0);
        xl[t] = c < NC ? xp[(c * kTokGroup + t) * 2 + 1] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float a = acc[r][t];
          a = dot2bf(w[r].x, xh[t].x, a);
          a = dot2bf(w[r].y, xh[t].y, a);
          a = dot2bf(w[r].z, xh[t].z, a);
          a = dot2bf(w[r].w, xh[t].w, a);
          a = dot2bf(w[r].x, xl[t].x, a);
          a = dot2bf(w[r].y, xl[t].y, a);
          a = dot2bf(w[r].z, xl[t].z, a);
          a = dot2bf(w[r].w, xl[t].w, a);
          acc[r][t] = a;
        }
    } else {
      const float *xp = static_cast<const float *>(xs);
      float xf[NT][CH];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < CH; ++j) xf[t][j] = c < NC ? xp[(c * kTokGroup + t) * CH + j] : 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float wf[CH];
        chunk_to_f32<W>(w[r], wf);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int j = 0; j < CH; ++j) acc[r][t] = fmaf(wf[j], xf[t][j], acc[r][t]);
      }
    }
  };
  auto batch_end = [&](int b, float(&acc)[8][NT]) {
    const float tot = wave_reduce_rows<NT>(acc, lane);
    constexpr int shift = 6 - log2i<8 * NT>();
    if ((lane & ((1 << shift) - 1)) == 0) {
      const int q = lane >> shift;
      const int r = q / NT, t = q % NT;
      if (t < ng) {
        const int a = asg[t];
        P[(size_t)a * H + h0 + 8 * b + r] = wgt[a] * tot;
      }
    }
  };
  stream_rows<W, NT>(rs, nb, nq, NC, lane, rowoff, ready, fma, batch_end);
}

template <class W>
__global__ __launch_bounds__(256) void routed_down_kernel(const float *__restrict__ A,
                                                          const typename W::T *__restrict__ wd,
                                                          RouteBufs r, float *__restrict__ P,
                                                          int H, int I) {
  // bf16 weights: [I / 8][kTokGroup][high, residual] bf16x8 pairs;
  // fp32 weights: [I / 4][kTokGroup][4] floats.  16 * I bytes either way.
  extern __shared__ uint4 xsm[];
  constexpr int CH = W::kChunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rows_per_item = 4 * kDownRowsPerWave;
  const int tiles = H / rows_per_item;
  const int items = uniform(r.meta[0]) * tiles;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int u = item / tiles, tile = item - u * tiles;
    const int e = uniform(r.union_list[u]);
    const int n = uniform(r.slot_n[u]);
    const typename W::T *wd_e = wd + (size_t)e * H * I;
    const int32_t *asg_all = r.slot_asg + u * kMaxT;
    const int h0 = uniform(tile * rows_per_item + wave * kDownRowsPerWave);
    for (int g0 = 0; g0 < n; g0 += kTokGroup) {
      const int ng = min(kTokGroup, n - g0);
      auto ready = [&]() {
        // activation rows of the group (wave-uniform scalar loads of the
        // assignment ids); one 16-byte weight chunk's worth per thread and row
        const float *arow[kTokGroup];
#pragma unroll
        for (int t = 0; t < kTokGroup; ++t) arow[t] = t < ng ? A + (size_t)asg_all[g0 + t] * I : nullptr;
        __syncthreads();  // previous group's readers are done with xs
        for (int c = tid; c < I / CH; c += 256) {
          if constexpr (std::is_same<W, WBf16>::value) {
            uint4 *xp = reinterpret_cast<uint4 *>(xsm);
#pragma unroll
            for (int t = 0; t < kTokGroup; ++t) {
              float x[8];
              if (arow[t]) {
                const float4 u = reinterpret_cast<const float4 *>(arow[t] + c * 8)[0];
                const float4 v = reinterpret_cast<const float4 *>(arow[t] + c * 8)[1];
                x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
                x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
              } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = 0.f;
              }
              uint4 hi, lo;
              split_hi_lo(x, hi, lo);
              xp[(c * kTokGroup + t) * 2] = hi;
              xp[(c * kTokGroup + t) * 2 + 1] = lo;
            }
          } else {
            float *xf = reinterpret_cast<float *>(xsm);
#pragma unroll
            for (int t = 0; t < kTokGroup; ++t) {
              const float4 u = arow[t] ? *reinterpret_cast<const float4 *>(arow[t] + c * 4)
                                       : make_float4(0, 0, 0, 0);
              xf[(c * kTokGroup + t) * 4 + 0] = u.x;
              xf[(c * kTokGroup + t) * 4 + 1] = u.y;
              xf[(c * kTokGroup + t) * 4 + 2] = u.z;
              xf[(c * kTokGroup + t) * 4 + 3] = u.w;
            }
          }
        }
        __syncthreads();
      };
      const int32_t *asg = asg_all + g0;
      if (ng <= 1)      down_item<W, 1>(wd_e, xsm, H, I, h0, lane, asg, r.wgt, ng, P, ready);
      else if (ng <= 2) down_item<W, 2>(wd_e, xsm, H, I, h0, lane, asg, r.wgt, ng, P, ready);
      else              down_item<W, 4>(wd_e, xsm, H, I, h0, lane, asg, r.wgt, ng, P, ready);
    }
  }
}

// ---------------------------------------------------------------------------
// Shared expert, MFMA: every position goes through the same weights, a dense
// (16 rows) x (up to 32 positions) contraction per tile.
// ---------------------------------------------------------------------------

// One workgroup per 16 intermediate units: gate rows and the matching up rows;
// its 8 waves split the hidden dimension.  A_s[t][i] = silu(g) * u.
template <class W, int NT>
__global__ __launch_bounds__(512) void shared_gateup_kernel(const typename W::T *__restrict__ xhat,
                                                            const typename W::T *__restrict__ wsgu,
                                                            float *__restrict__ A_s, int T, int H,
                                                            int I_s) {
  __shared__ float red[8 * 2 * NT * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int i_row = blockIdx.x * 16 + (lane & 15);
  int k0, k1;
  k_slice(H, mfma_kstep<W>(), wave, nw, k0, k1);
  f32x4 ag[NT], au[NT], acc[2 * NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) ag[n] = au[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  dense_acc_global<W, typename W::T, NT>(wsgu + (size_t)i_row * H, true, xhat, H, T, k0, k1, lane, ag);
  dense_acc_global<W, typename W::T, NT>(wsgu + (size_t)(I_s + i_row) * H, true, xhat, H, T, k0, k1,
                                         lane, au);
#pragma unroll
  for (int n = 0; n < NT; ++n) { acc[n] = ag[n]; acc[NT + n] = au[n]; }
  splitk_sum<2 * NT>(acc, red, wave, nw, lane);
  if (wave == 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = blockIdx.x * 16 + 4 * (lane >> 4) + r;
        const int t = n * 16 + (lane & 15);
        if (t < T) A_s[(size_t)t * I_s + i] = silu(acc[n][r]) * acc[NT + n][r];
      }
  }
}

// One workgroup per 16 hidden rows of W_sd [H][I_s]; 4 waves split I_s.
template <class W, int NT>
__global__ __launch_bounds__(256) void shared_down_kernel(const float *__restrict__ A_s,
                                                          const typename W::T *__restrict__ wsd,
                                                          float *__restrict__ P_s, int T, int H,
                                                          int I_s) {
  __shared__ float red[4 * NT * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int row = blockIdx.x * 16 + (lane & 15);
  int k0, k1;
  k_slice(I_s, mfma_kstep<W>(), wave, nw, k0, k1);
  f32x4 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  dense_acc_global<W, float, NT>(wsd + (size_t)row * I_s, true, A_s, I_s, T, k0, k1, lane, acc);
  splitk_sum<NT>(acc, red, wave, nw, lane);
  if (wave == 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hrow = blockIdx.x * 16 + 4 * (lane >> 4) + r;
        const int t = n * 16 + (lane & 15);
        if (t < T) P_s[(size_t)t * H + hrow] = acc[n][r];
      }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <typename F>
static hipError_t allow_lds(F *fn, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_routed_gateup(int wdtype, const void *xhat, const void *w_gate_up,
                                const RouteBufs &r, float *A, int T, int H, int E, int K, int I,
                                int grid, hipStream_t s) {
  (void)T; (void)E;
  const size_t lds = (size_t)H / (wdtype == 1 ? 8 : 4) * kTokGroup * 16;
  hipError_t err;
  if (wdtype == 1) {
    if ((err = allow_lds(routed_gateup_kernel<WBf16>, lds)) != hipSuccess) return err;
    routed_gateup_kernel<WBf16><<<grid, 256, lds, s>>>((const bf16_t *)xhat,
                                                       (const bf16_t *)w_gate_up, r, A, H, K, I);
  } else {
    if ((err = allow_lds(routed_gateup_kernel<WF32>, lds)) != hipSuccess) return err;
    routed_gateup_kernel<WF32><<<grid, 256, lds, s>>>((const float *)xhat, (const float *)w_gate_up,
                                                      r, A, H, K, I);
  }
  return hipGetLastError();
}

hipError_t launch_routed_down(int wdtype, const float *A, const void *w_down, const RouteBufs &r,
                              float *P, int H, int E, int K, int I, int grid, hipStream_t s) {
  (void)E; (void)K;
  const size_t lds = (size_t)I * 16;
  hipError_t err;
  if (wdtype == 1) {
    if ((err = allow_lds(routed_down_kernel<WBf16>, lds)) != hipSuccess) return err;
    routed_down_kernel<WBf16><<<grid, 256, lds, s>>>(A, (const bf16_t *)w_down, r, P, H, I);
  } else {
    if ((err = allow_lds(routed_down_kernel<WF32>, lds)) != hipSuccess) return err;
    routed_down_kernel<WF32><<<grid, 256, lds, s>>>(A, (const float *)w_down, r, P, H, I);
  }
  return hipGetLastError();
}

hipError_t launch_shared_gateup(int wdtype, const void *xhat, const void *ws_gate_up, float *A_s,
                                int T, int H, int I_s, hipStream_t s) {
  const int grid = I_s / 16;
  if (wdtype == 1) {
    if (T <= 16)
      shared_gateup_kernel<WBf16, 1><<<grid, 512, 0, s>>>((const bf16_t *)xhat,
                                                           (const bf16_t *)ws_gate_up, A_s, T, H, I_s);
    else
      shared_gateup_kernel<WBf16, 2><<<grid, 512, 0, s>>>((const bf16_t *)xhat,
                                                           (const bf16_t *)ws_gate_up, A_s, T, H, I_s);
  } else {
    if (T <= 16)
      shared_gateup_kernel<WF32, 1><<<grid, 512, 0, s>>>((const float *)xhat,
                                                          (const float *)ws_gate_up, A_s, T, H, I_s);
    else
      shared_gateup_kernel<WF32, 2><<<grid, 512, 0, s>>>((const float *)xhat,
                                                          (const float *)ws_gate_up, A_s, T, H, I_s);
  }
  return hipGetLastError();
}

hipError_t launch_shared_down(int wdtype, const float *A_s, const void *ws_down, float *P_s, int T,
                              int H, int I_s, hipStream_t s) {
  const int grid = H / 16;
  if (wdtype == 1) {
    if (T <= 16)
      shared_down_kernel<WBf16, 1><<<grid, 256, 0, s>>>(A_s, (const bf16_t *)ws_down, P_s, T, H, I_s);
    else
      shared_down_kernel<WBf16, 2><<<grid, 256, 0, s>>>(A_s, (const bf16_t *)ws_down, P_s, T, H, I_s);
  } else {
    if (T <= 16)
      shared_down_kernel<WF32, 1><<<grid, 256, 0, s>>>(A_s, (const float *)ws_down, P_s, T, H, I_s);
    else
      shared_down_kernel<WF32, 2><<<grid, 256, 0, s>>>(A_s, (const float *)ws_down, P_s, T, H, I_s);
  }
  return hipGetLastError();
}

}  // namespace bdd
