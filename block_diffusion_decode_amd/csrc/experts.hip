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

// Gate/up rows of one wave: gate rows i0..i0+3 and up rows I+i0..I+i0+3 of
// expert weights wgu_e [2I][H].  xs holds the group's activations as
// [chunk][kTokGroup positions] 16-byte entries.  Writes A[asg][i] = silu(g) * u.
template <class W, int NT>
__device__ __forceinline__ void gateup_rows(const typename W::T *__restrict__ wgu_e,
                                            const uint4 *__restrict__ xs, int H, int I, int i0,
                                            int lane, const int32_t *__restrict__ asg, int ng,
                                            float *__restrict__ A) {
  constexpr int CH = W::kChunk;
  const int NC = H / CH;
  float acc[8][NT];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;

  const typename W::T *rowp[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) rowp[r] = wgu_e + (size_t)(r < 4 ? i0 + r : I + i0 + r - 4) * H;

  for (int c = lane; c < NC; c += 64) {
    uint4 wv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) wv[r] = ld16_stream(rowp[r] + (size_t)c * CH);
    float xf[NT][CH];
#pragma unroll
    for (int t = 0; t < NT; ++t) chunk_to_f32<W>(xs[c * kTokGroup + t], xf[t]);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float wf[CH];
      chunk_to_f32<W>(wv[r], wf);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < CH; ++j) acc[r][t] = fmaf(wf[j], xf[t][j], acc[r][t]);
    }
  }

  constexpr int N = 8 * NT;
  float v[N];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) v[r * NT + t] = acc[r][t];
  const float tot = reduce_scatter<N>(v, lane);
  // value index q = lane >> shift; q < N/2 are gate rows, q + N/2 the matching
  // up rows, held by lane ^ 32.
  const float up = __shfl_xor(tot, 32);
  constexpr int shift = 6 - log2i<N>();
  if ((lane & 32) == 0 && (lane & ((1 << shift) - 1)) == 0) {
    const int q = lane >> shift;
    const int r = q / NT, t = q % NT;
    if (t < ng) A[(size_t)asg[t] * I + i0 + r] = silu(tot) * up;
  }
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
  const int items = r.meta[0] * tiles;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int u = item / tiles, tile = item - u * tiles;
    const int e = r.union_list[u];
    const int n = r.slot_n[u];
    const typename W::T *wgu_e = wgu + (size_t)e * 2 * I * H;
    const int32_t *asg_all = r.slot_asg + u * kMaxT;
    for (int g0 = 0; g0 < n; g0 += kTokGroup) {
      const int ng = min(kTokGroup, n - g0);
      __syncthreads();
      for (int idx = tid; idx < kTokGroup * NC; idx += 256) {
        const int t = idx / NC, c = idx - t * NC;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (t < ng) {
          const int tok = asg_all[g0 + t] / K;
          val = ld16(xhat + (size_t)tok * H + (size_t)c * CH);
        }
        xs[c * kTokGroup + t] = val;
      }
      __syncthreads();
      const int i0 = tile * 16 + wave * 4;
      const int32_t *asg = asg_all + g0;
      if (ng <= 1)      gateup_rows<W, 1>(wgu_e, xs, H, I, i0, lane, asg, ng, A);
      else if (ng <= 2) gateup_rows<W, 2>(wgu_e, xs, H, I, i0, lane, asg, ng, A);
      else              gateup_rows<W, 4>(wgu_e, xs, H, I, i0, lane, asg, ng, A);
    }
  }
}

// Down rows of one wave: rows h0..h0+7 of expert weights wd_e [H][I], against
// the group's fp32 activations xs [chunk][kTokGroup positions][kChunk].  Writes
// P[asg][h] = w_asg * (A_asg . W_d[h]).
template <class W, int NT>
__device__ __forceinline__ void down_rows(const typename W::T *__restrict__ wd_e,
                                          const float *__restrict__ xs, int H, int I, int h0,
                                          int lane, const int32_t *__restrict__ asg,
                                          const float *__restrict__ wgt, int ng,
                                          float *__restrict__ P) {
  constexpr int CH = W::kChunk;
  const int NC = I / CH;
  float acc[8][NT];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;

  for (int c = lane; c < NC; c += 64) {
    uint4 wv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) wv[r] = ld16_stream(wd_e + (size_t)(h0 + r) * I + (size_t)c * CH);
    float xf[NT][CH];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < CH; ++j) xf[t][j] = xs[(c * kTokGroup + t) * CH + j];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float wf[CH];
      chunk_to_f32<W>(wv[r], wf);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < CH; ++j) acc[r][t] = fmaf(wf[j], xf[t][j], acc[r][t]);
    }
  }

  constexpr int N = 8 * NT;
  float v[N];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) v[r * NT + t] = acc[r][t];
  const float tot = reduce_scatter<N>(v, lane);
  constexpr int shift = 6 - log2i<N>();
  if ((lane & ((1 << shift) - 1)) == 0) {
    const int q = lane >> shift;
    const int r = q / NT, t = q % NT;
    if (t < ng) {
      const int a = asg[t];
      P[(size_t)a * H + h0 + r] = wgt[a] * tot;
    }
  }
}

template <class W>
__global__ __launch_bounds__(256) void routed_down_kernel(const float *__restrict__ A,
                                                          const typename W::T *__restrict__ wd,
                                                          RouteBufs r, float *__restrict__ P,
                                                          int H, int I) {
  extern __shared__ float xsf[];  // [I / kChunk][kTokGroup][kChunk]
  constexpr int CH = W::kChunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles = H / 32;
  const int items = r.meta[0] * tiles;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int u = item / tiles, tile = item - u * tiles;
    const int e = r.union_list[u];
    const int n = r.slot_n[u];
    const typename W::T *wd_e = wd + (size_t)e * H * I;
    const int32_t *asg_all = r.slot_asg + u * kMaxT;
    for (int g0 = 0; g0 < n; g0 += kTokGroup) {
      const int ng = min(kTokGroup, n - g0);
      __syncthreads();
      for (int idx = tid; idx < kTokGroup * I; idx += 256) {
        const int t = idx / I, k = idx - t * I;
        const int c = k / CH, j = k - c * CH;
        xsf[(c * kTokGroup + t) * CH + j] = t < ng ? A[(size_t)asg_all[g0 + t] * I + k] : 0.f;
      }
      __syncthreads();
      const int h0 = tile * 32 + wave * 8;
      const int32_t *asg = asg_all + g0;
      if (ng <= 1)      down_rows<W, 1>(wd_e, xsf, H, I, h0, lane, asg, r.wgt, ng, P);
      else if (ng <= 2) down_rows<W, 2>(wd_e, xsf, H, I, h0, lane, asg, r.wgt, ng, P);
      else              down_rows<W, 4>(wd_e, xsf, H, I, h0, lane, asg, r.wgt, ng, P);
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
  const size_t lds = (size_t)I * kTokGroup * sizeof(float);
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
