// MFMA accumulation of a 16-row weight tile against the block's positions.
//
// Used where the contraction is dense over the block: the router (every
// position against every expert's router row) and the shared expert (every
// position through the same weights).  Weight rows stream from HBM once; the
// block's activations (at most 32 rows) are read from L2.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace bdd {

// acc[n] += W[row] . X[col]^T over k in [k0, k1) for the lane's MFMA slots.
// wrow points at this lane's weight row (row0 + (lane & 15)); row_ok marks
// rows inside the matrix.  X is [T][ldx] of XT (bf16 or fp32) in global
// memory; columns are positions n*16 + (lane & 15), zero beyond T.
// bf16 weights take k-steps of 32 (v_mfma_f32_16x16x32_bf16): lane group
// g = lane >> 4 covers [k + 8g, k + 8g + 8), i.e. 64 contiguous bytes per row
// per load instruction.  fp32 activations against bf16 weights are split into
// a bf16 high part and a bf16 residual (two MFMA passes).  fp32 weights take
// k-steps of 16 as four v_mfma_f32_16x16x4_f32 over a float4 per lane.
template <class W, typename XT, int NT>
__device__ __forceinline__ void dense_acc_global(const typename W::T *__restrict__ wrow, bool row_ok,
                                                 const XT *__restrict__ X, int ldx, int T, int k0,
                                                 int k1, int lane, f32x4 (&acc)[NT]) {
  const int i = lane & 15, g = lane >> 4;
  if constexpr (std::is_same<W, WBf16>::value) {
#pragma unroll 4
    for (int k = k0; k < k1; k += 32) {
      const int kc = k + 8 * g;
      const uint4 a = row_ok ? ld16_stream(wrow + kc) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int t = n * 16 + i;
        if constexpr (std::is_same<XT, bf16_t>::value) {
          const uint4 b = (t < T) ? ld16(X + (size_t)t * ldx + kc) : make_uint4(0, 0, 0, 0);
          acc[n] = mfma_bf16(a, b, acc[n]);
        } else {
          float x[8];
          if (t < T) {
            const float4 u = *reinterpret_cast<const float4 *>(X + (size_t)t * ldx + kc);
            const float4 v = *reinterpret_cast<const float4 *>(X + (size_t)t * ldx + kc + 4);
            x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
            x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = 0.f;
          }
          uint4 hi, lo;
          split_hi_lo(x, hi, lo);
          acc[n] = mfma_bf16(a, hi, acc[n]);
          acc[n] = mfma_bf16(a, lo, acc[n]);
        }
      }
    }
  } else {
    static_assert(std::is_same<XT, float>::value, "fp32 weights take fp32 activations");
#pragma unroll 4
    for (int k = k0; k < k1; k += 16) {
      const int kc = k + 4 * g;
      const float4 a = row_ok ? *reinterpret_cast<const float4 *>(wrow + kc) : make_float4(0, 0, 0, 0);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int t = n * 16 + i;
        const float4 b = (t < T) ? *reinterpret_cast<const float4 *>(X + (size_t)t * ldx + kc)
                                 : make_float4(0, 0, 0, 0);
        acc[n] = mfma_f32(a.x, b.x, acc[n]);
        acc[n] = mfma_f32(a.y, b.y, acc[n]);
        acc[n] = mfma_f32(a.z, b.z, acc[n]);
        acc[n] = mfma_f32(a.w, b.w, acc[n]);
      }
    }
  }
}

// k-step of the MFMA path for a weight type.
template <class W>
constexpr int mfma_kstep() { return std::is_same<W, WBf16>::value ? 32 : 16; }

// The k-range [k0, k1) of slice `part` when K is split into `parts` slices
// on k-step boundaries.
__device__ __forceinline__ void k_slice(int K, int kstep, int part, int parts, int &k0, int &k1) {
  const int steps = K / kstep;
  const int per = (steps + parts - 1) / parts;
  k0 = min(part * per, steps) * kstep;
  k1 = min((part + 1) * per, steps) * kstep;
}

// Sum acc over the waves of a workgroup through LDS (nw * NT * 256 floats);
// the total is valid in wave 0.  Ends with a barrier, so lds may be reused.
template <int NT>
__device__ __forceinline__ void splitk_sum(f32x4 (&acc)[NT], float *lds, int wave, int nw, int lane) {
  if (wave > 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) lds[((wave * NT + n) * 4 + r) * 64 + lane] = acc[n][r];
  }
  __syncthreads();
  if (wave == 0) {
    for (int w = 1; w < nw; ++w)
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[n][r] += lds[((w * NT + n) * 4 + r) * 64 + lane];
  }
  __syncthreads();
}

}  // namespace bdd
