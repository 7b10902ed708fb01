// Weight-streaming helpers shared by the expert kernels and the shared
// expert's gate/up (which runs beside the selection kernel).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace bdd {

// A buffer offset past every descriptor used here: such a load returns zeros
// without a memory access.  It pads the last prefetch of a stream and masks
// positions beyond a group.
constexpr uint32_t kOutOfRange = 0x7ff00000u;

// Two-deep streaming loop: step s + 1's loads are issued before step s's
// arithmetic.  The prefetch past the last step is an out-of-range load (no
// memory access), so the loop always has the same loads in flight and the
// compiler's in-order wait counts stay exact (a conditional prefetch makes it
// drain every load).
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

// The same with an epilogue `post` after some steps: a buffer is refilled
// with step s + 2 as soon as step s's arithmetic has read it, before post(s),
// so two steps' loads stay in flight through the epilogue.
template <class Bufs, class Load, class Step, class Post>
__device__ __forceinline__ void pipeline_post(int steps, Bufs &b0, Bufs &b1, Load load, Step step, Post post) {
  load(0, b0);
  load(1, b1);
  for (int s = 0; s < steps; s += 2) {
    step(s, b0);
    load(s + 2, b0);
    post(s);
    if (s + 1 >= steps) break;
    step(s + 1, b1);
    load(s + 3, b1);
    post(s + 1);
  }
}

// ---------------------------------------------------------------------------
// Shared expert, MFMA.  Every position goes through it, so its contraction is
// dense: 16x16 tiles with 16 weight rows as A and 16 positions as B (two
// column tiles for 32 positions), in one pass over its weights.  At k-step s
// lane group g = lane >> 4 holds chunk 4s + g of its row, so a load reads 64
// contiguous bytes of each of 16 rows.
// ---------------------------------------------------------------------------

template <class W>
__device__ __forceinline__ f32x4 mfma_chunk(const uint4 &a, const uint4 &b, f32x4 c) {
  if constexpr (std::is_same<W, WBf16>::value) {
    return mfma_bf16(a, b, c);
  } else {
    c = mfma_f32(__uint_as_float(a.x), __uint_as_float(b.x), c);
    c = mfma_f32(__uint_as_float(a.y), __uint_as_float(b.y), c);
    c = mfma_f32(__uint_as_float(a.z), __uint_as_float(b.z), c);
    return mfma_f32(__uint_as_float(a.w), __uint_as_float(b.w), c);
  }
}

constexpr int kSgSteps = 4;   // k-steps per load batch of the shared gate/up
struct SgBufs {
  uint4 a[kSgSteps][2];   // [k-step][gate, up]
  uint4 b[kSgSteps][2];   // [k-step][column tile]
};

// Gate/up rows i0 .. i0 + 15 (and Is + i0 ..) of the shared expert for every
// position; the four waves split the hidden dimension and add their partial
// tiles through LDS (`red`, 16 KiB).  A[T*K + t][i] = silu(gate) * up.
template <class W>
__device__ __forceinline__ void shared_gateup_item(const typename W::T *__restrict__ wsgu,
                                                   const typename W::T *__restrict__ xhat, int T, int H, int Is,
                                                   int TK, int Imax, int i0, int wave, int lane,
                                                   float *__restrict__ A, f32x4 *red) {
  typedef typename W::T WT;
  constexpr int CH = W::kChunk;
  const int li = lane & 15, g = lane >> 4;
  const int ncw = H / CH / 4;               // chunks of this wave's quarter of H
  const int cw0 = wave * ncw;
  const int ksteps = (ncw + 3) / 4;
  const rsrc_t rw = make_rsrc(wsgu, (uint32_t)(2 * Is * H) * sizeof(WT));
  const rsrc_t rx = make_rsrc(xhat, (uint32_t)(T * H) * sizeof(WT));
  const uint32_t rowg = (uint32_t)((i0 + li) * H) * sizeof(WT);
  const uint32_t rowu = (uint32_t)((Is + i0 + li) * H) * sizeof(WT);
  uint32_t rowx[2];
#pragma unroll
  for (int n = 0; n < 2; ++n)
    rowx[n] = n * 16 + li < T ? (uint32_t)((n * 16 + li) * H) * sizeof(WT) : kOutOfRange;
  f32x4 acc[2][2];   // [gate, up][column tile]
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[q][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load = [&](int bt, SgBufs &b) {
#pragma unroll
    for (int j = 0; j < kSgSteps; ++j) {
      const int ks = kSgSteps * bt + j;
      const int c = 4 * ks + g;
      const bool live = ks < ksteps && c < ncw;
      const uint32_t co = (uint32_t)((cw0 + c) * CH) * sizeof(WT);
      b.a[j][0] = buf_ld16(rw, live ? rowg + co : kOutOfRange, 0);
      b.a[j][1] = buf_ld16(rw, live ? rowu + co : kOutOfRange, 0);
#pragma unroll
      for (int n = 0; n < 2; ++n) b.b[j][n] = buf_ld16(rx, live ? rowx[n] + co : kOutOfRange, 0);
    }
  };
  auto step = [&](int, const SgBufs &b) {
#pragma unroll
    for (int j = 0; j < kSgSteps; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int n = 0; n < 2; ++n) acc[q][n] = mfma_chunk<W>(b.a[j][q], b.b[j][n], acc[q][n]);
  };
  SgBufs b0, b1;
  pipeline((ksteps + kSgSteps - 1) / kSgSteps, b0, b1, load, step);
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int n = 0; n < 2; ++n) red[((wave * 2 + q) * 2 + n) * 64 + lane] = acc[q][n];
  __syncthreads();
  if (wave < 2) {
    // wave n finishes column tile n: rows i0 + 4g + r, position 16n + li
    const int n = wave;
    f32x4 gt = red[n * 64 + lane], up = red[(2 + n) * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 a = red[((w * 2 + 0) * 2 + n) * 64 + lane], b = red[((w * 2 + 1) * 2 + n) * 64 + lane];
      gt += a;
      up += b;
    }
    const int t = n * 16 + li;
    if (t < T) {
      float4 o;
      o.x = silu(gt[0]) * up[0]; o.y = silu(gt[1]) * up[1];
      o.z = silu(gt[2]) * up[2]; o.w = silu(gt[3]) * up[3];
      *reinterpret_cast<float4 *>(A + (size_t)(TK + t) * Imax + i0 + 4 * g) = o;
    }
  }
  __syncthreads();  // `red` is free for the next item
}

}  // namespace bdd
