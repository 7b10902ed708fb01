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
// drain every load).  The loop body runs whole pairs of steps and an odd
// last step follows the loop: an exit between the two steps of a pair would
// join the loop's wait counts with the exit path's, and the compiler would
// then wait at the first step for the second buffer's loads as well.
template <class Bufs, class Load, class Step>
__device__ __forceinline__ void pipeline(int steps, Bufs &b0, Bufs &b1, Load load, Step step) {
  load(0, b0);
  int s = 0;
  for (; s + 1 < steps; s += 2) {
    load(s + 1, b1);
    step(s, b0);
    load(s + 2, b0);
    step(s + 1, b1);
  }
  if (s < steps) {
    load(s + 1, b1);
    step(s, b0);
  }
}

// The same with an epilogue `post` after some steps: a buffer is refilled
// with step s + 2 as soon as step s's arithmetic has read it, before post(s),
// so two steps' loads stay in flight through the epilogue.
template <class Bufs, class Load, class Step, class Post>
__device__ __forceinline__ void pipeline_post(int steps, Bufs &b0, Bufs &b1, Load load, Step step, Post post) {
  load(0, b0);
  load(1, b1);
  int s = 0;
  for (; s + 1 < steps; s += 2) {   // (whole pairs, as above)
    step(s, b0);
    load(s + 2, b0);
    post(s);
    step(s + 1, b1);
    load(s + 3, b1);
    post(s + 1);
  }
  if (s < steps) {
    step(s, b0);
    load(s + 2, b0);
    post(s);
  }
}

// ---------------------------------------------------------------------------
// Dense experts, MFMA.  Every position goes through the shared expert, and a
// routed expert picked by more than kTokGroup positions (common under skewed
// routing) sees many of them, so their contraction is dense: 16x16 tiles with
// 16 weight rows as A and 16 positions as B (two column tiles for 32
// positions), in one pass over the weights.  At k-step s lane group
// g = lane >> 4 holds chunk 4s + g of its row (the MFMA operand layout), so a
// load straight into operand order reads only 64 contiguous bytes of each of
// 16 rows.  The weights are therefore loaded as whole 128-byte lines of 8 rows
// and passed through LDS into operand order (stage_slot); the block's packed
// copy (xpack_unit) and the packed activations are already in operand order.
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

// Packed normalised block (the dense items' B operand): chunk C (kChunk
// elements) of position t sits at 16-byte unit (C / 4 * T + t) * 4 + C % 4,
// so the 16 positions x 4 chunks of one MFMA k-step are one contiguous KiB.
__device__ __forceinline__ uint32_t xpack_unit(int C, int t, int T) {
  return (uint32_t)(((C >> 2) * T + t) * 4 + (C & 3));
}

// Packed activations of one dense expert (a slot of Imax * 128 bytes): per
// k-step of 4 chunks, `planes` planes of kMaxT entries x 4 chunks of 16 B.
// bf16 weights take two planes, the bf16 high parts and the bf16 residuals
// of the fp32 activations; fp32 weights take one plane of fp32 values.
template <class W>
constexpr int act_planes() { return std::is_same<W, WBf16>::value ? 2 : 1; }
__device__ __forceinline__ uint32_t act_unit(int C, int plane, int e, int planes) {
  return (uint32_t)((((C >> 2) * planes + plane) * kMaxT + e) * 4 + (C & 3));
}

constexpr int kSgSteps = 4;   // k-steps per load batch of the shared gate/up beside selection
template <int STEPS, int NT>
struct DgBufs {
  uint4 a[STEPS / 2][4];   // [unit of 2 k-steps][gate rows 0-7, 8-15, up rows 0-7, 8-15]
  uint4 b[STEPS][NT];      // [k-step][column tile]
};

// v[n] for a compile-time n range and a runtime n, by value arithmetic (a
// runtime index into a register array would leave it in memory, which the
// compiler places in LDS addressed through the dispatch packet: a slow first
// load in every workgroup).
template <int NT>
__device__ __forceinline__ int pick_n(const int (&v)[NT], int n) {
  int r = v[0];
#pragma unroll
  for (int j = 1; j < NT; ++j) r = n == j ? v[j] : r;
  return r;
}

// Weight staging of the dense gate/up item.  A unit is 2 k-steps (8 chunks of
// 16 bytes, 128 bytes of a row): one load instruction reads 8 rows of it
// (lane l: row 8j + l / 8, chunk l % 8), 8 full 128-byte lines, and the wave
// writes the unit to its own 4 KiB of LDS and reads it back in operand order.
// Chunk c of row r sits at slot c ^ stage_swz(r): the 8 lanes of one row in a
// write, and the 16 rows of one chunk in a read (16 lanes at a time), fall on
// distinct 16-byte bank groups.
__device__ __forceinline__ int stage_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int stage_slot(int q, int r, int c) { return (q * 16 + r) * 8 + (c ^ stage_swz(r)); }

// Gate/up rows i0 .. i0 + 15 (and ie + i0 ..) of one expert, W_gu [2 ie][H],
// for up to 16 NT column entries (NT tiles of 16).  Lane (li, g) names entries
// li + 16 n by their positions pos[n] (-1: no entry).  The four waves split
// the hidden dimension, each starting its units `rot` units in (so concurrent
// items spread their reads of the packed block); each wave stages its
// weights through 4 KiB of its own span of `red` (4 * 2 * NT * 64 f32x4)
// and afterwards adds its partial tiles through all of it; wave n < NT finishes
// column tile n and stores silu(gate) * up into the packed activation slot.
template <class W, int STEPS, int NT>
__device__ __forceinline__ void dense_gateup_item(const typename W::T *__restrict__ w, int ie,
                                                  const typename W::T *__restrict__ xpk, int T, int H,
                                                  const int (&pos)[NT], int rot, int i0, int wave, int lane,
                                                  char *__restrict__ act, f32x4 *red) {
  typedef typename W::T WT;
  constexpr int CH = W::kChunk;
  const int li = lane & 15, g = lane >> 4;
  const int ncw = H / CH / 4;               // chunks of this wave's quarter of H
  const int cw0 = wave * ncw;
  static_assert(STEPS % 2 == 0, "the dense gate/up item streams whole units of 2 k-steps");
  constexpr int UB = STEPS / 2;             // units per load batch
  const int nunits = (ncw + 7) / 8;
  rot %= nunits;
  const rsrc_t rw = make_rsrc(w, (uint32_t)(2 * ie * H) * sizeof(WT));
  const rsrc_t rx = make_rsrc(xpk, (uint32_t)(T * H) * sizeof(WT));
  // this lane's row in a staging load, and its chunk in the unit
  const int sr = lane >> 3, sc = lane & 7;
  const uint32_t rowg = (uint32_t)((i0 + sr) * H) * sizeof(WT);
  // wave-uniform offsets of gate rows 8-15 and of the up rows (scalar offsets;
  // an out-of-range vector offset still returns zeros)
  const uint32_t rows8 = (uint32_t)(8 * H) * sizeof(WT), upo = (uint32_t)(ie * H) * sizeof(WT);
  // the wave's staging area (256 f32x4) lies inside the span its partial
  // tiles take in `red` afterwards (2 * NT * 64), so no other wave's
  // accumulator store can land on a unit still being staged
  f32x4 *stage = red + wave * 2 * NT * 64;
  f32x4 acc[2][NT];   // [gate, up][column tile]
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[q][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load = [&](int bt, DgBufs<STEPS, NT> &b) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int us = UB * bt + u;
      int ur = us + rot;
      ur = ur >= nunits ? ur - nunits : ur;
      const bool live_u = us < nunits;
      const int cs = 8 * ur + sc;
      const uint32_t co = (uint32_t)((cw0 + cs) * CH) * sizeof(WT);
      const bool ls = live_u && cs < ncw;
      const uint32_t vo = ls ? rowg + co : kOutOfRange;
      b.a[u][0] = buf_ld16(rw, vo, 0);
      b.a[u][1] = buf_ld16(rw, vo, rows8);
      b.a[u][2] = buf_ld16(rw, vo, upo);
      b.a[u][3] = buf_ld16(rw, vo, upo + rows8);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 8 * ur + 4 * h + g;
        const bool live = live_u && c < ncw;
#pragma unroll
        for (int n = 0; n < NT; ++n)
          b.b[2 * u + h][n] =
              buf_ld16(rx, live && pos[n] >= 0 ? xpack_unit(cw0 + c, pos[n], T) * 16u : kOutOfRange, 0);
      }
    }
  };
  auto step = [&](int, const DgBufs<STEPS, NT> &b) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      // Lanes read what other lanes of the wave wrote: a wave's LDS accesses
      // execute in issue order, and the wavefront-scope fences keep the
      // compiler from moving them across one another.
#pragma unroll
      for (int v = 0; v < 4; ++v)
        stage[stage_slot(v >> 1, 8 * (v & 1) + sr, sc)] = __builtin_bit_cast(f32x4, b.a[u][v]);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      uint4 a[2][2];   // [k-step of the unit][gate, up]
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 2; ++q) a[h][q] = __builtin_bit_cast(uint4, stage[stage_slot(q, li, 4 * h + g)]);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[q][n] = mfma_chunk<W>(a[h][q], b.b[2 * u + h][n], acc[q][n]);
    }
  };
  DgBufs<STEPS, NT> b0, b1;
  pipeline((nunits + UB - 1) / UB, b0, b1, load, step);
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int n = 0; n < NT; ++n) red[((wave * 2 + q) * NT + n) * 64 + lane] = acc[q][n];
  __syncthreads();
  if (wave < NT) {
    // wave n finishes column tile n: rows i0 + 4g + r, entry 16n + li
    const int n = wave;
    f32x4 gt = red[n * 64 + lane], up = red[(NT + n) * 64 + lane];
#pragma unroll
    for (int v = 1; v < 4; ++v) {
      const f32x4 a = red[((v * 2 + 0) * NT + n) * 64 + lane], b = red[((v * 2 + 1) * NT + n) * 64 + lane];
      gt += a;
      up += b;
    }
    const int my_pos = pick_n<NT>(pos, n);
    if (my_pos >= 0) {
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = silu(gt[r]) * up[r];
      const int e = 16 * n + li, i = i0 + 4 * g;
      if constexpr (std::is_same<W, WBf16>::value) {
        // four values: half of chunk i / 8, as high parts and residuals
        bf16_t hv[4], lv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          hv[r] = f2bf(o[r]);
          lv[r] = f2bf(o[r] - bf2f(hv[r]));
        }
        const uint32_t half = (uint32_t)(i & 7) * 2u;
        *reinterpret_cast<uint2 *>(act + act_unit(i >> 3, 0, e, 2) * 16u + half) =
            make_uint2(pack2(hv[0], hv[1]), pack2(hv[2], hv[3]));
        *reinterpret_cast<uint2 *>(act + act_unit(i >> 3, 1, e, 2) * 16u + half) =
            make_uint2(pack2(lv[0], lv[1]), pack2(lv[2], lv[3]));
      } else {
        *reinterpret_cast<float4 *>(act + act_unit(i >> 2, 0, e, 1) * 16u) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }
  __syncthreads();  // `red` is free for the next item
}

}  // namespace bdd
