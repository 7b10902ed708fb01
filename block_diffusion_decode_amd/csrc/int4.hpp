// Expert projections with 4-bit weights (the 4-bit tile format described in
// common.hpp).  Every 4-bit item runs on MFMA: a dense expert or the shared
// expert as two 16-entry column tiles, a token group (at most kTokGroup
// positions) as one.  Weights are read straight into operand order: one
// 16-byte lane load holds a row's four k-steps of a 128-column group, so each
// load instruction reads one contiguous KiB.
//
// Pages: [P3] 10100.com article on Clover-35B-A3B-Preview, part 03 (memory and
// quantisation: the model is deployed with INT4 weights; the pages give no
// format, the one read here is stated in common.hpp and in the library's
// header).
#pragma once

#include "common.hpp"
#include "stream.hpp"

namespace bdd {

// One packed 4-bit matrix of `rows` x `cols` (rows a multiple of 16, cols of 128).
struct I4Mat {
  const char *codes;        // tiles x groups x 1 KiB
  const uint16_t *scl;      // [tile][group][16] bf16
  int G;                    // 128-column groups per row
  uint32_t code_bytes;      // tiles * groups * 1 KiB
};
__host__ __device__ inline size_t i4_mat_bytes(int rows, int cols) {
  const size_t tiles = (size_t)((rows + 15) / 16);
  return tiles * (size_t)(8 * cols) + tiles * (size_t)(cols / kI4Group) * 32;
}
__device__ __forceinline__ I4Mat i4_mat(const void *packed, int rows, int cols) {
  I4Mat m;
  const int tiles = (rows + 15) / 16;
  m.G = cols / kI4Group;
  m.code_bytes = (uint32_t)tiles * (uint32_t)(8 * cols);
  m.codes = static_cast<const char *>(packed);
  m.scl = reinterpret_cast<const uint16_t *>(m.codes + m.code_bytes);
  return m;
}

// Sum of the 8 bf16 values of a chunk.
__device__ __forceinline__ float sum8_bf16(const uint4 &v) {
  return ((bf_lo(v.x) + bf_hi(v.x)) + (bf_lo(v.y) + bf_hi(v.y))) +
         ((bf_lo(v.z) + bf_hi(v.z)) + (bf_lo(v.w) + bf_hi(v.w)));
}
// The total of a per-lane value over the four lanes li, li + 16, li + 32, li + 48.
__device__ __forceinline__ float sum_over_kgroups(float v, int lane) {
  v += partner_f32<16>(v, lane);
  return v + partner_f32<32>(v, lane);
}

template <int NT>
struct I4GuBufs {
  uint4 a[2];            // gate and up codes of one group
  uint2 s[2];            // their scales (rows 4 g .. 4 g + 3)
  uint4 b[4][NT];        // the block's operand, four k-steps
};

// Gate/up of a 4-bit expert for intermediate rows i0 .. i0 + 15: gate tile
// i0 / 16 and up tile (ie + i0) / 16 of W_gu [2 ie][H], against NT column
// tiles of entries (lane (li, g) names entries li + 16 n by the positions
// pos[n], -1: none) of the packed normalised block.  The four waves take the
// 128-column groups round-robin, two groups' loads in flight per wave; per
// group the MFMAs sum (128 + n) x over the group, then the row's scale times
// (that sum - 136 sum x) joins the accumulator.  The waves' partial tiles are
// added in `red` (4 * 2 * NT * 64 f32x4); wave n then finishes column tile n:
// silu(gate) * up goes to the packed activation slot `act` (entry 16 n + li)
// when arow is null, else to A[arow[n]][i] (entries with arow[n] < 0 skipped).
template <int NT>
__device__ __forceinline__ void i4_gateup_item(const I4Mat &w, int ie, const bf16_t *__restrict__ xpk, int T,
                                               const int (&pos)[NT], int i0, int wave, int lane,
                                               char *__restrict__ act, float *__restrict__ A, const int *arow,
                                               int Imax, f32x4 *red) {
  const int li = lane & 15, g = lane >> 4;
  const int tg = i0 / 16, tu = (ie + i0) / 16;
  const int G = w.G;
  const I4Bits kb = i4_bits();
  const rsrc_t rc = make_rsrc(w.codes, w.code_bytes);
  const rsrc_t rs = make_rsrc(w.scl, w.code_bytes / 32u);   // scales: 32 bytes per tile and group
  const rsrc_t rx = make_rsrc(xpk, (uint32_t)(T * G * kI4Group) * 2u);
  f32x4 acc[2][NT];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[q][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ng = (G - wave + 3) / 4;   // this wave's groups: wave, wave + 4, ...
  auto load = [&](int st, I4GuBufs<NT> &b) {
    const int gq = wave + 4 * st;
    const bool live = st < ng;
    const int gc = live ? gq : 0;
    b.a[0] = buf_ld16(rc, live ? (uint32_t)lane * 16u : kOutOfRange, (uint32_t)(tg * G + gc) * 1024u);
    b.a[1] = buf_ld16(rc, live ? (uint32_t)lane * 16u : kOutOfRange, (uint32_t)(tu * G + gc) * 1024u);
    b.s[0] = buf_ld8(rs, live ? (uint32_t)g * 8u : kOutOfRange, (uint32_t)(tg * G + gc) * 32u);
    b.s[1] = buf_ld8(rs, live ? (uint32_t)g * 8u : kOutOfRange, (uint32_t)(tu * G + gc) * 32u);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int n = 0; n < NT; ++n)
        b.b[kk][n] = buf_ld16(rx, live && pos[n] >= 0 ? xpack_unit(4 * (4 * gc + kk) + g, pos[n], T) * 16u : kOutOfRange,
                              0);
  };
  auto step = [&](int st, const I4GuBufs<NT> &b) {
    if (st >= ng) return;
    float xs[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float v = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) v += sum8_bf16(b.b[kk][n]);
      xs[n] = kI4Offset * sum_over_kgroups(v, lane);
    }
    f32x4 p[2][NT];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int n = 0; n < NT; ++n) p[q][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 &aq = b.a[q];
        const uint4 e = i4_expand(kk == 0 ? aq.x : kk == 1 ? aq.y : kk == 2 ? aq.z : aq.w, kb);
#pragma unroll
        for (int n = 0; n < NT; ++n) p[q][n] = mfma_bf16(e, b.b[kk][n], p[q][n]);
      }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float sr[4] = {bf_lo(b.s[q].x), bf_hi(b.s[q].x), bf_lo(b.s[q].y), bf_hi(b.s[q].y)};
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[q][n][r] = fmaf(sr[r], p[q][n][r] - xs[n], acc[q][n][r]);
    }
  };
  I4GuBufs<NT> b0, b1;
  pipeline(ng, b0, b1, load, step);
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int n = 0; n < NT; ++n) red[((wave * 2 + q) * NT + n) * 64 + lane] = acc[q][n];
  __syncthreads();
  if (wave < NT) {
    const int n = wave;
    f32x4 gt = red[(0 * NT + n) * 64 + lane], up = red[(1 * NT + n) * 64 + lane];
#pragma unroll
    for (int v = 1; v < 4; ++v) {
      gt += red[((v * 2 + 0) * NT + n) * 64 + lane];
      up += red[((v * 2 + 1) * NT + n) * 64 + lane];
    }
    // (value arithmetic rather than a runtime index into pos / arow)
    int my_pos = pos[0];
#pragma unroll
    for (int j = 1; j < NT; ++j) my_pos = n == j ? pos[j] : my_pos;
    float o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = silu(gt[r]) * up[r];
    const int i = i0 + 4 * g;
    if (arow == nullptr) {
      if (my_pos >= 0) {
        // four values: half of chunk i / 8, as high parts and residuals
        const int e = 16 * n + li;
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
      }
    } else {
      int my_row = arow[0];
#pragma unroll
      for (int j = 1; j < NT; ++j) my_row = n == j ? arow[j] : my_row;
      if (my_row >= 0)
        *reinterpret_cast<float4 *>(A + (size_t)my_row * Imax + i) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
  __syncthreads();  // `red` is free for the next item
}

// Down projection of a 4-bit W_d [H][ie] for rows h0 .. h0 + 16 MT - 1 (MT
// tiles from h0 / 16), against NT column tiles of entries.  The activations come
// from the packed slot `act` (bf16 high parts and residuals, entry 16 n + li)
// when A is null, else from the fp32 rows A[arow[n]] (split into high parts
// and residuals here).  Each MFMA pass takes the high parts, then the
// residuals; per group the correction is 136 times the group's sum of both.
// The four waves take the groups round-robin and add their partial tiles in
// `red` (4 * MT * NT * 64 f32x4); P[prow[n]][h] receives the unweighted rows.
// From the packed slot, entries with live[n] < 0 are absent (prow is read
// only at the end).
template <int MT, int NT>
__device__ __forceinline__ void i4_down_item(const I4Mat &w, int ie, const char *__restrict__ act,
                                             const float *__restrict__ A, const int *arow, uint32_t a_bytes,
                                             int Imax, int H, const int (&live)[NT], const int (&prow)[NT], int h0,
                                             int wave, int lane, float *__restrict__ P, f32x4 *red) {
  const int li = lane & 15, g = lane >> 4;
  const int t0 = h0 / 16;
  const int G = w.G;
  const I4Bits kb = i4_bits();
  const rsrc_t rc = make_rsrc(w.codes, w.code_bytes);
  const rsrc_t rs = make_rsrc(w.scl, w.code_bytes / 32u);
  const rsrc_t ra = A ? make_rsrc(A, a_bytes) : make_rsrc(act, (uint32_t)ie * kActSlotPerI);
  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int gq = wave; gq < G; gq += 4) {
    uint4 a[MT];
    uint2 sc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      a[m] = buf_ld16(rc, (uint32_t)lane * 16u, (uint32_t)((t0 + m) * G + gq) * 1024u);
      sc[m] = buf_ld8(rs, (uint32_t)g * 8u, (uint32_t)((t0 + m) * G + gq) * 32u);
    }
    uint4 hi[4][NT], lo[4][NT];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int C = 4 * (4 * gq + kk) + g;     // chunk of 8 intermediate units
        if (A) {
          int my_row = arow[0];
#pragma unroll
          for (int j = 1; j < NT; ++j) my_row = n == j ? arow[j] : my_row;
          const uint32_t off = my_row >= 0 ? ((uint32_t)my_row * (uint32_t)Imax + (uint32_t)C * 8u) * 4u : kOutOfRange;
          const uint4 x0 = buf_ld16(ra, off, 0), x1 = buf_ld16(ra, off == kOutOfRange ? off : off + 16u, 0);
          const float f[8] = {__uint_as_float(x0.x), __uint_as_float(x0.y), __uint_as_float(x0.z),
                              __uint_as_float(x0.w), __uint_as_float(x1.x), __uint_as_float(x1.y),
                              __uint_as_float(x1.z), __uint_as_float(x1.w)};
          split_hi_lo(f, hi[kk][n], lo[kk][n]);
        } else {
          int my_live = live[0];
#pragma unroll
          for (int j = 1; j < NT; ++j) my_live = n == j ? live[j] : my_live;
          const bool ok = my_live >= 0;
          hi[kk][n] = buf_ld16(ra, ok ? act_unit(C, 0, 16 * n + li, 2) * 16u : kOutOfRange, 0);
          lo[kk][n] = buf_ld16(ra, ok ? act_unit(C, 1, 16 * n + li, 2) * 16u : kOutOfRange, 0);
        }
      }
    float xs[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float v = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) v += sum8_bf16(hi[kk][n]) + sum8_bf16(lo[kk][n]);
      xs[n] = kI4Offset * sum_over_kgroups(v, lane);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      f32x4 p[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) p[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint4 e = i4_expand(kk == 0 ? a[m].x : kk == 1 ? a[m].y : kk == 2 ? a[m].z : a[m].w, kb);
#pragma unroll
        for (int n = 0; n < NT; ++n) p[n] = mfma_bf16(e, lo[kk][n], mfma_bf16(e, hi[kk][n], p[n]));
      }
      const float sr[4] = {bf_lo(sc[m].x), bf_hi(sc[m].x), bf_lo(sc[m].y), bf_hi(sc[m].y)};
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[m][n][r] = fmaf(sr[r], p[n][r] - xs[n], acc[m][n][r]);
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) red[((wave * MT + m) * NT + n) * 64 + lane] = acc[m][n];
  __syncthreads();
  // wave v finishes output tiles v, v + 4, ... (tile q: row tile q / NT, column tile q % NT)
  for (int q = wave; q < MT * NT; q += 4) {
    const int m = q / NT, n = q % NT;
    f32x4 v = red[q * 64 + lane];
#pragma unroll
    for (int u = 1; u < 4; ++u) v += red[(u * MT * NT + q) * 64 + lane];
    int my_row = prow[0];
#pragma unroll
    for (int j = 1; j < NT; ++j) my_row = n == j ? prow[j] : my_row;
    if (my_row >= 0)
      *reinterpret_cast<float4 *>(P + (size_t)my_row * H + h0 + 16 * m + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
  }
  __syncthreads();  // `red` is free for the next item
}

}  // namespace bdd
