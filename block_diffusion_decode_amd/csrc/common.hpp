// Device helpers shared by the round's kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bdd {

constexpr int kWave = 64;
constexpr int kMaxT = 64;        // block positions handled per call
constexpr int kMaxE = 256;       // routed experts
constexpr int kActSlotPerI = 4 * kMaxT;  // bytes per intermediate unit of a packed activation slot (2 planes x kMaxT entries x bf16)
constexpr int kTokGroup = 4;     // positions per pass of the routed-expert kernels

typedef uint16_t bf16_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct WBf16 { typedef bf16_t T; static constexpr int kChunk = 8; };   // 16-byte chunk = 8 elements
struct WF32  { typedef float  T; static constexpr int kChunk = 4; };   // 16-byte chunk = 4 elements

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even (finite inputs; NaN -> quiet NaN).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ void unpack8(const uint4 &v, float (&f)[8]) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ uint32_t pack2(bf16_t lo, bf16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f2bf(v); }

// ---------------------------------------------------------------- memory

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
// Streaming load of weights that are read once per call.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) { return __builtin_bit_cast(bf16x8, v); }

// Wave-uniform copy of a value (lets the compiler keep it in an SGPR).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ unsigned long long uniform64(unsigned long long x) {
  return ((unsigned long long)(uint32_t)uniform((int)(x >> 32)) << 32) | (uint32_t)uniform((int)(uint32_t)x);
}

// Mask of the lanes below `lane` in a wave.
__device__ __forceinline__ unsigned long long lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Index of the j-th (from 0) set bit of m, for j < popcount(m): a binary
// search on the population counts of m's low bits.
__device__ __forceinline__ int nth_bit(unsigned long long m, int j) {
  int p = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const int c = __popcll((m >> p) & ((1ull << w) - 1ull));
    if (j >= c) {
      p += w;
      j -= c;
    }
  }
  return p;
}

// Raw buffer descriptor over [base, base + bytes): loads address it with a
// per-lane byte offset (VGPR) plus a wave-uniform byte offset (SGPR), and
// loads outside the range return zeros.  Word 3 = 32-bit data format.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// 16-byte streaming (non-temporal) load of weights read once per call.
__device__ __forceinline__ uint4 buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- cross-workgroup handoff
// One workgroup hands values to another workgroup of the same kernel (the
// last one to finish) as follows.  The values are stored and loaded as
// agent-scope atomics, so on this multi-XCD part they are not kept in a
// per-XCD L2.  The publishing workgroup's waves meet at a barrier (whose
// workgroup-scope release orders every wave's stores before it), then one
// thread increments the workgroup counter with an agent-scope release
// read-modify-write.  Only the workgroup whose increment returns the last
// count takes an agent-scope acquire fence: its increment read the end of the
// counter's release sequence, so the fence makes every value published before
// any earlier increment visible to it, and a barrier then passes that on to
// its other waves.  (An agent-scope acquire invalidates the XCD's L2 and a
// release writes it back; the workgroups that are not last take neither the
// invalidate nor an acquire they do not use.)
template <typename T>
__device__ __forceinline__ void publish(T *p, T v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
template <typename T>
__device__ __forceinline__ T fetch_published(const T *p) {
  return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Counts this workgroup as done (release of what it published) and returns
// whether it is the last of n; the last one has acquired what all the others
// published.
__device__ __forceinline__ bool count_done_last(int32_t *counter, int n) {
  const bool last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}
// Counts this workgroup (agent-scope release increment), then waits until
// the counter reaches n, with relaxed loads, and acquires once: after it,
// every value the n counted workgroups published before their increments is
// visible.  Gives up after max_spins sleeps and returns false.  (It waits for
// workgroups that may not have started, so n must not exceed the workgroups
// the device runs at once.)
__device__ __forceinline__ bool count_and_wait_all(int32_t *counter, int n, int max_spins) {
  __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  int spins = 0;
  bool ok = true;
  while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n) {
    if (++spins > max_spins) {
      ok = false;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return ok;
}

// ---------------------------------------------------------------- block-resident rounds
// A block's rounds can all be enqueued at once: each kernel of a round takes
// the block's resolved flag as its gate (null: always run) and returns at
// entry once the commit of an earlier round has set it.  The flag was written
// by an earlier kernel on the same stream, so a plain load sees it.
__device__ __forceinline__ bool gated_off(const int32_t *gate) {
  return gate != nullptr && __builtin_amdgcn_readfirstlane(*gate) != 0;
}

// ---------------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s));
  return v;
}
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
  return v;
}

template <int N>
constexpr int log2i() { return N <= 1 ? 0 : 1 + log2i<N / 2>(); }

// DPP wave reductions (VALU lane exchanges, no LDS): xor 1 and xor 2 within
// quads, mirror within 8 and 16 lanes, then row broadcasts 15 and 31 fold the
// four rows into lane 63, whose value is broadcast with readlane.  `old` is
// the identity element given to lanes a row mask leaves unwritten.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dppf(float old, float v) {
  return __int_as_float(dpp<CTRL, ROWS>(__float_as_int(old), __float_as_int(v)));
}
#define BDD_DPP_STEPS(F) F(0xB1, 0xF) F(0x4E, 0xF) F(0x141, 0xF) F(0x140, 0xF) F(0x142, 0xA) F(0x143, 0xC)

__device__ __forceinline__ float wave_sum_dpp(float v) {
#define BDD_STEP(C, R) v += dppf<C, R>(0.f, v);
  BDD_DPP_STEPS(BDD_STEP)
#undef BDD_STEP
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
#define BDD_STEP(C, R) v = fmaxf(v, dppf<C, R>(-3.402823466e38f, v));
  BDD_DPP_STEPS(BDD_STEP)
#undef BDD_STEP
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Largest value, lowest index among equal values; result uniform.
__device__ __forceinline__ void wave_argmax_dpp(float &v, int &i) {
#define BDD_STEP(C, R)                                              \
  {                                                                 \
    const float v2 = dppf<C, R>(-3.402823466e38f, v);               \
    const int i2 = dpp<C, R>(0x7fffffff, i);                        \
    const bool take = v2 > v || (v2 == v && i2 < i);                \
    v = take ? v2 : v;                                              \
    i = take ? i2 : i;                                              \
  }
  BDD_DPP_STEPS(BDD_STEP)
#undef BDD_STEP
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}

// keep + the partner's `send`, partners paired by a DPP pattern (S <= 8)
template <int S>
__device__ __forceinline__ float pair_level(float keep, float send) {
  static_assert(S >= 1 && S <= 8, "DPP levels");
  if constexpr (S == 8) {
    return keep + dppf<0x140, 0xF>(0.f, send);   // row_mirror
  } else if constexpr (S == 4) {
    return keep + dppf<0x141, 0xF>(0.f, send);   // row_half_mirror
  } else if constexpr (S == 2) {
    return keep + dppf<0x4E, 0xF>(0.f, send);    // quad_perm [2,3,0,1]
  } else {
    return keep + dppf<0xB1, 0xF>(0.f, send);    // quad_perm [1,0,3,2]
  }
}

// Levels 32 and 16: lo_half is the value lanes with bit S clear keep, hi_half
// the one lanes with bit S set keep.  The swap hands each lane its own kept
// value and its partner's copy of it, in some order; their sum is the level's
// result.
template <int S>
__device__ __forceinline__ float swap_sum(float lo_half, float hi_half) {
  const uint32_t a = __float_as_uint(lo_half), b = __float_as_uint(hi_half);
  if constexpr (S == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

template <int N, int S>
__device__ __forceinline__ void rs_level(float *v, int lane) {
  if constexpr (S >= 1) {
    if constexpr (N > 1) {
      constexpr int half = N / 2;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        if constexpr (S >= 16) {
          v[i] = swap_sum<S>(v[i], v[i + half]);
        } else {
          const bool upper = (lane & S) != 0;
          const float send = upper ? v[i] : v[i + half];
          const float keep = upper ? v[i + half] : v[i];
          v[i] = pair_level<S>(keep, send);
        }
      }
      rs_level<half, S / 2>(v, lane);
    } else {
      if constexpr (S >= 16) v[0] = swap_sum<S>(v[0], v[0]);
      else v[0] = pair_level<S>(v[0], v[0]);
      rs_level<1, S / 2>(v, lane);
    }
  }
}
// Reduce N partial values per lane across the 64 lanes of a wave, leaving
// lane l with the total of value index (l >> (6 - log2 N)).  N is a power of
// two <= 64.  Halving exchange: at each level (lane bit S = 32, 16, ..., 1)
// a lane keeps the half of its values selected by its own bit S and adds the
// partner's copy of that half; once one value is left the remaining levels
// are a plain butterfly.  Partners differ in bit S and agree on the higher
// bits: lane ^ 32 and lane ^ 16 through v_permlane32_swap / v_permlane16_swap,
// then the mirror within 16 and within 8 lanes and the quad exchanges through
// DPP, so no exchange goes through LDS.  Register indices are compile-time
// constants.
template <int N>
__device__ __forceinline__ float reduce_scatter(float (&v)[N], int lane) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
  rs_level<N, 32>(v, lane);
  return v[0];
}

// ---------------------------------------------------------------- 4-bit weights
// 4-bit weight-only matrices (two codes per byte, code n standing for n - 8,
// one bf16 scale per row and 128-column group) are packed in 16-row tiles:
// per tile and group one KiB in MFMA lane order (lane li + 16 g: row li; dword
// kk: the 8 codes of k-step 4 group + kk, columns 32 (4 group + kk) + 8 g + e,
// code e at bit 4 (e / 2) + 16 (e % 2)), then the scales [tile][group][16].
// ((x >> 4 d) & 0x000f000f) | 0x43004300 turns codes 2d and 2d + 1 into the
// bf16 pair 128 + n (exact), which MFMAs take as bf16 weights; a group's sum
// over (128 + n) h is its sum over (n - 8) h plus 136 sum h.
struct WI4 { typedef bf16_t T; static constexpr int kChunk = 8; };   // h is bf16
constexpr int kI4Group = 128;
constexpr float kI4Offset = 136.f;
// 8-byte load of scales: cached normally (a tile's 128-byte line of scales
// serves several load batches; the streaming hint would evict it in between)
__device__ __forceinline__ uint2 buf_ld8(rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
  return make_uint2(v.x, v.y);
}
// a's m bits inserted into c: one v_bfi_b32.  (Plain code, so the compiler's
// hazard tracking sees every instruction next to the MFMAs.)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) { return (a & m) | (c & ~m); }
// The expansion's mask and bias, held in vector registers: v_bfi_b32 takes
// no literal operand on this target, so with literal constants each insert
// became an and plus an or.  (mbcnt over an empty lane mask returns its
// addend; the compiler does not fold it into a literal.)
struct I4Bits {
  uint32_t m, c;
};
__device__ __forceinline__ I4Bits i4_bits() {
  return {__builtin_amdgcn_mbcnt_lo(0u, 0x000f000fu), __builtin_amdgcn_mbcnt_lo(0u, 0x43004300u)};
}
// codes 2d and 2d + 1 of a dword (see WI4) as the bf16 pair 128 + n
__device__ __forceinline__ uint4 i4_expand(uint32_t x, const I4Bits &k) {
  return make_uint4(and_or(x, k.m, k.c), and_or(x >> 4, k.m, k.c), and_or(x >> 8, k.m, k.c),
                    and_or(x >> 12, k.m, k.c));
}
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// The value of lane ^ S (S = 16 or 32), through v_permlane16/32_swap: the
// swap leaves a lane's own value in one result and its partner's in the other.
template <int S>
__device__ __forceinline__ uint32_t partner_u32(uint32_t v, int lane) {
  const auto r = S == 32 ? __builtin_amdgcn_permlane32_swap(v, v, false, false)
                         : __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (lane & S) ? r[0] : r[1];
}
template <int S>
__device__ __forceinline__ float partner_f32(float v, int lane) {
  return __uint_as_float(partner_u32<S>(__float_as_uint(v), lane));
}
template <int S>
__device__ __forceinline__ int partner_i32(int v, int lane) {
  return (int)partner_u32<S>((uint32_t)v, lane);
}


// ---------------------------------------------------------------- math

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4_f32.  For both, lane l holds
// A row (l & 15) and B column (l & 15) for k-group (l >> 4), and the 16x16
// result as rows 4*(l >> 4) + r, column (l & 15), r = 0..3.  Any consistent
// assignment of k values to (k-group, item) gives the same dot products.

__device__ __forceinline__ f32x4 mfma_bf16(const uint4 &a, const uint4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Split 8 fp32 values into bf16 high parts and bf16 residuals, so that a
// bf16 MFMA pass over each reproduces fp32-accurate products with bf16 weights.
__device__ __forceinline__ void split_hi_lo(const float (&x)[8], uint4 &hi, uint4 &lo) {
  bf16_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = f2bf(x[i]);
    l[i] = f2bf(x[i] - bf2f(h[i]));
  }
  hi = make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
  lo = make_uint4(pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7]));
}

}  // namespace bdd
