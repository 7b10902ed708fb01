// LM head with a fused softmax-confidence/argmax epilogue, and the
// LowConfidence commit.
//
// Pages: [P1] aitujian.cn article on Clover-35B-A3B-Preview, section 三: each
// round runs one forward over the block, takes every position's argmax and its
// probability (the confidence), writes positions with confidence >= 0.95 for
// good, and when none reaches it forces the single most confident one; written
// tokens are never revised.  [P2] goremy.ai "What Is Clover-35B-A3B? Block
// Diffusion on a Qwen3.6 MoE", "How does confidence-threshold block decoding
// work?" (same loop; scores each masked position).
//
// conf = max_v softmax(z)_v = 1 / sum_v exp(z_v - max z), so the kernel keeps,
// per position, a running (max, sum of exp(z - max), argmax) over vocabulary
// tiles and never stores a logit.
#include <float.h>
#include <limits.h>
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace bdd {

constexpr int kLmWaves = 16;

// Online-softmax merge of (m2, s2, i2) into (m, s, i): max, rescaled sum,
// lowest index among equal maxima.
__device__ __forceinline__ void sm_merge(float &m, float &s, int &i, float m2, float s2, int i2) {
  if (s2 == 0.f) return;
  if (s == 0.f) { m = m2; s = s2; i = i2; return; }
  if (m2 > m) {
    s = s * __expf(m - m2) + s2;
    m = m2;
    i = i2;
  } else if (m2 < m) {
    s += s2 * __expf(m2 - m);
  } else {
    s += s2;
    i = min(i, i2);
  }
}

// Each lane loads one 16-byte unit per MFMA k-step: k-step s of a 16-row tile
// is one contiguous KiB of the packed weight in which lane l = li + 16 g finds
// its operand (row li, chunk 4s + g) at byte 16 l.  Loads go in batches of
// lm_batch<W>() such units; two batches are in flight per wave.
//
// 4-bit weights (WI4): one KiB unit covers a whole 128-column group of the
// tile, four k-steps: lane l's 16 bytes hold, in dword kk, the 8 codes of row
// li at columns 32 (4 grp + kk) + 8 g + e, code e at bit 4 (e / 2) + 16 (e % 2).
// ((x >> 4 d) & 0x000f000f) | 0x43004300 then turns codes 2d and 2d + 1 into
// the bf16 values 128 + n (exact), which the MFMA takes as it takes bf16
// weights.  With S = sum over the group of h, a group's tile sum is
// sum (128 + n) h = sum (n - 8) h + 136 S, so the kernel subtracts 136 S and
// multiplies by the row's scale once per group.  Scales: 16 bf16 per (tile,
// group), after all the codes; lane (li, g) reads those of its output rows
// 4g .. 4g + 3.
//
// Units per tile per load batch, and tiles a wave streams side by side: a
// 4-bit wave of a block of up to 32 positions works on two tiles at once, so
// every block operand it reads from LDS feeds both tiles' MFMAs (a bf16 tile
// is HBM-bound on its own).
//
// H phases: a block of up to 32 positions is staged whole (one phase).  A
// wider one (64 positions: 256 KiB of bf16 at H = 2048) would not fit in
// LDS, so the block is staged half of H at a time: each wave takes its tiles
// in groups of lm_group() tile steps, runs the group's k-steps over the
// staged half into per-tile accumulators, the workgroup restages the other
// half, and the group's k-steps over that half finish its tiles.  The next
// group starts with the half that is staged, so a workgroup restages once
// per group, and every weight still streams once.
template <class W, int NT>
constexpr int lm_phases() { return NT > 2 ? 2 : 1; }
template <class W, int NT>
constexpr int lm_batch() { return std::is_same<W, WI4>::value ? 2 : (NT > 2 ? 4 : 8); }
template <class W, int NT>
constexpr int lm_tiles() { return std::is_same<W, WI4>::value && NT <= 2 ? 2 : 1; }
template <class W, int NT>
constexpr int lm_group() { return NT > 2 ? 2 : 1; }
template <class W, int NT>
struct LmBufs {
  uint4 a[lm_tiles<W, NT>()][lm_batch<W, NT>()];
  uint2 sc[lm_tiles<W, NT>()][std::is_same<W, WI4>::value ? lm_batch<W, NT>() : 1];
};
// A buffer offset past every LM-head tile: such a load returns zeros without
// a memory access (pads the prefetches past a wave's last step).
constexpr uint32_t kLmOutOfRange = 0x7ff00000u;

// Merge the per-workgroup partials of every position (fixed order), then the
// commit rule on the still-masked positions.  Run by one whole workgroup of
// any multiple of 64 threads.  Each half-wave merges one position: its 32
// lanes load every 32nd partial (all loads issued before any merge), then
// fold their results pairwise, lower lane first.
constexpr int kCommitBatch = 8;
__device__ void commit_block(const float *__restrict__ part_m, const float *__restrict__ part_s,
                             const int32_t *__restrict__ part_i, int nparts, int T, float threshold,
                             int32_t *__restrict__ tokens, float *__restrict__ conf,
                             int32_t *__restrict__ choice, int32_t *__restrict__ round_info,
                             int32_t *__restrict__ resolved_flag) {
  __shared__ float s_conf[kMaxT];
  __shared__ int s_choice[kMaxT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int hl = lane & 31;
  // the block's tokens, read ahead of the merge by the wave that commits
  const int tok = (wave == 0 && lane < T) ? tokens[lane] : 0;
  for (int tp = 2 * wave; tp < T; tp += 2 * nw) {
    const int t = tp + (lane >> 5);
    const bool live = t < T;
    float m = -FLT_MAX, s = 0.f;
    int i = INT_MAX;
    for (int base = hl; base < nparts; base += 32 * kCommitBatch) {
      float pm[kCommitBatch], ps[kCommitBatch];
      int pi[kCommitBatch];
      // (after the acquire of the workgroup count, or a kernel boundary:
      // plain loads of clamped indices, all in flight together; entries past
      // the partials are then neutralised)
#pragma unroll
      for (int j = 0; j < kCommitBatch; ++j) {
        const int p = base + 32 * j;
        const size_t at = (size_t)min(t, T - 1) * nparts + min(p, nparts - 1);
        pm[j] = part_m[at];
        ps[j] = part_s[at];
        pi[j] = part_i[at];
      }
#pragma unroll
      for (int j = 0; j < kCommitBatch; ++j) {
        const bool ok = live && base + 32 * j < nparts;
        ps[j] = ok ? ps[j] : 0.f;
        pi[j] = ok ? pi[j] : INT_MAX;
      }
#pragma unroll
      for (int j = 0; j < kCommitBatch; ++j) sm_merge(m, s, i, pm[j], ps[j], pi[j]);
    }
#pragma unroll
    for (int sft = 1; sft <= 16; sft <<= 1) {
      const float m2 = __shfl_xor(m, sft), s2 = __shfl_xor(s, sft);
      const int i2 = __shfl_xor(i, sft);
      // both partners merge the same pair in the same order: lower lane first
      if (lane & sft) {
        float mm = m2, ss = s2;
        int ii = i2;
        sm_merge(mm, ss, ii, m, s, i);
        m = mm; s = ss; i = ii;
      } else {
        sm_merge(m, s, i, m2, s2, i2);
      }
    }
    if (live && hl == 0) {
      const float c = 1.0f / s;
      s_conf[t] = c;
      s_choice[t] = i;
      conf[t] = c;
      choice[t] = i;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const bool in = lane < T;
    const bool masked = in && tok == -1;
    const float c = in ? s_conf[lane] : 0.f;
    const unsigned long long pass = __ballot(masked && c >= threshold);
    const unsigned long long msk = __ballot(masked);
    int committed = 0, fallback = 0;
    bool write = false;
    if (pass) {
      write = (pass >> lane) & 1ull;
      committed = __popcll(pass);
    } else if (msk) {
      float bv = masked ? c : -FLT_MAX;
      int bi = masked ? lane : INT_MAX;
      wave_argmax_dpp(bv, bi);
      write = lane == bi;
      committed = 1;
      fallback = 1;
    }
    if (write) tokens[lane] = s_choice[lane];
    const int left = __popcll(msk) - committed;
    if (lane == 0) {
      round_info[0] = committed;
      round_info[1] = fallback;
      round_info[2] = left;
      round_info[3] = left == 0 ? 1 : 0;
      if (resolved_flag && left == 0) *resolved_flag = 1;
    }
  }
}

__global__ __launch_bounds__(1024) void commit_kernel(const float *__restrict__ part_m,
                                                      const float *__restrict__ part_s,
                                                      const int32_t *__restrict__ part_i,
                                                      int nparts, int T, float threshold,
                                                      int32_t *__restrict__ tokens,
                                                      float *__restrict__ conf,
                                                      int32_t *__restrict__ choice,
                                                      int32_t *__restrict__ round_info,
                                                      const int32_t *__restrict__ gate,
                                                      int32_t *__restrict__ resolved_flag) {
  if (gated_off(gate)) return;
  commit_block(part_m, part_s, part_i, nparts, T, threshold, tokens, conf, choice, round_info, resolved_flag);
}

// Start of a block whose rounds are all enqueued at once: every position
// MASK, the per-round info slots cleared, the resolved flag (the rounds'
// gate) cleared.  A kernel rather than memsets, so it can sit in a graph.
__global__ __launch_bounds__(256) void block_start_kernel(int32_t *__restrict__ tokens, int T,
                                                          int32_t *__restrict__ info, int words,
                                                          int32_t *__restrict__ flag) {
  for (int i = threadIdx.x; i < T; i += blockDim.x) tokens[i] = -1;
  for (int i = threadIdx.x; i < words; i += blockDim.x) info[i] = 0;
  if (threadIdx.x == 0) *flag = 0;
}

// One workgroup (16 waves) per CU.  The block's normalised hidden states are
// staged once in LDS as [chunk][position] 16-byte entries; each wave takes
// 16-row vocabulary tiles round-robin (wave w of workgroup b starts at tile
// w * grid + b, so a workgroup's tiles are spread over the whole weight
// rather than one contiguous MiB per round, which evened out the finish times
// of the workgroups on the different XCDs), streams the rows with 16-byte loads,
// multiplies them by the staged positions on MFMA, and folds the 16 x 32
// logits into its running (max, sum, argmax).
// With `done_count` given, the workgroup that finishes last (agent-scope
// release counter over partials published as agent-scope atomics; the last
// one acquires)
// also merges the partials and runs the commit, then clears the counter.  The
// counter must be zero when the kernel starts.
template <class W, int NT>
__global__ __launch_bounds__(1024) void lmhead_kernel(const typename W::T *__restrict__ hhat,
                                                      const typename W::T *__restrict__ wlm,
                                                      const uint16_t *__restrict__ scl, int T,
                                                      int H, int V, float *__restrict__ part_m,
                                                      float *__restrict__ part_s,
                                                      int32_t *__restrict__ part_i,
                                                      int32_t *__restrict__ done_count, float threshold,
                                                      int32_t *__restrict__ tokens,
                                                      float *__restrict__ conf,
                                                      int32_t *__restrict__ choice,
                                                      int32_t *__restrict__ round_info,
                                                      const int32_t *__restrict__ gate,
                                                      int32_t *__restrict__ resolved_flag) {
  extern __shared__ uint4 xs[];  // [H / kChunk][16 * NT]
  __shared__ float sm[kLmWaves][16 * NT], ssum[kLmWaves][16 * NT];
  __shared__ int si[kLmWaves][16 * NT];
  constexpr int CH = W::kChunk;
  constexpr int TP = 16 * NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NC = H / CH;
  const int li = lane & 15, g = lane >> 4;
  if (gated_off(gate)) return;
  float m[NT], s[NT];
  int am[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) { m[n] = -FLT_MAX; s[n] = 0.f; am[n] = INT_MAX; }

  // The wave's tiles (first, first + stride, ...) and their k-step batches
  // form one flat sequence of load steps, so the next tile's first batch is in
  // flight during a tile's epilogue, and the first batch during the staging.
  constexpr bool I4 = std::is_same<W, WI4>::value;
  const I4Bits kb = i4_bits();
  constexpr int LB = lm_batch<W, NT>();
  constexpr int TW = lm_tiles<W, NT>();
  constexpr int PH = lm_phases<W, NT>();
  constexpr int TG = lm_group<W, NT>();
  static_assert(PH == 1 || TP == 64, "a phased block is staged one position per lane");
  const int ntiles = (V + 15) / 16;
  const int ksteps = NC / 4;                    // MFMA k-steps per tile
  const int lsteps = I4 ? ksteps / 4 : ksteps;  // KiB load units per tile
  // phase 0 takes the first ceil(lsteps / PH) units of a tile, phase 1 the rest
  const int lph0 = (lsteps + PH - 1) / PH;
  const int cpu = NC / lsteps;                  // staged chunks per unit
  const int NCP = lph0 * cpu;                   // staged chunks (the larger phase)
  const int nb = (lph0 + LB - 1) / LB;          // load batches per tile and phase
  float *hs = reinterpret_cast<float *>(xs + NCP * TP);   // [H / 128][16 NT]: group sums of h (WI4)
  const int first = uniform(wave * (int)gridDim.x + (int)blockIdx.x);
  const int stride = gridDim.x * kLmWaves;
  const int my_tiles = first < ntiles ? (ntiles - 1 - first) / stride + 1 : 0;
  // with phases every wave runs the same steps (the restages are workgroup
  // barriers): as many groups as the workgroup's first wave, which has the
  // most tiles; a wave's steps past its own tiles load and fold nothing
  const int tiles0 = (int)blockIdx.x < ntiles ? (ntiles - 1 - (int)blockIdx.x) / stride + 1 : 0;
  const int ngroups = ((tiles0 + TW - 1) / TW + TG - 1) / TG;
  const int gsteps = PH * TG * nb;              // steps per group
  const int steps = PH == 1 ? (my_tiles + TW - 1) / TW * nb : ngroups * gsteps;
  // A step: tile step k (tiles TW k .. TW k + TW - 1 of the wave), batch b,
  // the H phase hph it covers, its tile step kin within the group and
  // whether it belongs to the group's second phase (which finishes the
  // tiles).  Two cursors walk the steps by increments (no divisions): one for
  // the MFMAs, one for the loads two steps ahead.
  struct Step {
    int k, b, hph, kin, pi, grp;
    __device__ bool second() const { return pi == PH - 1; }
    __device__ int u0(int l0) const { return hph * l0; }                       // the phase's first unit
    __device__ int units(int l0, int ls) const { return hph ? ls - l0 : l0; }   // and its units
    __device__ void next(int nbatch) {
      if (++b < nbatch) return;
      b = 0;
      if (++kin < TG) {
        ++k;
        return;
      }
      kin = 0;
      if (++pi < PH) {
        k -= TG - 1;
      } else {
        pi = 0;
        ++grp;
        ++k;
      }
      hph = (grp & 1) ? PH - 1 - pi : pi;
    }
  };
  const uint32_t vbase = (uint32_t)lane * 16u;
  const uint32_t tile_bytes = I4 ? (uint32_t)(8 * H) : (uint32_t)(16 * H * (int)sizeof(typename W::T));
  auto load = [&](int st, const Step &d, LmBufs<W, NT> &bf) {
    const bool live = st < steps;
#pragma unroll
    for (int q = 0; q < TW; ++q) {
      const int kt = TW * d.k + q;   // the wave's tile number (past my_tiles: no access)
      const bool lq = live && kt < my_tiles;
      const size_t tile = (size_t)(first + (lq ? kt : 0) * stride);
      // descriptor over the tile's packed rows (rows past V were packed as zeros)
      const rsrc_t rs = make_rsrc(reinterpret_cast<const char *>(wlm) + tile * tile_bytes, tile_bytes);
#pragma unroll
      for (int j = 0; j < LB; ++j) {  // units past the phase or the stream: no access
        const int u = d.b * LB + j;
        bf.a[q][j] = buf_ld16(rs, lq && u < d.units(lph0, lsteps) ? vbase : kLmOutOfRange,
                              (uint32_t)min(d.u0(lph0) + u, lsteps - 1) * 1024u);
      }
      if constexpr (I4) {
        const rsrc_t rq = make_rsrc(scl + tile * (size_t)lsteps * 16, (uint32_t)lsteps * 32u);
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          const int u = d.b * LB + j;
          bf.sc[q][j] = buf_ld8(rq, lq && u < d.units(lph0, lsteps) ? (uint32_t)g * 8u : kLmOutOfRange,
                                (uint32_t)min(d.u0(lph0) + u, lsteps - 1) * 32u);
        }
      }
    }
  };
  f32x4 acc[TG][TW][NT];
#pragma unroll
  for (int i = 0; i < TG; ++i)
#pragma unroll
    for (int q = 0; q < TW; ++q)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[i][q][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one step's MFMAs into the accumulators of tile step i of the group
  auto mma_into = [&](f32x4 (&ac)[TW][NT], const Step &d, const LmBufs<W, NT> &bf) {
    if constexpr (I4) {
#pragma unroll
      for (int j = 0; j < LB; ++j) {
        const int grp = d.b * LB + j;   // the group within the phase
        if (grp >= d.units(lph0, lsteps)) break;
        f32x4 ag[TW][NT];
#pragma unroll
        for (int q = 0; q < TW; ++q)
#pragma unroll
          for (int n = 0; n < NT; ++n) ag[q][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          uint4 bv[NT];
#pragma unroll
          for (int n = 0; n < NT; ++n) bv[n] = xs[((grp * 4 + kk) * 4 + g) * TP + n * 16 + li];
#pragma unroll
          for (int q = 0; q < TW; ++q) {
            const uint4 &aq = bf.a[q][j];
            const uint4 e = i4_expand(kk == 0 ? aq.x : kk == 1 ? aq.y : kk == 2 ? aq.z : aq.w, kb);
#pragma unroll
            for (int n = 0; n < NT; ++n) ag[q][n] = mfma_bf16(e, bv[n], ag[q][n]);
          }
        }
        float off[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) off[n] = kI4Offset * hs[(d.u0(lph0) + grp) * TP + n * 16 + li];
#pragma unroll
        for (int q = 0; q < TW; ++q) {
          const uint2 sq = bf.sc[q][j];
          const float sr[4] = {bf_lo(sq.x), bf_hi(sq.x), bf_lo(sq.y), bf_hi(sq.y)};
#pragma unroll
          for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) ac[q][n][r] = fmaf(sr[r], ag[q][n][r] - off[n], ac[q][n][r]);
        }
      }
      return;
    }
    const uint4(&a)[LB] = bf.a[0];
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int ks = d.b * LB + j;   // the k-step within the phase
      if (ks >= d.units(lph0, lsteps)) break;
      const int c = ks * 4 + g;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const uint4 bv = xs[c * TP + n * 16 + li];
        if constexpr (std::is_same<W, WBf16>::value) {
          ac[0][n] = mfma_bf16(a[j], bv, ac[0][n]);
        } else {
          ac[0][n] = mfma_f32(__uint_as_float(a[j].x), __uint_as_float(bv.x), ac[0][n]);
          ac[0][n] = mfma_f32(__uint_as_float(a[j].y), __uint_as_float(bv.y), ac[0][n]);
          ac[0][n] = mfma_f32(__uint_as_float(a[j].z), __uint_as_float(bv.z), ac[0][n]);
          ac[0][n] = mfma_f32(__uint_as_float(a[j].w), __uint_as_float(bv.w), ac[0][n]);
        }
      }
    }
  };
  // epilogue of a finished tile step: lane holds rows row0 + 4g + r (r =
  // 0..3) of column li + 16n; fold them into the running (max, sum, argmax)
  auto fold = [&](f32x4 (&ac)[TW][NT], int k) {
#pragma unroll
    for (int q = 0; q < TW; ++q) {
    // (a tile past the wave's last has row0 >= V: it folds nothing)
    const int row0 = (first + (TW * k + q) * stride) * 16;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float tmax = -FLT_MAX;
      int targ = INT_MAX;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = row0 + 4 * g + r;
        if (v < V && (targ == INT_MAX || ac[q][n][r] > tmax)) { tmax = ac[q][n][r]; targ = v; }
      }
      {
        const float m2 = partner_f32<16>(tmax, lane);
        const int a2 = partner_i32<16>(targ, lane);
        if (a2 != INT_MAX && (targ == INT_MAX || m2 > tmax || (m2 == tmax && a2 < targ))) {
          tmax = m2;
          targ = a2;
        }
      }
      {
        const float m2 = partner_f32<32>(tmax, lane);
        const int a2 = partner_i32<32>(targ, lane);
        if (a2 != INT_MAX && (targ == INT_MAX || m2 > tmax || (m2 == tmax && a2 < targ))) {
          tmax = m2;
          targ = a2;
        }
      }
      float tsum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = row0 + 4 * g + r;
        if (v < V) tsum += __expf(ac[q][n][r] - tmax);
      }
      tsum += partner_f32<16>(tsum, lane);
      tsum += partner_f32<32>(tsum, lane);
      sm_merge(m[n], s[n], am[n], tmax, tsum, targ);
      ac[q][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    }
  };
  // a step's MFMAs (into the accumulators of its tile step in the group)
  auto run = [&](const Step &d, const LmBufs<W, NT> &bf) {
#pragma unroll
    for (int i = 0; i < TG; ++i)
      if (d.kin == i) mma_into(acc[i], d, bf);
  };
  // Phased staging: one wave instruction gathers chunk c of the half into
  // xs[c][*] straight from memory (lane t: position t, 16 bytes; positions
  // past T read as zeros), so no registers hold the block while the weight
  // loads stay in flight.
  const rsrc_t rh = make_rsrc(hhat, (uint32_t)(T * H) * (uint32_t)sizeof(typename W::T));
  auto stage_half = [&](int hph) {
    const uint32_t vo = lane < T ? (uint32_t)lane * (uint32_t)H * (uint32_t)sizeof(typename W::T) : kLmOutOfRange;
    const int nc = (hph ? lsteps - lph0 : lph0) * cpu;
    for (int c = wave; c < nc; c += kLmWaves)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rh, (__attribute__((address_space(3))) void *)(xs + c * TP), 16, (int)vo,
          (int)((uint32_t)((hph * NCP + c) * CH) * (uint32_t)sizeof(typename W::T)), 0, 0);
    __builtin_amdgcn_s_waitcnt(0);   // (the lgkm/vm counts: the gathers have landed)
  };

  Step cc = {0, 0, 0, 0, 0, 0}, cl = cc;   // compute and load cursors
  LmBufs<W, NT> a0, a1;
  load(0, cl, a0);
  cl.next(nb);
  load(1, cl, a1);
  cl.next(nb);
  if constexpr (PH == 1) {
    // stage the block: batches of 8 independent loads per thread
    for (int base = tid; base < TP * NC; base += 8 * (int)blockDim.x) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int idx = base + j * (int)blockDim.x;
        const int t = idx / NC, c = idx - t * NC;
        v[j] = (idx < TP * NC && t < T) ? ld16(hhat + (size_t)t * H + (size_t)c * CH) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int idx = base + j * (int)blockDim.x;
        const int t = idx / NC, c = idx - t * NC;
        if (idx < TP * NC) xs[c * TP + t] = v[j];
      }
    }
  } else {
    stage_half(0);
  }
  if constexpr (I4) {
    // per (group, position): the sum of the group's 128 values of h, from
    // the staged block, or with phases (the staged block holds half of H)
    // from memory, its 16 loads in flight together; the same sum order
    if constexpr (PH == 1) __syncthreads();
    for (int idx = tid; idx < (H / kI4Group) * TP; idx += (int)blockDim.x) {
      const int grp = idx / TP, t = idx - grp * TP;
      float sum = 0.f;
      if constexpr (PH == 1) {
        for (int c = grp * (kI4Group / 8); c < (grp + 1) * (kI4Group / 8); ++c) {
          float f[8];
          unpack8(xs[c * TP + t], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) sum += f[e];
        }
      } else if (t < T) {
        uint4 v[kI4Group / 8];
#pragma unroll
        for (int c = 0; c < kI4Group / 8; ++c) v[c] = ld16(hhat + (size_t)t * H + (size_t)(grp * (kI4Group / 8) + c) * 8);
#pragma unroll
        for (int c = 0; c < kI4Group / 8; ++c) {
          float f[8];
          unpack8(v[c], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) sum += f[e];
        }
      }
      hs[idx] = sum;
    }
  }
  __syncthreads();
  // A buffer is refilled as soon as its MFMAs have read it, before a tile's
  // epilogue, so two batches stay in flight through the epilogue.  Loads past
  // the last step are out of range (no access): the loop always has the same
  // loads in flight and the compiler's in-order wait counts stay exact.
  // After a step: the tile step's epilogue after its last batch of the
  // group's second phase, or the restage after the group's first phase (the
  // same step in every wave).
  auto after = [&](const Step &d) {
    if (d.b != nb - 1) return;
    if (d.second()) {
#pragma unroll
      for (int i = 0; i < TG; ++i)
        if (d.kin == i) fold(acc[i], d.k);
    } else {
      if constexpr (PH > 1) {
        if (d.kin == TG - 1) {
          __syncthreads();   // every wave is done with the staged half
          stage_half(1 - d.hph);
          __syncthreads();
        }
      }
    }
  };
  // Always two steps per trip (an odd count runs one step past the end: its
  // loads were out of range, so its MFMAs add zeros, and a tile past the
  // wave's last folds nothing).  An exit between the two steps would join
  // the loop's load-count state with the exit path's, and the compiler then
  // waits at the first step for the second buffer's loads as well: one batch
  // in flight instead of two.
  for (int st = 0; st < steps; st += 2) {
    run(cc, a0);
    load(st + 2, cl, a0);
    cl.next(nb);
    after(cc);
    cc.next(nb);
    run(cc, a1);
    load(st + 3, cl, a1);
    cl.next(nb);
    after(cc);
    cc.next(nb);
  }

  if (lane < 16) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      sm[wave][n * 16 + lane] = m[n];
      ssum[wave][n * 16 + lane] = s[n];
      si[wave][n * 16 + lane] = am[n];
    }
  }
  __syncthreads();
  if (tid < T) {
    float mm = -FLT_MAX, ss = 0.f;
    int ii = INT_MAX;
    for (int w = 0; w < kLmWaves; ++w) sm_merge(mm, ss, ii, sm[w][tid], ssum[w][tid], si[w][tid]);
    publish(part_m + (size_t)tid * gridDim.x + blockIdx.x, mm);
    publish(part_s + (size_t)tid * gridDim.x + blockIdx.x, ss);
    publish(part_i + (size_t)tid * gridDim.x + blockIdx.x, ii);
  }
  if (done_count == nullptr) return;
  __shared__ int s_last;
  __syncthreads();   // the published partials are ordered before the count
  if (tid == 0) s_last = count_done_last(done_count, (int)gridDim.x);
  __syncthreads();   // the last workgroup's waves read after its acquire
  if (!s_last) return;
  commit_block(part_m, part_s, part_i, gridDim.x, T, threshold, tokens, conf, choice, round_info, resolved_flag);
  if (tid == 0) publish(done_count, 0);
}

// Packs w_lm [V][H] into the tile layout the LM-head kernel streams: for
// tile tau (rows 16 tau .. 16 tau + 15) and MFMA k-step s, a contiguous
// 16-byte-per-lane block where lane l = li + 16 g holds row 16 tau + li,
// elements [s*KS + g*CH, s*KS + g*CH + CH) (KS = 4 CH: 32 for bf16, 16 for
// fp32).  Rows past V are zero.  One thread per 16-byte unit.
template <class W>
__global__ __launch_bounds__(256) void pack_lm_kernel(const typename W::T *__restrict__ w, int V, int H,
                                                      uint4 *__restrict__ out, long long units) {
  constexpr int CH = W::kChunk;
  const int S = H / (4 * CH);
  for (long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x; u < units;
       u += (long long)gridDim.x * blockDim.x) {
    const int l = (int)(u & 63);
    const long long blk = u >> 6;
    const long long tau = blk / S;
    const int st = (int)(blk - tau * S);
    const long long row = tau * 16 + (l & 15);
    const int k0 = st * 4 * CH + (l >> 4) * CH;
    out[u] = row < V ? ld16(w + row * H + k0) : make_uint4(0, 0, 0, 0);
  }
}

// 4-bit LM head: codes [V][H / 2] (column 2j in the low nibble of byte j) and
// scales [V][H / 128] bf16 into the layout described at WI4: one thread per
// 16-byte unit (tile tau, group grp, lane l); the lanes with g = 0 also place
// the unit's 16 scales.  Rows past V get zero codes and zero scales.
__global__ __launch_bounds__(256) void pack_lm_i4_kernel(const uint8_t *__restrict__ codes,
                                                         const uint16_t *__restrict__ scales, int V, int H,
                                                         uint4 *__restrict__ out, uint16_t *__restrict__ sout,
                                                         long long units) {
  const int G = H / kI4Group;
  for (long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x; u < units;
       u += (long long)gridDim.x * blockDim.x) {
    const int l = (int)(u & 63), li = l & 15, g = l >> 4;
    const long long blk = u >> 6;
    const long long tau = blk / G;
    const int grp = (int)(blk - tau * G);
    const long long row = tau * 16 + li;
    uint32_t d[4] = {0u, 0u, 0u, 0u};
    if (row < V) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint8_t *src = codes + row * (H / 2) + ((grp * 4 + kk) * 32 + 8 * g) / 2;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t byte = src[b];
          d[kk] |= (byte & 15u) << (4 * b) | (byte >> 4) << (16 + 4 * b);
        }
      }
    }
    out[u] = make_uint4(d[0], d[1], d[2], d[3]);
    if (g == 0) sout[blk * 16 + li] = row < V ? scales[row * G + grp] : (uint16_t)0;
  }
}

size_t lmhead_packed_bytes(int wdtype, int H, int V) {
  const size_t tiles = (size_t)((V + 15) / 16);
  if (wdtype == 2) return tiles * (size_t)(8 * H) + tiles * (size_t)(H / kI4Group) * 32;
  return tiles * 16 * H * (wdtype == 1 ? 2 : 4);
}

hipError_t launch_pack_lm_int4(const void *codes, const void *scales, int V, int H, void *packed,
                               hipStream_t s) {
  const size_t tiles = (size_t)((V + 15) / 16);
  const long long units = (long long)(tiles * (size_t)(8 * H) / 16);
  const int grid = (int)((units + 255) / 256 < 65536 ? (units + 255) / 256 : 65536);
  pack_lm_i4_kernel<<<grid, 256, 0, s>>>((const uint8_t *)codes, (const uint16_t *)scales, V, H,
                                         (uint4 *)packed,
                                         (uint16_t *)((char *)packed + tiles * (size_t)(8 * H)), units);
  return hipGetLastError();
}

hipError_t launch_pack_lm(int wdtype, const void *w_lm, int V, int H, void *packed, hipStream_t s) {
  const long long units = (long long)(lmhead_packed_bytes(wdtype, H, V) / 16);
  const int grid = (int)((units + 255) / 256 < 65536 ? (units + 255) / 256 : 65536);
  if (wdtype == 1)
    pack_lm_kernel<WBf16><<<grid, 256, 0, s>>>((const bf16_t *)w_lm, V, H, (uint4 *)packed, units);
  else
    pack_lm_kernel<WF32><<<grid, 256, 0, s>>>((const float *)w_lm, V, H, (uint4 *)packed, units);
  return hipGetLastError();
}

// One workgroup per CU at most; with m = ceil(tiles / (waves of the chip))
// tiles per wave, the grid shrinks to ceil(tiles / (kLmWaves * m)) so that
// every wave streams m tiles (or m - 1 in the last workgroup) and none idles
// through the last round.
int lmhead_grid(int cus, int V) {
  const int tiles = (V + 15) / 16;
  const int m = (tiles + cus * kLmWaves - 1) / (cus * kLmWaves);
  const int g = (tiles + kLmWaves * m - 1) / (kLmWaves * m);
  return g < cus ? g : cus;
}

size_t lmhead_lds_bytes(int wdtype, int T, int H) {
  // (above 32 positions the staged block holds the first ceil(units / 2)
  // load units' columns: two phases)
  const int tp = T <= 16 ? 16 : T <= 32 ? 32 : 64;
  const int ph = T <= 32 ? 1 : 2;
  const int ch = wdtype == 0 ? 4 : 8;
  const int unit_cols = wdtype == 2 ? kI4Group : 4 * ch;    // columns of one load unit
  const int units = H / unit_cols;
  const size_t chunks = (size_t)((units + ph - 1) / ph) * (unit_cols / ch);
  return chunks * tp * 16 + (wdtype == 2 ? (size_t)(H / kI4Group) * tp * 4 : 0);
}

template <typename F>
static hipError_t allow_lds(F *fn, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <class W, int NT>
static hipError_t lmhead_launch(const void *hhat, const void *w_lm, int T, int H, int V, float *pm,
                                float *ps, int32_t *pi, int grid, const LmCommit *fused, hipStream_t s) {
  typedef typename W::T WT;
  constexpr int dt = std::is_same<W, WI4>::value ? 2 : std::is_same<W, WBf16>::value ? 1 : 0;
  const size_t lds = lmhead_lds_bytes(dt, T, H);
  hipError_t err = allow_lds(lmhead_kernel<W, NT>, lds);
  if (err != hipSuccess) return err;
  // 4-bit heads: the scales follow the codes in the packed buffer
  const uint16_t *scl =
      dt == 2 ? (const uint16_t *)((const char *)w_lm + (size_t)((V + 15) / 16) * (size_t)(8 * H)) : nullptr;
  lmhead_kernel<W, NT><<<grid, 1024, lds, s>>>(
      (const WT *)hhat, (const WT *)w_lm, scl, T, H, V, pm, ps, pi, fused ? fused->done_count : nullptr,
      fused ? fused->threshold : 0.f, fused ? fused->tokens : nullptr, fused ? fused->conf : nullptr,
      fused ? fused->choice : nullptr, fused ? fused->round_info : nullptr, fused ? fused->gate : nullptr,
      fused ? fused->resolved_flag : nullptr);
  return hipGetLastError();
}

hipError_t launch_lmhead(int wdtype, const void *hhat, const void *w_lm, int T, int H, int V,
                         float *part_m, float *part_s, int32_t *part_i, int grid, const LmCommit *fused,
                         hipStream_t s) {
  // one, two or four 16-position column tiles (four: the block staged half
  // of H at a time)
  if (wdtype == 2)
    return T <= 16   ? lmhead_launch<WI4, 1>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s)
           : T <= 32 ? lmhead_launch<WI4, 2>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s)
                     : lmhead_launch<WI4, 4>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s);
  if (wdtype == 1)
    return T <= 16   ? lmhead_launch<WBf16, 1>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s)
           : T <= 32 ? lmhead_launch<WBf16, 2>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s)
                     : lmhead_launch<WBf16, 4>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s);
  return T <= 16   ? lmhead_launch<WF32, 1>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s)
         : T <= 32 ? lmhead_launch<WF32, 2>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s)
                   : lmhead_launch<WF32, 4>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s);
}

hipError_t launch_block_start(int32_t *tokens, int T, int32_t *info, int words, int32_t *flag, hipStream_t s) {
  block_start_kernel<<<1, 256, 0, s>>>(tokens, T, info, words, flag);
  return hipGetLastError();
}

hipError_t launch_commit(const float *part_m, const float *part_s, const int32_t *part_i,
                         int nparts, int T, float threshold, int32_t *tokens, float *conf,
                         int32_t *choice, int32_t *round_info, hipStream_t s, const int32_t *gate,
                         int32_t *resolved_flag) {
  commit_kernel<<<1, 1024, 0, s>>>(part_m, part_s, part_i, nparts, T, threshold, tokens, conf,
                                   choice, round_info, gate, resolved_flag);
  return hipGetLastError();
}

}  // namespace bdd
