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
// units per tile per load batch, and tiles a wave streams side by side: a
// 4-bit wave works on two tiles at once, so every block operand it reads from
// LDS feeds both tiles' MFMAs (a bf16 tile is HBM-bound on its own)
template <class W>
constexpr int lm_batch() { return std::is_same<W, WI4>::value ? 2 : 8; }
template <class W>
constexpr int lm_tiles() { return std::is_same<W, WI4>::value ? 2 : 1; }
template <class W>
struct LmBufs {
  uint4 a[lm_tiles<W>()][lm_batch<W>()];
  uint2 sc[lm_tiles<W>()][std::is_same<W, WI4>::value ? lm_batch<W>() : 1];
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
// acquire-release counter over partials published as agent-scope atomics)
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
  constexpr int LB = lm_batch<W>();
  constexpr int TW = lm_tiles<W>();
  const int ntiles = (V + 15) / 16;
  const int ksteps = NC / 4;                    // MFMA k-steps per tile
  const int lsteps = I4 ? ksteps / 4 : ksteps;  // KiB load units per tile
  const int nb = (lsteps + LB - 1) / LB;
  float *hs = reinterpret_cast<float *>(xs + NC * TP);   // [H / 128][16 NT]: group sums of h (WI4)
  const int first = uniform(wave * (int)gridDim.x + (int)blockIdx.x);
  const int stride = gridDim.x * kLmWaves;
  const int my_tiles = first < ntiles ? (ntiles - 1 - first) / stride + 1 : 0;
  const int steps = (my_tiles + TW - 1) / TW * nb;   // TW tiles per step sequence
  const uint32_t vbase = (uint32_t)lane * 16u;
  const uint32_t tile_bytes = I4 ? (uint32_t)(8 * H) : (uint32_t)(16 * H * (int)sizeof(typename W::T));
  auto load = [&](int st, LmBufs<W> &bf) {
    const bool live = st < steps;
    const int k = live ? st / nb : 0, b = st - (st / nb) * nb;
#pragma unroll
    for (int q = 0; q < TW; ++q) {
      const int kt = TW * k + q;   // the wave's tile number (past my_tiles: no access)
      const bool lq = live && kt < my_tiles;
      const size_t tile = (size_t)(first + (lq ? kt : 0) * stride);
      // descriptor over the tile's packed rows (rows past V were packed as zeros)
      const rsrc_t rs = make_rsrc(reinterpret_cast<const char *>(wlm) + tile * tile_bytes, tile_bytes);
#pragma unroll
      for (int j = 0; j < LB; ++j)   // units past the tile or the stream: no access
        bf.a[q][j] = buf_ld16(rs, lq && b * LB + j < lsteps ? vbase : kLmOutOfRange,
                              (uint32_t)min(b * LB + j, lsteps - 1) * 1024u);
      if constexpr (I4) {
        const rsrc_t rq = make_rsrc(scl + tile * (size_t)lsteps * 16, (uint32_t)lsteps * 32u);
#pragma unroll
        for (int j = 0; j < LB; ++j)
          bf.sc[q][j] = buf_ld8(rq, lq && b * LB + j < lsteps ? (uint32_t)g * 8u : kLmOutOfRange,
                                (uint32_t)min(b * LB + j, lsteps - 1) * 32u);
      }
    }
  };
  f32x4 acc[TW][NT];
#pragma unroll
  for (int q = 0; q < TW; ++q)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[q][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](int st, const LmBufs<W> &bf) {
    const int b = st % nb;
    if constexpr (I4) {
#pragma unroll
      for (int j = 0; j < LB; ++j) {
        const int grp = b * LB + j;
        if (grp >= lsteps) break;
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
        for (int n = 0; n < NT; ++n) off[n] = kI4Offset * hs[grp * TP + n * 16 + li];
#pragma unroll
        for (int q = 0; q < TW; ++q) {
          const uint2 sq = bf.sc[q][j];
          const float sr[4] = {bf_lo(sq.x), bf_hi(sq.x), bf_lo(sq.y), bf_hi(sq.y)};
#pragma unroll
          for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[q][n][r] = fmaf(sr[r], ag[q][n][r] - off[n], acc[q][n][r]);
        }
      }
      return;
    }
    const uint4(&a)[LB] = bf.a[0];
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int ks = b * LB + j;
      if (ks >= ksteps) break;
      const int c = ks * 4 + g;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const uint4 bv = xs[c * TP + n * 16 + li];
        if constexpr (std::is_same<W, WBf16>::value) {
          acc[0][n] = mfma_bf16(a[j], bv, acc[0][n]);
        } else {
          acc[0][n] = mfma_f32(__uint_as_float(a[j].x), __uint_as_float(bv.x), acc[0][n]);
          acc[0][n] = mfma_f32(__uint_as_float(a[j].y), __uint_as_float(bv.y), acc[0][n]);
          acc[0][n] = mfma_f32(__uint_as_float(a[j].z), __uint_as_float(bv.z), acc[0][n]);
          acc[0][n] = mfma_f32(__uint_as_float(a[j].w), __uint_as_float(bv.w), acc[0][n]);
        }
      }
    }
  };
  // epilogue of a finished tile: lane holds rows row0 + 4g + r (r = 0..3) of
  // column li + 16n; fold them into the running (max, sum, argmax)
  auto epilogue = [&](int st) {
#pragma unroll
    for (int q = 0; q < TW; ++q) {
    // (a tile past the wave's last has row0 >= V: it folds nothing)
    const int row0 = (first + (TW * (st / nb) + q) * stride) * 16;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float tmax = -FLT_MAX;
      int targ = INT_MAX;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = row0 + 4 * g + r;
        if (v < V && (targ == INT_MAX || acc[q][n][r] > tmax)) { tmax = acc[q][n][r]; targ = v; }
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
        if (v < V) tsum += __expf(acc[q][n][r] - tmax);
      }
      tsum += partner_f32<16>(tsum, lane);
      tsum += partner_f32<32>(tsum, lane);
      sm_merge(m[n], s[n], am[n], tmax, tsum, targ);
      acc[q][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    }
  };

  LmBufs<W> a0, a1;
  load(0, a0);
  load(1, a1);
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
  __syncthreads();
  if constexpr (I4) {
    // per (group, position): the sum of the group's 128 values of h
    for (int idx = tid; idx < (H / kI4Group) * TP; idx += (int)blockDim.x) {
      const int grp = idx / TP, t = idx - grp * TP;
      float sum = 0.f;
      for (int c = grp * (kI4Group / 8); c < (grp + 1) * (kI4Group / 8); ++c) {
        float f[8];
        unpack8(xs[c * TP + t], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += f[e];
      }
      hs[idx] = sum;
    }
    __syncthreads();
  }
  // A buffer is refilled as soon as its MFMAs have read it, before a tile's
  // epilogue, so two batches stay in flight through the epilogue.  Loads past
  // the last step are out of range (no access): the loop always has the same
  // loads in flight and the compiler's in-order wait counts stay exact.
  for (int st = 0; st < steps; st += 2) {
    mma(st, a0);
    load(st + 2, a0);
    if (st % nb == nb - 1) epilogue(st);
    if (st + 1 >= steps) break;
    mma(st + 1, a1);
    load(st + 3, a1);
    if ((st + 1) % nb == nb - 1) epilogue(st + 1);
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
  if (tid == 0) s_last = count_done(done_count) == (int)gridDim.x - 1;
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
  const int tp = T <= 16 ? 16 : 32;
  const int ch = wdtype == 0 ? 4 : 8;
  return (size_t)(H / ch) * tp * 16 + (wdtype == 2 ? (size_t)(H / kI4Group) * tp * 4 : 0);
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
  if (T > 32) {
    // two passes over the vocabulary, positions 0..31 and 32..T-1 (partials
    // [T][grid]: the second pass writes rows 32..), then the commit
    const LmCommit gate_only = {nullptr, 0.f, nullptr, nullptr, nullptr, nullptr, fused ? fused->gate : nullptr,
                                nullptr};
    const size_t es = wdtype == 0 ? 4 : 2;
    const size_t off = (size_t)32 * grid;
    hipError_t err = launch_lmhead(wdtype, hhat, w_lm, 32, H, V, part_m, part_s, part_i, grid, &gate_only, s);
    if (err != hipSuccess) return err;
    err = launch_lmhead(wdtype, static_cast<const char *>(hhat) + (size_t)32 * H * es, w_lm, T - 32, H, V,
                        part_m + off, part_s + off, part_i + off, grid, &gate_only, s);
    if (err != hipSuccess || !fused || !fused->done_count) return err;
    return launch_commit(part_m, part_s, part_i, grid, T, fused->threshold, fused->tokens, fused->conf,
                         fused->choice, fused->round_info, s, fused->gate, fused->resolved_flag);
  }
  if (wdtype == 2)
    return T <= 16 ? lmhead_launch<WI4, 1>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s)
                   : lmhead_launch<WI4, 2>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s);
  if (wdtype == 1)
    return T <= 16 ? lmhead_launch<WBf16, 1>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s)
                   : lmhead_launch<WBf16, 2>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s);
  return T <= 16 ? lmhead_launch<WF32, 1>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s)
                 : lmhead_launch<WF32, 2>(hhat, w_lm, T, H, V, part_m, part_s, part_i, grid, fused, s);
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
