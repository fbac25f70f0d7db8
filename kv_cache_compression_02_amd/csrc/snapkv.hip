// SnapKV prompt-KV selection and compaction on gfx950.
//
// The method (abeam.tech summary of "SnapKV: LLM Knows What You are Looking
// for Before Generation", section 技術の仕組み › 処理の流れ, steps 1-4): the last
// `w` prompt queries attend to the prompt; for every prefix position the
// softmax weights it receives from those queries are summed per head (the
// vote); the votes are smoothed by a 1D max-pool; each head keeps its
// top-scoring prefix positions and their K/V rows are concatenated with the
// window's own rows.
//
// Kernel sequence per call (all on the caller's stream, no host sync). Two
// score schedules share the selection and the gather:
//
// single pass (bf16, the default where it runs):
//   snap_coop_prep   per head: clear the workspace state; each window row's
//                    reference score R_i (its largest score against the
//                    window keys it sees) from one wave of MFMA
//   snap_wave_bf16   persistent grid of independent waves over 32-key tiles:
//                    MFMA scores, e_ij = 2^(s_ij - R_i) kept in registers,
//                    row sums merged exactly in fixed point across the grid,
//                    votes once the head's normaliser is published (K read
//                    once); snap_coop_bf16 is the lockstep form for shorter
//                    heads
//   snap_pool        max-pool of the votes and the per-head 12-bit histogram
//                    of pooled scores (exact votes recomputed first for any
//                    head the score kernel flagged, or every head if its
//                    status word reports a wait that ran out)
// two passes (fp32, or where the single pass cannot run):
//   snap_stats_*     per chunk of keys: each window row's max and sum of
//                    2^(s - m) (softmax pass 1); clears the counters
//   snap_stats_merge each row's (max, 1/sum) from the chunk partials
//   snap_votes_*     scores again, normalised and summed over the window rows
//                    (pass 2), max-pooled in LDS with a recomputed halo, and
//                    the histogram of pooled scores
// then, for both:
//   snap_select      per head: the histogram bin holding the k-th largest
//                    pooled score; positions above it go straight to a
//                    bitmap, the bin's members are ranked by (score desc,
//                    position asc); the head's last workgroup compacts the
//                    bitmap into ascending positions (pooling the raw votes
//                    itself for radii up to 4 under the single pass);
//                    snap_select_head does the same in one workgroup per
//                    head for heads of at most 16384 prefix positions
//   snap_gather      copy the kept K/V rows and the window rows to the outputs
//
// Scores live in the base-2 domain: s2 = (q.k) * log2(e)/sqrt(D), so the
// softmax is 2^(s2 - m2) / sum; it equals exp(s - m)/sum exactly in real
// arithmetic.
#include <math.h>

#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>
#include <tuple>
#include <utility>

#include "common.hpp"

namespace kvc {
namespace {

constexpr int kTile = 32;            // keys per MFMA tile (the 32x32 output's N or M side)
constexpr int kThreads = 256;        // workgroup size of the streaming kernels
constexpr int kWaves = kThreads / kWave;
constexpr int kChunkMfma = 2048;     // keys per workgroup, bf16 MFMA vote pass
constexpr int kStatChunkMfma = 2048; // keys per workgroup, bf16 MFMA statistics pass
constexpr int kChunkF32 = 256;       // keys per workgroup, fp32 path (a key per thread)
constexpr int kMaxWindow = 32;
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 19;       // pooled >= 0: bits 30..19 = exponent + 4 mantissa bits
constexpr int kMaxPoolRadius = 32;
constexpr int kSelCtrWords = 3;     // per head: candidates listed, selection workgroups finished,
                                    // selection workgroups whose histogram is in (single pass)
constexpr float kNegBig = -1.0e30f;  // "no score" sentinel: 2^(kNegBig - m) == 0

// ------------------------------------------------------------------ loaders

// The lane's contiguous half row: elements [half*D/2, half*D/2 + D/2) as D/16
// MFMA k-step fragments of 8 bf16. The contraction index is permuted the same
// way for Q and K, so the dot product is unchanged while each lane reads one
// contiguous 64/128-byte run. Plain loads, also for keys streamed once: a
// row's cache lines are read by D/16 separate instructions of the wave, and
// with the nontemporal bit they were evicted between those reads (the two
// score passes then fetched 23-28% more than K and ran 2.4x slower).
template <int D>
__device__ __forceinline__ void load_half_row(const uint16_t* p, bf16x8_t (&f)[D / 16]) {
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = __builtin_bit_cast(bf16x8_t, src[s]);
}


template <int D>
__device__ __forceinline__ void zero_frag(bf16x8_t (&f)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = __builtin_bit_cast(bf16x8_t, u32x4_t{0, 0, 0, 0});
}

// Row m of the 32x32 MFMA accumulator held in register r of a lane in half `half`.
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// ------------------------------------------------------- row-stat merging

// Clear one head's histogram and selection counters (run by the statistics
// pass; the kernels that fill them start after it has finished).
__device__ __forceinline__ void clear_head(unsigned* hist, unsigned* sel_ctr, int bh) {
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) hist[static_cast<int64_t>(bh) * kHistBins + i] = 0;
  if (threadIdx.x < kSelCtrWords) sel_ctr[bh * kSelCtrWords + threadIdx.x] = 0;
}

// Merge the per-chunk partials (m, l) of the 32 window rows of head bh into
// st[row] = (m2, 1/l) in LDS. Every thread of the block calls it; the loads
// of a batch are in flight together.
__device__ void merge_stats_to_lds(int bh, int nchunk, const float2* __restrict__ part, float2* st) {
  constexpr int kGroups = kThreads / 32;
  constexpr int kBatch = 8;
  __shared__ float2 red[kGroups][32];
  const int row = threadIdx.x & 31, grp = threadIdx.x >> 5;
  float m = kNegBig, l = 0.f;
  const float2* pb = part + static_cast<int64_t>(bh) * nchunk * 32;
  for (int c0 = grp; c0 < nchunk; c0 += kBatch * kGroups) {
    float2 pp[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = c0 + i * kGroups;
      pp[i] = c < nchunk ? pb[c * 32 + row] : make_float2(kNegBig, 0.f);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) lse2_merge(m, l, pp[i].x, pp[i].y);
  }
  red[grp][row] = make_float2(m, l);
  __syncthreads();
  if (threadIdx.x < 32) {
    float mm = red[0][row].x, ll = red[0][row].y;
#pragma unroll
    for (int g = 1; g < kGroups; ++g) lse2_merge(mm, ll, red[g][row].x, red[g][row].y);
    st[row] = make_float2(mm, 1.f / ll);
  }
  __syncthreads();
}

// Each window row's (m2, 1/l) of head blockIdx.x from its per-chunk partials,
// once per head between the two passes.
__global__ __launch_bounds__(kThreads) void snap_stats_merge(const float2* __restrict__ part, int nchunk,
                                                             float2* __restrict__ rowstat) {
  __shared__ float2 st[32];
  merge_stats_to_lds(blockIdx.x, nchunk, part, st);
  if (threadIdx.x < 32) rowstat[blockIdx.x * 32 + threadIdx.x] = st[threadIdx.x];
}

// Max-pool and histogram of one chunk: sv holds the votes of prefix keys
// [e0, e1) = [c0 - r, c1 + r) clipped to [0, t0); pooled[j] for j in [c0, c1)
// is the max over the neighbours that exist, and each pooled value's top 12
// bits are counted in the LDS histogram sh (merged into hist by the caller).
__device__ void pool_and_count(const float* sv, int e0, int e1, int c0, int c1, int r, int avg, float* pooled_row,
                               unsigned* sh) {
  for (int j = c0 + static_cast<int>(threadIdx.x); j < c1; j += kThreads) {
    // the in-range neighbours j-r .. j+r (e0 and e1 clip at the prefix's ends)
    const int lo = max(j - r, e0) - e0, hi = min(j + r, e1 - 1) - e0;
    float m = sv[lo];
    if (avg) {  // their mean, summed in position order
      for (int d = lo + 1; d <= hi; ++d) m += sv[d];
      m /= static_cast<float>(hi - lo + 1);
    } else {  // their maximum
      for (int d = lo + 1; d <= hi; ++d) m = fmaxf(m, sv[d]);
    }
    pooled_row[j] = m;
    atomicAdd(&sh[(__float_as_uint(m) >> kHistShift) & (kHistBins - 1)], 1u);
  }
}

__device__ void flush_hist(const unsigned* sh, unsigned* hist_row) {
  for (int i = threadIdx.x; i < kHistBins; i += static_cast<int>(blockDim.x))
    if (sh[i]) atomicAdd(&hist_row[i], sh[i]);
}

// ------------------------------------------------ pass 1: row statistics

// bf16, MFMA 32x32x16. Output orientation S^T: M = keys of the tile, N = the 32
// window queries, so each lane owns one query (lane & 31) and 16 keys, and the
// per-query running (max, sum) stays in registers.
template <int D>
__global__ __launch_bounds__(kThreads) void snap_stats_bf16(
    const uint16_t* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qst, int qrow0,
    const uint16_t* __restrict__ k, int64_t ksb, int64_t ksh, int64_t kst, int H, int L, int w,
    int nchunk, float scale_log2, float2* __restrict__ part, unsigned* __restrict__ hist,
    unsigned* __restrict__ sel_ctr) {
  constexpr int KS = D / 16;
  const int chunk = blockIdx.x, bh = blockIdx.y;
  if (chunk == 0) clear_head(hist, sel_ctr, bh);
  const int b = bh / H, h = bh - b * H;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int col = lane & 31, half = lane >> 5;
  const int t0 = L - w;

  bf16x8_t qf[KS];
  if (col < w)
    load_half_row<D>(q + b * qsb + h * qsh + static_cast<int64_t>(qrow0 + col) * qst + half * (D / 2), qf);
  else
    zero_frag<D>(qf);

  const uint16_t* kb = k + b * ksb + h * ksh + half * (D / 2);
  const int key0 = chunk * kStatChunkMfma;
  const int key1 = min(L, key0 + kStatChunkMfma);
  constexpr int kStep = kWaves * kTile;
  float m_run = kNegBig, l_run = 0.f;

  int tile = key0 + wave * kTile;
  bf16x8_t kf[KS];
  if (tile < key1) load_half_row<D>(kb + static_cast<int64_t>(min(tile + col, L - 1)) * kst, kf);
  for (; tile < key1; tile += kStep) {
    bf16x8_t kn[KS];
    const int nt = tile + kStep;
    if (nt < key1) load_half_row<D>(kb + static_cast<int64_t>(min(nt + col, L - 1)) * kst, kn);
    f32x16_t acc = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], acc, 0, 0, 0);
    float sv[16];
    float tmax = kNegBig;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = tile + acc_row(r, half);
      const bool vis = (j < L) && (j <= t0 + col);  // query col sits at position t0 + col
      sv[r] = vis ? acc[r] * scale_log2 : kNegBig;
      tmax = fmaxf(tmax, sv[r]);
    }
    const float mnew = fmaxf(m_run, tmax);
    float add = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) add += fast_exp2(sv[r] - mnew);
    l_run = l_run * fast_exp2(m_run - mnew) + add;
    m_run = mnew;
    if (nt < key1) {
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[s] = kn[s];
    }
  }
  // lanes col and col+32 hold the same query
  lse2_merge(m_run, l_run, lane_xor<32>(m_run), lane_xor<32>(l_run));
  __shared__ float2 wred[kWaves][32];
  if (half == 0) wred[wave][col] = make_float2(m_run, l_run);
  __syncthreads();
  if (threadIdx.x < 32) {
    float m = wred[0][threadIdx.x].x, l = wred[0][threadIdx.x].y;
#pragma unroll
    for (int i = 1; i < kWaves; ++i) lse2_merge(m, l, wred[i][threadIdx.x].x, wred[i][threadIdx.x].y);
    part[(static_cast<int64_t>(bh) * nchunk + chunk) * 32 + threadIdx.x] = make_float2(m, l);
  }
}

// fp32, VALU: one key per thread, the window rows in LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void snap_stats_f32(
    const float* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qst, int qrow0,
    const float* __restrict__ k, int64_t ksb, int64_t ksh, int64_t kst, int H, int L, int w,
    int nchunk, float scale_log2, float2* __restrict__ part, unsigned* __restrict__ hist,
    unsigned* __restrict__ sel_ctr) {
  __shared__ float qs[kMaxWindow][D];
  __shared__ float ss[kMaxWindow][kThreads + 1];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  if (chunk == 0) clear_head(hist, sel_ctr, bh);
  const int b = bh / H, h = bh - b * H;
  const int t0 = L - w;
  for (int i = threadIdx.x; i < kMaxWindow * D; i += kThreads) {
    const int r = i / D, d = i - r * D;
    qs[r][d] = r < w ? q[b * qsb + h * qsh + static_cast<int64_t>(qrow0 + r) * qst + d] : 0.f;
  }
  __syncthreads();
  const int j = chunk * kChunkF32 + threadIdx.x;
  const float* kr = k + b * ksb + h * ksh + static_cast<int64_t>(min(j, L - 1)) * kst;
  float s[kMaxWindow];
#pragma unroll
  for (int i = 0; i < kMaxWindow; ++i) s[i] = 0.f;
  for (int d = 0; d < D; d += 4) {
    const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(kr + d);
#pragma unroll
    for (int i = 0; i < kMaxWindow; ++i)
      s[i] += qs[i][d] * kv[0] + qs[i][d + 1] * kv[1] + qs[i][d + 2] * kv[2] + qs[i][d + 3] * kv[3];
  }
#pragma unroll
  for (int i = 0; i < kMaxWindow; ++i) {
    const bool vis = i < w && j < L && j <= t0 + i;
    ss[i][threadIdx.x] = vis ? s[i] * scale_log2 : kNegBig;
  }
  __syncthreads();
  // 32 rows x 8 segments of 32 keys; the 8 segments of a row are adjacent lanes
  const int row = threadIdx.x >> 3, seg = threadIdx.x & 7;
  float m = kNegBig;
  for (int c = seg * 32; c < seg * 32 + 32; ++c) m = fmaxf(m, ss[row][c]);
  float l = 0.f;
  for (int c = seg * 32; c < seg * 32 + 32; ++c) l += fast_exp2(ss[row][c] - m);
  lse2_merge(m, l, lane_xor<1>(m), lane_xor<1>(l));
  lse2_merge(m, l, lane_xor<2>(m), lane_xor<2>(l));
  lse2_merge(m, l, lane_xor<4>(m), lane_xor<4>(l));
  if (seg == 0) part[(static_cast<int64_t>(bh) * nchunk + chunk) * 32 + row] = make_float2(m, l);
}

// ------------------------------------------- pass 2: votes, pooling, histogram

// A workgroup owns prefix keys [c0, c1) and computes the votes of [e0, e1) =
// [c0 - r, c1 + r) clipped to the prefix, so that it can max-pool its own keys
// without a second pass (the 2r halo keys are recomputed; with 1024-key chunks
// that is one extra partial MFMA tile).

// bf16, MFMA 32x32x16. Output orientation S: M = the 32 window queries, N =
// keys, so each lane owns one key (lane & 31) and 16 queries; its vote is a
// sum over registers plus one exchange with the other half of the wave.
template <int D>
__global__ __launch_bounds__(kThreads) void snap_votes_bf16(
    const uint16_t* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qst, int qrow0,
    const uint16_t* __restrict__ k, int64_t ksb, int64_t ksh, int64_t kst, int H, int L, int w, int r, int avg,
    float scale_log2, const float2* __restrict__ rowstat, float* __restrict__ vote, float* __restrict__ pooled,
    unsigned* __restrict__ hist) {
  constexpr int KS = D / 16;
  __shared__ float sv[kChunkMfma + 2 * kMaxPoolRadius];
  __shared__ unsigned sh[kHistBins];
  __shared__ float2 stat[32];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  if (threadIdx.x < 32) stat[threadIdx.x] = rowstat[bh * 32 + threadIdx.x];
  __syncthreads();
  const int b = bh / H, h = bh - b * H;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int col = lane & 31, half = lane >> 5;
  const int t0 = L - w;
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) sh[i] = 0;

  bf16x8_t qf[KS];
  if (col < w)
    load_half_row<D>(q + b * qsb + h * qsh + static_cast<int64_t>(qrow0 + col) * qst + half * (D / 2), qf);
  else
    zero_frag<D>(qf);
  float mr[16], il[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = acc_row(i, half);
    if (m < w) {
      const float2 st = stat[m];
      mr[i] = st.x;
      il[i] = st.y;
    } else {  // zero query row: score 0, weight 0
      mr[i] = 0.f;
      il[i] = 0.f;
    }
  }

  const uint16_t* kb = k + b * ksb + h * ksh + half * (D / 2);
  const int c0 = chunk * kChunkMfma, c1 = min(t0, c0 + kChunkMfma);
  const int e0 = max(0, c0 - r), e1 = min(t0, c1 + r);
  constexpr int kStep = kWaves * kTile;

  int tile = e0 + wave * kTile;
  bf16x8_t kf[KS];
  if (tile < e1) load_half_row<D>(kb + static_cast<int64_t>(min(tile + col, t0 - 1)) * kst, kf);
  for (; tile < e1; tile += kStep) {
    bf16x8_t kn[KS];
    const int nt = tile + kStep;
    if (nt < e1) load_half_row<D>(kb + static_cast<int64_t>(min(nt + col, t0 - 1)) * kst, kn);
    f32x16_t acc = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[s], kf[s], acc, 0, 0, 0);
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v += fast_exp2(acc[i] * scale_log2 - mr[i]) * il[i];
    v += lane_xor<32>(v);
    const int j = tile + col;
    if (half == 0 && j < e1) {
      sv[j - e0] = v;
      if (vote && j >= c0 && j < c1) vote[static_cast<int64_t>(bh) * t0 + j] = v;
    }
    if (nt < e1) {
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[s] = kn[s];
    }
  }
  __syncthreads();
  pool_and_count(sv, e0, e1, c0, c1, r, avg, pooled + static_cast<int64_t>(bh) * t0, sh);
  __syncthreads();
  flush_hist(sh, hist + static_cast<int64_t>(bh) * kHistBins);
}

// fp32, VALU: a key per thread, the window rows and their statistics in LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void snap_votes_f32(
    const float* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qst, int qrow0,
    const float* __restrict__ k, int64_t ksb, int64_t ksh, int64_t kst, int H, int L, int w, int r, int avg,
    float scale_log2, const float2* __restrict__ rowstat, float* __restrict__ vote, float* __restrict__ pooled,
    unsigned* __restrict__ hist) {
  __shared__ float qs[kMaxWindow][D];
  __shared__ float2 st[kMaxWindow];
  __shared__ float sv[kChunkF32 + 2 * kMaxPoolRadius];
  __shared__ unsigned sh[kHistBins];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int t0 = L - w;
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) sh[i] = 0;
  for (int i = threadIdx.x; i < kMaxWindow * D; i += kThreads) {
    const int rr = i / D, d = i - rr * D;
    qs[rr][d] = rr < w ? q[b * qsb + h * qsh + static_cast<int64_t>(qrow0 + rr) * qst + d] : 0.f;
  }
  if (threadIdx.x < kMaxWindow)
    st[threadIdx.x] = static_cast<int>(threadIdx.x) < w ? rowstat[bh * 32 + threadIdx.x] : make_float2(0.f, 0.f);
  __syncthreads();
  const int c0 = chunk * kChunkF32, c1 = min(t0, c0 + kChunkF32);
  const int e0 = max(0, c0 - r), e1 = min(t0, c1 + r);
  for (int j = e0 + static_cast<int>(threadIdx.x); j < e1; j += kThreads) {
    const float* kr = k + b * ksb + h * ksh + static_cast<int64_t>(j) * kst;
    float s[kMaxWindow];
#pragma unroll
    for (int i = 0; i < kMaxWindow; ++i) s[i] = 0.f;
    for (int d = 0; d < D; d += 4) {
      const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(kr + d);
#pragma unroll
      for (int i = 0; i < kMaxWindow; ++i)
        s[i] += qs[i][d] * kv[0] + qs[i][d + 1] * kv[1] + qs[i][d + 2] * kv[2] + qs[i][d + 3] * kv[3];
    }
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxWindow; ++i)
      if (i < w) v += fast_exp2(s[i] * scale_log2 - st[i].x) * st[i].y;
    sv[j - e0] = v;
    if (vote && j >= c0 && j < c1) vote[static_cast<int64_t>(bh) * t0 + j] = v;
  }
  __syncthreads();
  pool_and_count(sv, e0, e1, c0, c1, r, avg, pooled + static_cast<int64_t>(bh) * t0, sh);
  __syncthreads();
  flush_hist(sh, hist + static_cast<int64_t>(bh) * kHistBins);
}

// ------------------------------------ single-pass scores (cooperative, bf16)
//
// One read of K. A persistent grid of G workgroups (two per compute unit, all
// resident: cooperative launch) walks units of kCoopUnit consecutive keys of
// one head: workgroup g takes units u = r*G + g in rounds r = 0, 1, .... In
// round r it
//   * writes the votes of the unit of round r - kCoopLag, whose scores waited
//     in register bank (r - kCoopLag) % kCoopBanks; they need the head's
//     log-normaliser c_i = log2(sum_j 2^(s_ij)) of every window row i;
//   * scores the unit of round r from K staged in LDS by direct-to-LDS loads
//     issued during round r - 1, into bank r % kCoopBanks, and folds the
//     unit's per-row (m, l) (m the unit's row max, l its sum of 2^(s - m))
//     into a running pair for the head; after its last unit of the head the
//     workgroup adds l * 2^(m - R_i) to the head's row accumulators.
// R_i is a reference score of row i (its largest score against the window's
// own keys, computed beforehand), so every accumulated term is bounded below
// by the window key's own term of about 1. A row accumulator is a fixed-point
// integer: kCoopWords 64-bit words, word k summing terms of weight
// 2^(16 k + kCoopDigitBase) relative to 2^R_i; each term (a 24-bit mantissa
// shifted by less than 16 bits) is one integer atomic add, so the total is
// the same in every order. Completion is counted per head (one count per
// contributing workgroup): the workgroup whose count increment finishes a
// head converts its words into c_i and publishes them, tagged ready. Each cross-workgroup step waits only on something issued a
// round earlier (a contribution is complete before the count is raised, the
// count's return picks the finisher, the digits' loads land before the
// conversion, readers prefetch c a round ahead): at HBM-saturating load such
// round trips take microseconds, and none of them stalls the K stream.
// A unit whose row max exceeds R_i by more than kCoopOvfGap (a logit spread
// beyond the fixed-point range) flags its head, whose c_i is then merged
// exactly from the per-unit (m, l) partials in unit order.
constexpr int kCoopThreads = 256;            // 4 waves, one 32-key tile each per unit
constexpr int kCoopUnit = kWaves * kTile;    // 128 keys
constexpr int kCoopBanks = 8;
constexpr int kCoopLag = kCoopBanks - 1;     // rounds between a unit's scores and its votes
constexpr int kCoopWords = 20;               // accumulator words per row (a term lands in word <= 18)
constexpr int kCoopDigitBase = -160;
constexpr int kCoopRowWords = 544;           // row stride in 64-bit words: 4 KB + 256 B, so that the
                                             // rows' atomics spread over memory channels
constexpr int kCoopHeadWords = 32 * kCoopRowWords;
constexpr int kCoopFinWords = 24;            // words per row the finisher stages (room for the carries)
static_assert(kCoopWords < kCoopFinWords, "the staged words must hold every term's word and its carries");
constexpr int kCoopCtrWords = 32;            // per head: [0] unit count, [16] overflow flag
constexpr float kCoopOvfGap = 150.f;
constexpr unsigned kCoopSpin = 1u << 22;

__device__ __forceinline__ void st_agent_u2(uint2* p, uint2 v) {
  const unsigned long long u = (static_cast<unsigned long long>(v.y) << 32) | v.x;
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint2 ld_agent_u2(const uint2* p) {
  const unsigned long long u = __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2(static_cast<unsigned>(u), static_cast<unsigned>(u >> 32));
}

typedef __attribute__((address_space(3))) void lds_void;

// Cache-policy bits of a direct-to-LDS load that streams data read once (the
// nontemporal bit): on this device such a stream of K tiles moves measurably
// more bytes per second than with the default policy.
constexpr int kNtLoad = 2;

// LDS row layout shared by K tiles and Q: a row is D*2 bytes of kP 16-byte
// pieces; piece p of row R sits in slot p ^ (R & (kP-1)), so the 32 rows a
// wave reads for one MFMA k-step hit distinct banks.
template <int D>
struct CoopLayout {
  static constexpr int kRowB = D * 2;
  static constexpr int kP = kRowB / 16;               // pieces per row (16 or 8)
  static constexpr int kTileB = kTile * kRowB;        // bytes per 32-row tile
  static constexpr int kInstPerTile = kTileB / 1024;  // direct loads per tile (64 lanes x 16 B)
  static constexpr int kRowsPerInst = 1024 / kRowB;
  static constexpr int kKBytes = kWaves * kTileB;
  static constexpr int kQBytes = kTileB;              // 32 window rows
};

// Direct-to-LDS loads of one unit's K tiles, spread over waves 0..2. Rows
// beyond the data are clamped to valid rows; their scores are masked or never
// written.
template <int D>
__device__ __forceinline__ void coop_issue_k_loads(const uint16_t* kb, int64_t kst, int key0, int L,
                                                   unsigned char* kbuf, int wave, int lane) {
  using Ly = CoopLayout<D>;
  for (int i = wave; i < kWaves * Ly::kInstPerTile; i += 3) {
    const int tile = i / Ly::kInstPerTile, sub = i - tile * Ly::kInstPerTile;
    const int row = sub * Ly::kRowsPerInst + lane / Ly::kP;  // row within the tile
    const int slot = lane % Ly::kP;
    const int piece = slot ^ (row & (Ly::kP - 1));
    const int key = min(key0 + tile * kTile + row, L - 1);
    __builtin_amdgcn_global_load_lds(kb + static_cast<int64_t>(key) * kst + piece * 8,
                                     (lds_void*)(kbuf + tile * Ly::kTileB + sub * 1024), 16, 0, 0);
  }
}

// The same loads for a unit whose 128 rows all exist: instruction i covers
// unit rows i*kRowsPerInst + lane/kP, so its address is a uniform row base
// plus a per-lane 32-bit offset (lane/kP) * row_bytes + 16 * piece, where
// piece = (lane % kP) ^ (lane / kP) ^ ((i * kRowsPerInst) & (kP - 1)) (the
// two xor terms occupy disjoint bits).
template <int D>
__device__ __forceinline__ void coop_issue_k_full(const char* rows, int64_t row_bytes, unsigned char* kbuf, int wave,
                                                  int lane) {
  using Ly = CoopLayout<D>;
  const unsigned lrow = static_cast<unsigned>(lane / Ly::kP) * static_cast<unsigned>(row_bytes);
  const unsigned x16 = static_cast<unsigned>((lane % Ly::kP) ^ (lane / Ly::kP)) << 4;
  for (int i = wave; i < kWaves * Ly::kInstPerTile; i += 3) {
    const unsigned b16 = static_cast<unsigned>((i * Ly::kRowsPerInst) & (Ly::kP - 1)) << 4;
    const char* base = rows + static_cast<int64_t>(i * Ly::kRowsPerInst) * row_bytes;
    __builtin_amdgcn_global_load_lds(base + (lrow + (x16 ^ b16)), (lds_void*)(kbuf + i * 1024), 16, 0, kNtLoad);
  }
}

// Direct-to-LDS loads of the 32 window query rows (rows past the window
// repeat its last row), spread over waves 0..2.
template <int D>
__device__ __forceinline__ void coop_issue_q_loads(const uint16_t* qb, int64_t qst, int w, unsigned char* qbuf,
                                                   int wave, int lane) {
  using Ly = CoopLayout<D>;
  for (int sub = wave; sub < Ly::kInstPerTile; sub += 3) {
    const int row = sub * Ly::kRowsPerInst + lane / Ly::kP;
    const int slot = lane % Ly::kP;
    const int piece = slot ^ (row & (Ly::kP - 1));
    __builtin_amdgcn_global_load_lds(qb + static_cast<int64_t>(min(row, w - 1)) * qst + piece * 8,
                                     (lds_void*)(qbuf + sub * 1024), 16, 0, 0);
  }
}

// MFMA fragment of row R (lane & 31) from a swizzled LDS tile: k-step s of
// half h uses piece h*(kP/2) + s.
template <int D>
__device__ __forceinline__ bf16x8_t lds_frag(const unsigned char* tile, int R, int half, int s) {
  using Ly = CoopLayout<D>;
  const int piece = half * (Ly::kP / 2) + s;
  const int slot = piece ^ (R & (Ly::kP - 1));
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(tile + R * Ly::kRowB + slot * 16));
}

// Workgroup barrier for LDS exchanges only: waits for this wave's LDS
// operations, not for its vector-memory ones, so direct-to-LDS loads of the
// next round (and pending global stores) stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Reference score of every window row (largest score against the window's
// own keys it sees; rows past the window repeat the last row's), and the per-head state of the single pass cleared: row
// accumulators, count and overflow flag, published normalisers, histogram
// and selection counters. One workgroup per head.
template <int D>
__global__ __launch_bounds__(kThreads) void snap_coop_prep(
    const uint16_t* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qst, int qrow0,
    const uint16_t* __restrict__ k, int64_t ksb, int64_t ksh, int64_t kst, int H, int L, int w, float scale_log2,
    float* __restrict__ ref, unsigned long long* __restrict__ acc, unsigned* __restrict__ cnt,
    uint2* __restrict__ stat, unsigned* __restrict__ hist, unsigned* __restrict__ sel_ctr,
    unsigned* __restrict__ status) {
  const int bh = blockIdx.x, b = bh / H, h = bh - b * H;
  // status[0]: the score kernel's failure code (0 none; a bounded wait that
  // ran out: 1 vote weights, 2 merge slot, 3 a head's publication, 4 a head
  // still unfinished after the last round, 5 a head's queries); status[1],
  // status[2]: its residency gate
  // wave 0's query and key rows first (the kernel's one round trip to
  // memory), the clearing stores while they are in flight
  constexpr int KS = D / 16;
  const int lane = threadIdx.x & (kWave - 1), col = lane & 31, half = lane >> 5;
  bf16x8_t qf[KS], kf[KS];
  if (threadIdx.x < kWave) {
    const int rw = min(col, w - 1);
    load_half_row<D>(q + b * qsb + h * qsh + static_cast<int64_t>(qrow0 + rw) * qst + half * (D / 2), qf);
    load_half_row<D>(k + b * ksb + h * ksh + static_cast<int64_t>(L - w + rw) * kst + half * (D / 2), kf);
  }
  if (bh == 0 && threadIdx.x < 3) status[threadIdx.x] = 0;
  for (int i = threadIdx.x; i < 32 * kCoopFinWords; i += kThreads)
    acc[static_cast<int64_t>(bh) * kCoopHeadWords + (i / kCoopFinWords) * kCoopRowWords + i % kCoopFinWords] = 0;
  {
    u32x4_t* hv = reinterpret_cast<u32x4_t*>(hist + static_cast<int64_t>(bh) * kHistBins);  // 16 KB, 16-byte aligned
    for (int i = threadIdx.x; i < kHistBins / 4; i += kThreads) hv[i] = u32x4_t{0u, 0u, 0u, 0u};
  }
  if (threadIdx.x < kCoopCtrWords) cnt[bh * kCoopCtrWords + threadIdx.x] = 0;
  if (threadIdx.x < 32) stat[bh * 32 + threadIdx.x] = make_uint2(0u, 0u);
  if (threadIdx.x < kSelCtrWords) sel_ctr[bh * kSelCtrWords + threadIdx.x] = 0;
  // the window's 32 x 32 score block on one wave's MFMA: the window keys as
  // rows (M), the window queries as columns (N), so each lane holds 16 keys'
  // scores for query (lane & 31) and the row max takes one exchange between
  // the wave's halves; rows and keys past the window repeat row w - 1
  if (threadIdx.x < kWave) {
    f32x16_t sc = {};
#pragma unroll
    for (int st = 0; st < KS; ++st) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], sc, 0, 0, 0);
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = acc_row(i, half);
      if (j <= col && j < w) m = fmaxf(m, sc[i] * scale_log2);
    }
    m = fmaxf(m, lane_xor<32>(m));
    if (half == 0) ref[bh * 32 + col] = m;
  }
}

// Everything one workgroup of the single pass needs across rounds.
struct CoopCtx {
  const uint16_t* q;
  int64_t qsb, qsh, qst;
  int qrow0;
  const uint16_t* k;
  int64_t ksb, ksh, kst;
  int H, L, w, t0, nunit, G, g, rounds;
  float scale_log2;
  const float* ref;
  unsigned long long* acc;
  unsigned* cnt;
  uint2* stat;
  float2* part;
  unsigned* status;
  float* vote;
  unsigned char* kbuf0;  // K tiles of even rounds
  unsigned char* kbuf1;  // K tiles of odd rounds
  unsigned char* qbuf;
  float2 (*wred)[32];
  float* s_c;
  unsigned long long (*s_fin)[kCoopFinWords];
  int cnt_target;        // contributions per head: min(units per head, G)
  int wave, lane, col, half;
};

// Wave 3's bookkeeping carried from round to round.
struct CoopPipe {
  int ack_head;                  // head of the unit contributed last round (its count is due)
  int cnt_head;                  // head whose count was raised last round
  unsigned cnt_ret;              // that count's value before the increment
  int fin_head;                  // head being finished: its words were loaded into LDS last round
  unsigned fin_ovf;              // that head's overflow flag
  float fin_ref;                 // that head's reference score of row lane & 31
  int run_head;                  // head of the running (m, l) pair, -1 if none
  float run_m, run_l;            // running row max and sum of this workgroup's units of run_head
  uint2 pre;                     // normaliser prefetched for the next round's votes
  float ref;                     // reference score of row lane & 31 for this round's unit
  int q_head;                    // head whose Q rows sit in LDS
};

__device__ __forceinline__ int coop_head(const CoopCtx& c, int r) { return (r * c.G + c.g) / c.nunit; }

// lane & 31, opaque to the optimiser: addresses derived from it are formed
// where they are used (a scalar base plus a 32-bit lane offset) instead of
// being kept live as 64-bit per-lane pointers across the whole round loop.
__device__ __forceinline__ int coop_row(const CoopCtx& c) {
  int row = c.lane & 31;
  asm volatile("" : "+v"(row));
  return row;
}

// x, opaque to the optimiser: values derived from it inside a rarely taken
// branch are computed there, instead of being hoisted out of the round loop
// and kept live (or spilled) for the whole kernel.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// K tiles of round r's unit into `kbuf` (waves 0..2).
template <int D>
__device__ __forceinline__ void coop_issue_k(const CoopCtx& c, int r, unsigned char* kbuf) {
  if (c.wave >= 3) return;
  const int u = r * c.G + c.g;
  const int bh = u / c.nunit, key0 = (u - bh * c.nunit) * kCoopUnit;
  const int b = bh / c.H, h = bh - b * c.H;
  const uint16_t* kb = c.k + b * c.ksb + h * c.ksh;
  if (key0 + kCoopUnit <= c.L)
    coop_issue_k_full<D>(reinterpret_cast<const char*>(kb + static_cast<int64_t>(key0) * c.kst), c.kst * 2, kbuf,
                         c.wave, c.lane);
  else
    coop_issue_k_loads<D>(kb, c.kst, key0, c.L, kbuf, c.wave, c.lane);
}

// Q rows of round r's head, unless they are the ones already staged.
template <int D>
__device__ __forceinline__ void coop_issue_q(const CoopCtx& c, CoopPipe& p, int r) {
  const int bh = coop_head(c, r);
  if (bh == p.q_head) return;
  p.q_head = bh;
  if (c.wave >= 3) return;
  const int b = bh / c.H, h = bh - b * c.H;
  coop_issue_q_loads<D>(c.q + b * c.qsb + h * c.qsh + static_cast<int64_t>(c.qrow0) * c.qst, c.qst, c.w, c.qbuf,
                        c.wave, c.lane);
}

// The head's normaliser from its accumulator words (staged in s_fin[row]):
// exact carry propagation into 16-bit digits, the total's leading 24 bits as
// mf * 2^E with mf in [1, 2), then c = R + E + log2(mf). Lanes 0..31.
__device__ __forceinline__ float coop_words_to_c(unsigned long long (*s_fin)[kCoopFinWords], int row, float R) {
  unsigned long long carry = 0;
  int top = -1;
#pragma unroll 1
  for (int k = 0; k < kCoopFinWords; ++k) {
    const unsigned long long v = s_fin[row][k] + carry;
    s_fin[row][k] = v & 0xffffull;
    carry = v >> 16;
    if (v & 0xffffull) top = k;
  }
  if (top < 0) return R;  // no mass at all (cannot happen for a window row)
  unsigned long long wv = 0;
#pragma unroll 1
  for (int k = top; k > top - 4; --k) wv = (wv << 16) | (k >= 0 ? s_fin[row][k] : 0ull);
  const int lz = __clzll(static_cast<long long>(wv));
  wv <<= lz;  // total ~ wv * 2^(16 (top - 3) + kCoopDigitBase - lz), leading bit at 63
  const int E = 16 * (top - 3) + kCoopDigitBase - lz + 63;
  const float mf = __uint_as_float(0x3f800000u | static_cast<unsigned>((wv >> 40) & 0x7fffffu));
  return R + (static_cast<float>(E) + __builtin_amdgcn_logf(mf));
}

// Exact normaliser of a flagged head: merge of its per-unit (m, l) partials
// in unit order (lanes 0..31, one row each).
__device__ __forceinline__ float coop_exact_c(const CoopCtx& c, int bh, int row) {
  float m = kNegBig, l = 0.f;
  const float2* pb = c.part + static_cast<int64_t>(bh) * c.nunit * 32;
  for (int u0 = 0; u0 < c.nunit; u0 += 4) {
    uint2 pp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pp[i] = u0 + i < c.nunit ? ld_agent_u2(reinterpret_cast<const uint2*>(&pb[(u0 + i) * 32 + row]))
                               : make_uint2(__float_as_uint(kNegBig), 0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) lse2_merge(m, l, __uint_as_float(pp[i].x), __uint_as_float(pp[i].y));
  }
  return m + __builtin_amdgcn_logf(l);  // v_log_f32: log2 to about an ulp, no constants to keep live
}

// Adds a row's l * 2^(m - R) to its accumulator (lanes 0..31, rows < w):
// l * 2^gap = y * 2^n with y = l * 2^(gap - n) in [l, 2l) and l >= 1 (the
// max term), y = mant * 2^(ey - 23) exactly, so the term is the 24-bit mant
// at bit pos = ey - 23 + n - kCoopDigitBase, i.e. mant << (pos % 16) in word
// pos / 16. Terms below word 0 are dropped (they are at least 2^-100 times
// the window key's own term); a gap above kCoopOvfGap flags the head.
__device__ __forceinline__ void fixed_point_add(unsigned long long* acc_head, unsigned* ovf_flag, int row, float m,
                                                float l, float R) {
  const float gap = m - R;
  if (gap > kCoopOvfGap) {
    atomicOr(ovf_flag, 1u);
  } else if (gap > static_cast<float>(kCoopDigitBase + 60)) {
    const float n = floorf(gap);
    const float y = l * fast_exp2(gap - n);
    const unsigned bits = __float_as_uint(y);
    unsigned long long mant = (bits & 0x7fffffu) | 0x800000u;
    int pos = static_cast<int>((bits >> 23) & 0xffu) - 127 - 23 + static_cast<int>(n) - kCoopDigitBase;
    if (pos < 0) {
      mant >>= -pos;  // -pos < 40 here
      pos = 0;
    }
    const unsigned off = static_cast<unsigned>(row * kCoopRowWords + (pos >> 4)) * 8u;
    atomicAdd(reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(acc_head) + off), mant << (pos & 15));
  }
}

__device__ __forceinline__ void coop_contribute(const CoopCtx& c, int bh, int row, float m, float l, float R) {
  fixed_point_add(c.acc + static_cast<int64_t>(bh) * kCoopHeadWords, &c.cnt[bh * kCoopCtrWords + 16], row, m, l, R);
}

// End-of-round bookkeeping of wave 3 (after the unit's row statistics are in
// (m, l) of lanes 0..31 when `contributed`), entered after the round's
// closing wait: whatever it issues is used only after the next round's.
__device__ __forceinline__ void coop_bookkeeping(const CoopCtx& c, CoopPipe& p, bool contributed, int unit, float m,
                                                 float l, int r) {
  const int row = coop_row(c);
  // (a) finish the head whose words were staged last round
  if (p.fin_head >= 0) {
    float cv = 0.f;
    if (__builtin_amdgcn_readfirstlane(p.fin_ovf) == 0u) {
      if (c.lane < 32) cv = coop_words_to_c(c.s_fin, row, p.fin_ref);
    } else {
      if (c.lane < 32 && row < c.w) cv = coop_exact_c(c, p.fin_head, row);
    }
    if (c.lane < 32 && row < c.w) st_agent_u2(&c.stat[p.fin_head * 32 + row], make_uint2(__float_as_uint(cv), 1u));
    p.fin_head = -1;
  }
  // (b) the count raised last round: the last contribution makes this
  // workgroup the finisher; stage the head's words in LDS
  if (p.cnt_head >= 0) {
    if (static_cast<unsigned>(__builtin_amdgcn_readfirstlane(p.cnt_ret)) == static_cast<unsigned>(c.cnt_target - 1)) {
      const unsigned long long* a = c.acc + static_cast<int64_t>(p.cnt_head) * kCoopHeadWords;
      constexpr int kPieces = 32 * kCoopFinWords / 2;  // 16-byte pieces
#pragma unroll
      for (int i = 0; i < kPieces / 64; ++i) {
        const int piece = i * 64 + c.lane, prow = piece / (kCoopFinWords / 2), pj = piece % (kCoopFinWords / 2);
        __builtin_amdgcn_global_load_lds(a + prow * kCoopRowWords + pj * 2,
                                         (lds_void*)(&c.s_fin[0][0] + i * 128), 16, 0, 16 /* sc1 */);
      }
      p.fin_ovf = __hip_atomic_load(&c.cnt[p.cnt_head * kCoopCtrWords + 16], __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
      p.fin_ref = c.ref[p.cnt_head * 32 + row];
      p.fin_head = p.cnt_head;
    }
    p.cnt_head = -1;
  }
  // (c) last round's contribution is complete: count it
  if (p.ack_head >= 0) {
    unsigned ret = 0;
    if (c.lane == 0) ret = atomicAdd(&c.cnt[p.ack_head * kCoopCtrWords], 1u);
    p.cnt_ret = ret;
    p.cnt_head = p.ack_head;
    p.ack_head = -1;
  }
  // (d) this round's unit: its partial, the running pair, and the
  // contribution after this workgroup's last unit of the head
  if (contributed) {
    const int bh = unit / c.nunit;
    if (c.lane < 32)
      st_agent_u2(reinterpret_cast<uint2*>(&c.part[static_cast<int64_t>(unit) * 32 + row]),
                  make_uint2(__float_as_uint(m), __float_as_uint(l)));
    if (p.run_head == bh) {
      lse2_merge(p.run_m, p.run_l, m, l);
    } else {
      p.run_m = m;
      p.run_l = l;
      p.run_head = bh;
    }
    if (!(r + 1 < c.rounds && coop_head(c, r + 1) == bh)) {
      if (c.lane < 32 && row < c.w) coop_contribute(c, bh, row, p.run_m, p.run_l, p.ref);
      p.ack_head = bh;
      p.run_head = -1;
    }
  }
}

template <int D, int BANK>
__device__ __forceinline__ void coop_round(const CoopCtx& c, CoopPipe& p,
                                           f32x16_t (&sc)[kCoopBanks], int r) {
  using Ly = CoopLayout<D>;
  constexpr int KS = D / 16;
  const int rb = r - kCoopLag;
  const bool do_b = rb >= 0 && rb < c.rounds, do_a = r < c.rounds;
  // ---- round start: the previous round's closing wait covered the staged K
  // and the prefetched normalisers and reference scores
  if (c.wave == 3) {
    if (do_b) {
      const int hb = coop_head(c, rb);
      const int row = c.lane & 31;
      uint2 pre = p.pre;
      if (__ballot(row < c.w && pre.y != 1u) != 0ull) {  // not yet published: wait (bounded)
        unsigned polls = 0;
        bool late;
        do {
          __builtin_amdgcn_s_sleep(2);
          pre = ld_agent_u2(&c.stat[hb * 32 + row]);
          __builtin_amdgcn_s_waitcnt(0);  // every exit from here has its load back
          late = __ballot(row < c.w && pre.y != 1u) != 0ull;
        } while (late && ++polls < kCoopSpin);
        if (late && c.lane == 0) __hip_atomic_store(c.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
      }
      if (c.lane < 32) c.s_c[c.lane] = __uint_as_float(pre.x);
    }
    const int last = max(c.rounds - 1, 0);
    p.pre = ld_agent_u2(&c.stat[coop_head(c, min(max(rb + 1, 0), last)) * 32 + (c.lane & 31)]);
    p.ref = c.ref[coop_head(c, min(r, last)) * 32 + (c.lane & 31)];
  }
  lds_barrier();  // everyone is past round r - 1: its K buffer is free again
  if (r + 1 < c.rounds) coop_issue_k<D>(c, r + 1, (BANK & 1) ? c.kbuf0 : c.kbuf1);
  // ---- votes of the unit of round rb (bank (BANK + 1) % kCoopBanks)
  if (do_b) {
    const int u = rb * c.G + c.g;
    const int bh = u / c.nunit, c0 = (u - bh * c.nunit) * kCoopUnit;
    const f32x16_t& s = sc[(BANK + 1) % kCoopBanks];
    float v = 0.f;
    if (c.w == kMaxWindow) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v += fast_exp2(s[i] - c.s_c[acc_row(i, c.half)]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = acc_row(i, c.half);
        v += row < c.w ? fast_exp2(s[i] - c.s_c[row]) : 0.f;
      }
    }
    v += lane_xor<32>(v);
    const int j = c0 + c.wave * kTile + c.col;
    if (c.half == 0 && j < c.t0) c.vote[static_cast<int64_t>(bh) * c.t0 + j] = v;
  }
  // ---- scores of the unit of round r into bank BANK
  float m = kNegBig, l = 0.f;
  int unit = 0;
  if (do_a) {
    unit = r * c.G + c.g;
    const int bh = unit / c.nunit, c0 = (unit - bh * c.nunit) * kCoopUnit;
    const unsigned char* tile = ((BANK & 1) ? c.kbuf1 : c.kbuf0) + c.wave * Ly::kTileB;
    f32x16_t acc = {}, bt = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t qf = lds_frag<D>(c.qbuf, c.col, c.half, s);
      const bf16x8_t kf = lds_frag<D>(tile, c.col, c.half, s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf, acc, 0, 0, 0);
      bt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf, bt, 0, 0, 0);
      if (s % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // bound the fragments held in flight
    }
    const int jt = c0 + c.wave * kTile;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[BANK][i] = acc[i] * c.scale_log2;
    if (c0 + kCoopUnit <= c.t0) {  // the whole unit is prefix: every query sees every key
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        bt[i] *= c.scale_log2;
        m = fmaxf(m, bt[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = jt + acc_row(i, c.half);
        bt[i] = (j < c.L && j <= c.t0 + c.col) ? bt[i] * c.scale_log2 : kNegBig;
        m = fmaxf(m, bt[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) l += fast_exp2(bt[i] - m);
    lds_barrier();  // staged Q consumed
    if (r + 1 < c.rounds) coop_issue_q<D>(c, p, r + 1);
    lse2_merge(m, l, lane_xor<32>(m), lane_xor<32>(l));
    if (c.half == 0) c.wred[c.wave][c.col] = make_float2(m, l);
    lds_barrier();
    if (c.wave == 3) {
      float2 a = c.wred[0][c.lane & 31];
#pragma unroll
      for (int i = 1; i < kWaves; ++i) lse2_merge(a.x, a.y, c.wred[i][c.lane & 31].x, c.wred[i][c.lane & 31].y);
      m = a.x;
      l = a.y;
    }
  }
  // closing wait, all waves: the next round's K tiles (waves 0..2); this
  // round's prefetches and last round's contributions, count and digit loads
  // (wave 3)
  __builtin_amdgcn_s_waitcnt(0);
  if (c.wave == 3) coop_bookkeeping(c, p, do_a, unit, m, l, r);
}

template <int D>
__global__ __launch_bounds__(kCoopThreads, 2) void snap_coop_bf16(
    const uint16_t* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qst, int qrow0,
    const uint16_t* __restrict__ k, int64_t ksb, int64_t ksh, int64_t kst, int H, int L, int w, int nunit,
    int total_units, float scale_log2, const float* __restrict__ ref, unsigned long long* __restrict__ acc,
    unsigned* __restrict__ cnt, uint2* __restrict__ stat, float2* __restrict__ part,
    unsigned* __restrict__ status, float* __restrict__ vote) {
  using Ly = CoopLayout<D>;
  __shared__ __attribute__((aligned(16))) unsigned char kbuf0[Ly::kKBytes];
  __shared__ __attribute__((aligned(16))) unsigned char kbuf1[Ly::kKBytes];
  __shared__ __attribute__((aligned(16))) unsigned char qbuf[Ly::kQBytes];
  __shared__ float2 wred[kWaves][32];
  __shared__ float s_c[32];
  __shared__ unsigned long long s_fin[32][kCoopFinWords];

  CoopCtx c;
  c.q = q; c.qsb = qsb; c.qsh = qsh; c.qst = qst; c.qrow0 = qrow0;
  c.k = k; c.ksb = ksb; c.ksh = ksh; c.kst = kst;
  c.H = H; c.L = L; c.w = w; c.t0 = L - w; c.nunit = nunit;
  c.G = static_cast<int>(gridDim.x); c.g = static_cast<int>(blockIdx.x);
  c.rounds = (total_units - c.g + c.G - 1) / c.G;
  c.cnt_target = min(nunit, c.G);
  c.scale_log2 = scale_log2;
  c.ref = ref; c.acc = acc; c.cnt = cnt; c.stat = stat; c.part = part; c.status = status; c.vote = vote;
  c.kbuf0 = kbuf0; c.kbuf1 = kbuf1; c.qbuf = qbuf; c.wred = wred; c.s_c = s_c; c.s_fin = s_fin;
  c.lane = lane_id(); c.col = c.lane & 31; c.half = c.lane >> 5;
  c.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);  // uniform: keeps wave-indexed
                                                                                     // addresses in scalar registers
  CoopPipe p;
  p.ack_head = p.cnt_head = p.fin_head = -1;
  p.cnt_ret = 0;
  p.fin_ovf = 0;
  p.run_head = -1;
  p.run_m = kNegBig;
  p.run_l = 0.f;
  p.pre = make_uint2(0u, 0u);
  p.fin_ref = 0.f;
  p.ref = 0.f;
  p.q_head = -1;
  f32x16_t sc[kCoopBanks];
  if (c.rounds > 0) {
    coop_issue_k<D>(c, 0, c.kbuf0);
    coop_issue_q<D>(c, p, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  // every unit's votes (round rounds - 1 + kCoopLag) and its head's
  // bookkeeping (three rounds after its last unit) fall inside the loop
  static_assert(kCoopBanks == 8, "the round loop below is unrolled over the register banks");
  for (int r0 = 0; r0 < c.rounds + kCoopLag; r0 += kCoopBanks) {
    coop_round<D, 0>(c, p, sc, r0);
    coop_round<D, 1>(c, p, sc, r0 + 1);
    coop_round<D, 2>(c, p, sc, r0 + 2);
    coop_round<D, 3>(c, p, sc, r0 + 3);
    coop_round<D, 4>(c, p, sc, r0 + 4);
    coop_round<D, 5>(c, p, sc, r0 + 5);
    coop_round<D, 6>(c, p, sc, r0 + 6);
    coop_round<D, 7>(c, p, sc, r0 + 7);
  }
}

// --------------------------- single-pass scores, independent waves (bf16)
//
// The single-pass computation with the workgroup's lockstep removed and the
// softmax reorganised around a fixed per-row offset. R_i (the reference score
// of window row i, computed beforehand) is one of row i's own scores, so with
// e_ij = 2^(s_ij - R_i) and L_i = sum_j e_ij >= 1 the normaliser is
// c_i = R_i + log2 L_i and the vote of key j is
//     vote_j = sum_i 2^(s_ij - c_i) = sum_i e_ij * w_i,   w_i = 1 / L_i <= 1,
// exactly (in real arithmetic). Scores are therefore exponentiated once; the
// row sums need no running maximum, and the votes no exponential.
//
// Every wave is a worker of its own: worker v = g * kWvWaves + wave takes the
// 32-key tiles u = r * W + v in rounds r = 0, 1, ... (W = G * kWvWaves
// workers; tiles numbered head by head, a head's tile count padded to a
// multiple of kWvWaves, so that the tiles of one workgroup in one round share
// a head). A wave keeps its next tile in flight while it works on the
// current one: K by direct-to-LDS loads into a private two-slot ring. The
// workgroup's waves share two query slots in LDS: a head's window queries
// are loaded once per workgroup, two heads ahead, by the last wave to read
// the slot's previous head (wv_take_q), and each wave reads them into its
// registers at its first tile of the head. One MFMA orientation serves both
// uses: lane = key, registers = rows.
// Round r's e_ij wait in register bank r % kWvBanks and each lane adds them
// into per-row partial sums; just before round r's values replace them, the
// bank's previous contents (the tile of round r - kWvBanks) become votes.
// At the end of a head a wave reduces its partial sums across lanes, stores
// them in an LDS slot of its workgroup, and the workgroup's designated wave
// for that head ((h + g) % kWvWaves, spreading the work evenly) adds the
// waves' sums in wave order and contributes them to the head's fixed-point
// row accumulators (order-independent integer adds that also count the
// contributions). The workgroup whose count increment completes the head
// stages the accumulators into LDS, converts them into w_i once every
// contribution has landed, and publishes them. A wave's only full wait is
// the one for its next tile at the start of a round; everything else it
// issued in the previous round is complete there too, so each cross-worker
// step takes a round and none of them holds up the K stream.
//
// e_ij is finite unless a score exceeds its row's reference by 2^127; such a
// head is flagged and the pooling kernel recomputes its votes exactly (the
// usual path's votes of that head are discarded).
//
// Registers: the nine banks (144), Q (32), the MFMA accumulator and the row
// sums fill most of the 256 a wave has at two waves per SIMD, so every
// per-lane value a round needs is derived inside the round from one opaque
// lane index instead of being kept live across the loop (a spilled value's
// reload would have to wait behind the next tile's loads).
constexpr int kWvWaves = 8;
constexpr unsigned kWvGateSpin = 1u << 14;  // residency-check polls (~1 ms) before the exact fallback
constexpr int kWvThreads = kWvWaves * kWave;
constexpr int kWvBanks = 9;
constexpr int kWvRowWords = 24;  // accumulator words per row a finisher stages (values in words 0..19)
constexpr int kWvFinBufs = 2;    // finisher staging buffers, by head mod 2
constexpr int kWvMaxSpan = kWvBanks - 3;  // a head spans at most this many rounds after its first
constexpr int kWvMinRounds = 8;            // rounds a layer of heads shorter than a round must fill
constexpr unsigned kWvSpin = 1u << 18;  // polls before a wait gives up (far beyond any legitimate wait)
constexpr unsigned kWvSpinForced = 0u;   // the testing limit: every wait that has to wait gives up
constexpr int kWvOvfWord = 20;   // a non-finite row sum adds its count here (the head is then flagged)
constexpr unsigned long long kWvCountOne = 1ull << 48;

template <int D>
struct WvLayout {
  static constexpr int kRowB = D * 2;
  static constexpr int kP = kRowB / 16;               // 16-byte pieces per row
  static constexpr int kTileB = kTile * kRowB;        // bytes per 32-row tile
  static constexpr int kInst = kTileB / 1024;         // direct loads per tile (64 lanes x 16 B)
  static constexpr int kRowsPerInst = 1024 / kRowB;
};

// A finisher's copy of one head's accumulator words (row-major, kWvRowWords per row).
struct WvFin {
  unsigned long long words[32 * kWvRowWords];
};

struct WvShared {
  float lslot[2][kWvWaves][32];  // the waves' row sums of head h, in slot h & 1
  float s_wr[kWvWaves][32];      // each wave's vote weights w_i for its votes, then (later in
                                 // the same round) the reference scores R_i of its tile
  int fin_owner[kWvFinBufs];     // head staged in a finisher buffer, -1 if free
  int mcnt[2];                   // waves that have stored their sums in a slot
  int mtag[2];                   // the head a slot is open for
  int qtag[2];                   // workgroup head sequence index whose queries have landed in query slot s
  int qreads[2];                 // waves that have read the queries in query slot s
};

struct WvPos {
  int head, h, t;      // processing index t of head `head` (h = head % H)
  int a;               // the head's tile it scores (wv_rot)
  const char* kh;      // K row 0 of that head
  const char* kt;      // K row 32 a of that head
};

struct WvCtx {
  const uint16_t* q;
  int64_t qsb, qsh, qst;
  int qrow0;
  const uint16_t* k;
  int64_t ksb, ksh, kst;
  int H, L, w, t0, nt, BH, G, g, W, rounds, wave;
  int tgt;     // workgroups that contribute to each head: G, or nt / kWvWaves when a head is shorter than a round
  bool small;  // a head is shorter than a round: every workgroup takes a new head every round
  int64_t tile_b, dk_head, dk_batch;  // bytes per K tile; steps of WvPos::kh to the next head, batch
  unsigned spin;  // polls before a cross-worker wait gives up (kWvSpin; kWvSpinForced for tests)
  float scale_log2;
  const float* ref;
  unsigned long long* acc;
  unsigned* cnt;
  uint2* stat;
  unsigned* status;
  float* vote;
  WvShared* sh;
  WvFin* fin;  // the finisher buffers: an array of their own, so that LDS accesses to the
               // workgroup's other shared state are known not to alias their direct loads
  unsigned char* qs;  // the workgroup's two query slots, a tile each
  int wq, wr;        // heads shorter than a round: W / nt and W % nt
  unsigned h_rcp;    // min(ceil(2^32 / H), 2^32 - 1), for head / H without a division
};

// head / H for 0 <= head < 2^31: for H >= 2 the high word of head * h_rcp is
// the quotient or one more (the product overshoots head / H by less than
// head / 2^32 < 1/2); for H = 1 it is the quotient or one less; one compare
// in each direction corrects it.
__device__ __forceinline__ int wv_batch_of(const WvCtx& c, int head) {
  int b = static_cast<int>(__umulhi(static_cast<unsigned>(head), c.h_rcp));
  if (b * c.H > head) --b;
  if ((b + 1) * c.H <= head) ++b;
  return b;
}

// A wave's state carried from round to round.
struct WvPipe {
  int fin_head;      // the next head this wave finishes (heads g + G * wave + W * i), >= BH: none left
  unsigned fin_cnt;  // that head's contribution count, read (agent scope) last round
  int merge_head;    // head this wave merges for its workgroup once all its waves have stored their sums
  int merge_idx;     // that head's index in the workgroup's sequence of heads (its slot is merge_idx & 1)
  uint2 pre[2];      // vote weights prefetched for the votes of the rounds of each parity
  float rref[2];     // reference score of row lane & 31 for the tiles of each round parity
  int vhead, vtile;  // head and processing index of the tile whose votes are next (round r - kWvBanks)
  bool gave_up;      // a bounded wait has run out: no further waits (the results are invalid)
  int qhead;         // head whose query fragments are in the registers, -1: none
  int qpub;          // workgroup head sequence index of the queries this wave loaded into a
                     // query slot last round (marked landed at the next round's start), -1: none
};

// The tile of head `head` that processing index t scores: t rotated by
// head % kWvWaves within the head's nt tiles. Without it the head's last
// tiles (the window's own keys, whose scores are masked) would fall to the
// same wave in every head, which then trails the others by that extra work
// more with each head; rotated, they go to a different wave each time.
__device__ __forceinline__ int wv_rot(const WvCtx& c, int head, int t) {
  const int a = t + (head & (kWvWaves - 1));
  return a >= c.nt ? a - c.nt : a;
}

// The next round's tile: W tiles on (W <= tiles per head, so at most one
// head boundary); the head's K base moves by precomputed byte steps.
__device__ __forceinline__ WvPos wv_next(const WvCtx& c, WvPos p) {
  if (c.small) {  // heads shorter than a round: W / nt or one more heads on, pointers recomputed
    const int carry = p.t + c.wr >= c.nt ? 1 : 0;  // t < nt and W % nt < nt: at most one more
    p.t += c.wr - carry * c.nt;
    p.head += c.wq + carry;
    const int b = wv_batch_of(c, p.head);
    p.h = p.head - b * c.H;
    p.kh = reinterpret_cast<const char*>(c.k + b * c.ksb + p.h * c.ksh);
  } else {
    p.t += c.W;
    if (p.t >= c.nt) {
      p.t -= c.nt;
      ++p.head;
      p.kh += c.dk_head;
      if (++p.h == c.H) {
        p.h = 0;
        p.kh += c.dk_batch;
      }
    }
  }
  p.a = wv_rot(c, p.head, p.t);
  p.kt = p.kh + static_cast<int64_t>(p.a) * c.tile_b;
  return p;
}

// The tile after t for the vote tracker (head and tile only).
__device__ __forceinline__ void wv_next_ht(const WvCtx& c, int& head, int& t) {
  if (c.small) {
    const int carry = t + c.wr >= c.nt ? 1 : 0;
    t += c.wr - carry * c.nt;
    head += c.wq + carry;
    return;
  }
  t += c.W;
  if (t >= c.nt) {
    t -= c.nt;
    ++head;
  }
}

// Direct-to-LDS loads of one 32-row K tile into `slot` (XOR-swizzled rows:
// 16-byte piece p of row R at slot p ^ (R & (kP-1))).
template <int D>
__device__ __forceinline__ void wv_issue_k(const WvCtx& c, const WvPos& p, unsigned char* slot, int lane) {
  using Ly = WvLayout<D>;
  const int key0 = p.a * kTile;
  if (__builtin_expect(key0 + kTile <= c.L, 1)) {
    // instruction i covers rows i*kRowsPerInst + lane/kP: a uniform row base plus
    // the per-lane 32-bit offset (lane/kP) * row_bytes + 16 * piece
    const char* rows = p.kt;
    const int64_t rb = c.kst * 2;
    const unsigned lrow = static_cast<unsigned>(lane / Ly::kP) * static_cast<unsigned>(rb);
    const unsigned x16 = static_cast<unsigned>((lane % Ly::kP) ^ (lane / Ly::kP)) << 4;
#pragma unroll
    for (int i = 0; i < Ly::kInst; ++i) {
      const unsigned b16 = static_cast<unsigned>((i * Ly::kRowsPerInst) & (Ly::kP - 1)) << 4;
      __builtin_amdgcn_global_load_lds(rows + static_cast<int64_t>(i * Ly::kRowsPerInst) * rb + (lrow + (x16 ^ b16)),
                                       (lds_void*)(slot + i * 1024), 16, 0, kNtLoad);
    }
  } else {  // the head's last, ragged tile or a padding tile: rows clamped to the data
    const uint16_t* kb = reinterpret_cast<const uint16_t*>(p.kt) - static_cast<int64_t>(key0) * c.kst;
#pragma unroll
    for (int i = 0; i < Ly::kInst; ++i) {
      const int row = i * Ly::kRowsPerInst + lane / Ly::kP;
      const int piece = (lane % Ly::kP) ^ (row & (Ly::kP - 1));
      const int key = min(key0 + row, c.L - 1);
      __builtin_amdgcn_global_load_lds(kb + static_cast<int64_t>(key) * c.kst + piece * 8,
                                       (lds_void*)(slot + i * 1024), 16, 0, kNtLoad);
    }
  }
}

// The first window query row of head `head`.
__device__ __forceinline__ const uint16_t* wv_q_base(const WvCtx& c, int head) {
  const int b = wv_batch_of(c, head), h = head - b * c.H;
  return c.q + b * c.qsb + h * c.qsh + static_cast<int64_t>(c.qrow0) * c.qst;
}

// Direct-to-LDS loads of a head's window queries (first row qb) into a query
// slot, laid out as a K tile (32 rows, XOR-swizzled; rows past the window
// repeat its last row), so that the MFMA fragments of the queries are read
// with the same addresses as a tile's. Four rows per instruction: each reads
// whole rows, where loading the fragments straight into registers takes 16
// bytes from each of 64 rows per instruction (the loads of every head change
// then measured ~15 us of the 131K layer's score kernel).
template <int D>
__device__ __forceinline__ void wv_issue_q(const WvCtx& c, const uint16_t* qb, unsigned char* slot, int lane) {
  using Ly = WvLayout<D>;
#pragma unroll
  for (int i = 0; i < Ly::kInst; ++i) {
    const int row = i * Ly::kRowsPerInst + lane / Ly::kP;
    const int piece = (lane % Ly::kP) ^ (row & (Ly::kP - 1));
    __builtin_amdgcn_global_load_lds(qb + static_cast<int64_t>(min(row, c.w - 1)) * c.qst + piece * 8,
                                     (lds_void*)(slot + i * 1024), 16, 0, 0);
  }
}

// s_waitcnt vmcnt(0), as the builtin (so that the compiler's own wait
// placement knows every vector-memory operation issued so far is complete:
// later uses of last round's loads need no wait that would also hold for
// this round's tile) and as a compiler barrier (the tile's LDS reads stay
// after it).
__device__ __forceinline__ void wait_vm_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt not waited for
  asm volatile("" ::: "memory");
}

// LDS add (by the lanes of the calling branch), issued as inline assembly:
// as a compiler atomic it would make the compiler wait for the direct loads
// in flight into the tile ring as well.
__device__ __forceinline__ void lds_add(int* p, int v) {
  const unsigned a = static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) int*)p));
  asm volatile("ds_add_u32 %0, %1" : : "v"(a), "v"(v) : "memory");
}

// The same, returning the value before the add (its LDS wait included).
__device__ __forceinline__ int lds_add_rtn_i(int* p, int v) {
  const unsigned a = static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) int*)p));
  int r;
  asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(a), "v"(v) : "memory");
  return r;
}

// Adds a workgroup's row sum L (of e_ij = 2^(s_ij - R_i)) to row `row` of a
// head's fixed-point accumulator: L = mant * 2^(ey - 23), so the 24-bit
// mantissa goes to bit pos = ey - 23 - kCoopDigitBase, i.e. mant << (pos % 16)
// in word pos / 16 (pos <= 264 for a finite fp32), together with a count of 1
// in bits 48..63 (a word's value part stays below 2^48: at most 2^9 terms
// below 2^39 each). Sums below 2^-100 (at least 2^-100 times the row's total)
// add only the count, a non-finite one adds its count to word kWvOvfWord.
__device__ __forceinline__ void wv_add_sum(unsigned long long* acc_head, int row, float L) {
  unsigned long long* arow = reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(acc_head) +
                                                                   static_cast<unsigned>(row * kCoopRowWords) * 8u);
  if (!(L <= 3.0e38f)) {
    atomicAdd(arow + kWvOvfWord, kWvCountOne);
  } else if (L < 7.9e-31f) {  // 2^-100
    atomicAdd(arow, kWvCountOne);
  } else {
    const unsigned bits = __float_as_uint(L);
    const unsigned long long mant = (bits & 0x7fffffu) | 0x800000u;
    const int pos = static_cast<int>(bits >> 23) - 127 - 23 - kCoopDigitBase;
    atomicAdd(arow + (pos >> 4), (mant << (pos & 15)) + kWvCountOne);
  }
}

// Head h's vote weight of row lane & 31 from its staged words (lanes of half
// 0 take words 0..11, half 1 words 12..23): L = sum of the value parts (each
// word's is below 2^48, exact in a double, and so is each scaled term; both
// halves add the two partial sums in the same order, so the value is the same
// in every lane and every run), w = 1 / L. `count` is the row's number of
// contributions and `ovf` whether one of them was not finite.
__device__ __forceinline__ float wv_words_to_w(const WvFin& f, int lane, unsigned& count, bool& ovf) {
  constexpr int kHalf = kWvRowWords / 2;
  const int row = lane & 31, half = lane >> 5;
  const uint2* wr = reinterpret_cast<const uint2*>(f.words) + row * kWvRowWords + half * kHalf;
  const int e0 = 16 * half * kHalf + kCoopDigitBase;
  double t = 0.0;
  unsigned n = 0;
  bool o = false;
#pragma unroll 1
  for (int k = 0; k < kHalf; ++k) {  // rare path: a rolled loop keeps its registers few
    const uint2 x = wr[k];
    n += x.y >> 16;
    const int word = half * kHalf + k;
    if (word == kWvOvfWord) o = (x.y >> 16) != 0u;
    if (word < kWvOvfWord) {
      const double d = __builtin_amdgcn_ldexp(static_cast<double>(x.y & 0xffffu), 32) + static_cast<double>(x.x);
      t += __builtin_amdgcn_ldexp(d, e0 + 16 * k);
    }
  }
  t += lane_xor<32>(t);
  count = n + lane_xor_u<32>(n);
  ovf = o;
  return t > 0.0 ? static_cast<float>(1.0 / t) : 0.f;
}

// Direct-to-LDS copy of head h's accumulator words into finisher buffer
// h % kWvFinBufs (which must be free or already h's).
__device__ __forceinline__ void wv_stage(const WvCtx& c, int h, int lane) {
  const int b = h & (kWvFinBufs - 1);
  WvFin& f = c.fin[b];
  asm volatile("" ::: "memory");
  if (c.sh->fin_owner[b] != h) {
    // taken by compare-and-swap (two finisher waves of a workgroup, heads
    // G apart, map to the same buffer); while another head holds it (only if
    // its finisher had to retry for rounds) a bounded wait, then taken anyway
    int prev = 0;
    for (unsigned polls = 0; polls < kWvSpin; ++polls) {
      if (lane == 0) prev = atomicCAS(&c.sh->fin_owner[b], -1, h);
      prev = __builtin_amdgcn_readfirstlane(prev);
      if (prev == -1 || prev == h) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (prev != -1 && prev != h && lane == 0) c.sh->fin_owner[b] = h;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  const unsigned long long* a = c.acc + static_cast<int64_t>(h) * kCoopHeadWords;
  constexpr int kHalf = kWvRowWords / 2;  // 16-byte pieces per row
#pragma unroll
  for (int i = 0; i < 32 * kHalf / 64; ++i) {
    const int piece = i * 64 + lane, prow = piece / kHalf, pj = piece - prow * kHalf;
    __builtin_amdgcn_global_load_lds(a + prow * kCoopRowWords + pj * 2, (lds_void*)(f.words + i * 128), 16, 0,
                                     16 /* sc1 */);
  }
}

// The finisher's work for head h: stage the words, wait for them, and once
// every window row has all G contributions (else stage again: one may still
// be in flight; bounded) publish the vote weights (0 for a flagged head,
// whose votes are recomputed). Staging and use within one call, with a full
// wait between them, leave no direct load into LDS in flight behind it.
__device__ __forceinline__ void wv_publish(const WvCtx& c, WvPipe& p, int h, int lane) {
  const int ln = opaque(lane), row = ln & 31;
  const WvFin& f = c.fin[h & (kWvFinBufs - 1)];
  for (unsigned t = 0; t < c.spin; ++t) {
    wv_stage(c, h, ln);
    wait_vm_all();
    unsigned count;
    bool ovf;
    float wv = wv_words_to_w(f, ln, count, ovf);
    if (__ballot(row < c.w && count != static_cast<unsigned>(c.tgt)) == 0ull) {
      if (__ballot(ovf) != 0ull) wv = 0.f;
      if (ln < 32 && row < c.w) st_agent_u2(&c.stat[h * 32 + row], make_uint2(__float_as_uint(wv), 1u));
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // buffer read before it is released
      if (ln == 0) c.sh->fin_owner[h & (kWvFinBufs - 1)] = -1;
      asm volatile("" ::: "memory");
      return;
    }
    __builtin_amdgcn_s_sleep(2);  // a contribution is still in flight
  }
  p.gave_up = true;
  if (ln == 0) __hip_atomic_store(c.status, 3u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The merge of head h (sequence index idx) for this workgroup, by its
// designated wave, once all kWvWaves waves have stored their row sums in slot
// idx & 1: the sums added in wave order, the slot reopened for sequence index
// idx + 2, the result added to the
// head's accumulators, and the head's count raised (no return is waited for).
// The head's finisher, fixed in advance, reads the count and, once all G
// workgroups have counted, stages and converts the words (which carry their
// own contribution counts, so an increment need not wait for its
// contributions to land).
__device__ __forceinline__ void wv_try_merge(const WvCtx& c, WvPipe& p, int lane) {
  WvShared* sh = c.sh;
  const int h = p.merge_head, idx = c.small ? p.merge_idx : h, sl = idx & 1, ln = opaque(lane), col = ln & 31;
  asm volatile("" ::: "memory");
  if (__builtin_amdgcn_readfirstlane(sh->mcnt[sl]) != kWvWaves) return;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  float L = sh->lslot[sl][0][col];
#pragma unroll
  for (int wv = 1; wv < kWvWaves; ++wv) L += sh->lslot[sl][wv][col];
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // sums read before the slot reopens
  if (ln == 0) {
    sh->mcnt[sl] = 0;
    sh->mtag[sl] = idx + 2;
  }
  asm volatile("" ::: "memory");
  if (ln < 32 && col < c.w) wv_add_sum(c.acc + static_cast<int64_t>(h) * kCoopHeadWords, col, L);
  if (ln == 0) atomicAdd(&c.cnt[h * kCoopCtrWords] + opaque(0), 1u);
  p.merge_head = -1;
}

// Finishers. Head h is finished by wave (h / G) % kWvWaves of workgroup
// h % G, so that the finishing work (a staging round trip and the
// conversion) is spread over the workgroups rather than given to the last
// one to count, which is the one furthest behind: as finisher it would fall
// further behind and stay last. A finisher reads its head's count (agent
// scope) every round once it has reached the head, and publishes at the start
// of the round after the count shows all G workgroups.
__device__ __forceinline__ void wv_finish(const WvCtx& c, WvPipe& p, int lane) {
  wv_publish(c, p, p.fin_head, lane);
  p.fin_head += c.W;
  p.fin_cnt = 0u;
}

// The same inside a bounded wait: the count read now, after the full wait.
__device__ __forceinline__ void wv_finish_poll(const WvCtx& c, WvPipe& p, int lane) {
  if (p.fin_head >= c.BH) return;
  const unsigned n = __hip_atomic_load(&c.cnt[p.fin_head * kCoopCtrWords], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (static_cast<unsigned>(__builtin_amdgcn_readfirstlane(n)) == static_cast<unsigned>(c.tgt)) wv_finish(c, p, lane);
}

// Work this wave owes other waves, done after a full wait (every memory
// operation it issued before is complete): merge its workgroup's sums of a
// head it is designated for, and (in a bounded wait) finish its head if that
// head's count is complete. Every bounded wait of the kernel calls it, so
// that no wave waits for something it owes itself.
__device__ __forceinline__ void wv_service(const WvCtx& c, WvPipe& p, int lane) {
  if (p.merge_head >= 0) wv_try_merge(c, p, lane);
  wv_finish_poll(c, p, lane);
}

// The next round's prefetches: the vote weights for its votes (head
// pre_head) and the reference score of its tile (head ref_head).
// (Addresses here and in the votes are a uniform base plus an unsigned 32-bit
// lane offset, which the scalar-base addressing form takes directly.)
template <int PAR>
__device__ __forceinline__ void wv_prefetch(const WvCtx& c, WvPipe& p, int pre_head, int ref_head, int lane) {
  const unsigned row = static_cast<unsigned>(lane & 31);
  p.pre[PAR ^ 1] = ld_agent_u2(reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(c.stat + pre_head * 32) +
                                                              row * 8u));
  p.rref[PAR ^ 1] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(c.ref + ref_head * 32) + row * 4u);
}

// Votes of the tile (head hv, tile tv) whose e_ij are in s, with the weights
// `pre` prefetched a round ago (waited for, bounded, if the head is not yet
// published). Rows past the window have weight 0 (never published).
__device__ __forceinline__ void wv_votes(const WvCtx& c, WvPipe& p, uint2 pre, const f32x16_t& s, int hv, int tv,
                                         int lane) {
  const int row = lane & 31, half = lane >> 5;
  if (__builtin_expect(!p.gave_up && __ballot(row < c.w && pre.y != 1u) != 0ull, 0)) {
    unsigned polls = 0;
    bool late;
    do {
      __builtin_amdgcn_s_sleep(2);
      pre = ld_agent_u2(&c.stat[hv * 32 + row]);
      wait_vm_all();  // every exit from here has its load back
      wv_service(c, p, lane);  // what this wave owes others may be what it waits for
      late = __ballot(row < c.w && pre.y != 1u) != 0ull;
    } while (late && ++polls < c.spin);
    if (late) {  // a protocol failure: record it and never wait again
      p.gave_up = true;
      if (lane == 0) __hip_atomic_store(c.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  float* ws = c.sh->s_wr[c.wave];
  if (half == 0) ws[row] = __uint_as_float(pre.x);
  float v = 0.f;
#pragma unroll
  for (int a = 0; a < 4; ++a) {  // registers 4a..4a+3 hold rows 8a + 4 half + 0..3
    const f32x4_t ww = *reinterpret_cast<const f32x4_t*>(ws + 8 * a + 4 * half);
#pragma unroll
    for (int e = 0; e < 4; ++e) v = fmaf(s[4 * a + e], ww[e], v);
  }
  v += lane_xor<32>(v);
  const int j = tv * kTile + row;
  float* vrow = c.vote + static_cast<int64_t>(hv) * c.t0 + tv * kTile;  // uniform
  // nontemporal: the K stream reads faster beside streaming stores than beside plain ones
  if (half == 0 && j < c.t0)
    __builtin_nontemporal_store(v, reinterpret_cast<float*>(reinterpret_cast<char*>(vrow) + static_cast<unsigned>(row) * 4u));
}

// This wave has scored its last tile of head h: its per-lane row sums are
// reduced across the lanes of each half (a transposing butterfly: after the
// steps over lane bits 0..3 a lane keeps register bitrev4(lane & 15); a last
// step adds the partner across bit 4), the results go to slot idx & 1 of the
// workgroup (idx: the head's index in the workgroup's sequence of heads; once
// the slot is open for idx), and the designated wave (idx + g) % kWvWaves
// merges them when all waves have stored theirs (now if it is the last, else
// at a later service). A non-finite sum flags the head.
// (a & m) | (b & ~m) for a mask m that is all ones or all zeros per lane: the
// lane-dependent choice between two registers, written so that the compiler
// cannot turn it into an indexed read of the register array (which it lowers
// as a chain of compares and selects over all sixteen elements).
__device__ __forceinline__ float lane_pick(float a, float b, unsigned m) {
  return __uint_as_float((__float_as_uint(a) & m) | (__float_as_uint(b) & ~m));
}

__device__ __forceinline__ void wv_head_end(const WvCtx& c, WvPipe& p, int h, int idx, f32x16_t& ls, int lane) {
  const int ln = opaque(lane);
  // step over lane bit k: a lane with the bit set keeps the upper half of its
  // registers and sends the lower half (masks opaque, all ones where the bit is set)
  const unsigned m1 = opaque(-(ln & 1)), m2 = opaque(-((ln >> 1) & 1)), m4 = opaque(-((ln >> 2) & 1)),
                 m8 = opaque(-((ln >> 3) & 1));
  float x8[8], x4[4], x2[2], x1;
#pragma unroll
  for (int i = 0; i < 8; ++i) x8[i] = lane_pick(ls[i + 8], ls[i], m1) + lane_xor<1>(lane_pick(ls[i], ls[i + 8], m1));
#pragma unroll
  for (int i = 0; i < 4; ++i) x4[i] = lane_pick(x8[i + 4], x8[i], m2) + lane_xor<2>(lane_pick(x8[i], x8[i + 4], m2));
#pragma unroll
  for (int i = 0; i < 2; ++i) x2[i] = lane_pick(x4[i + 2], x4[i], m4) + lane_xor<4>(lane_pick(x4[i], x4[i + 2], m4));
  x1 = lane_pick(x2[1], x2[0], m8) + lane_xor<8>(lane_pick(x2[0], x2[1], m8));
  x1 += lane_xor<16>(x1);
#pragma unroll
  for (int i = 0; i < 16; ++i) ls[i] = 0.f;
  const int r = ((ln & 1) << 3) | ((ln & 2) << 1) | ((ln & 4) >> 1) | ((ln & 8) >> 3);
  const int row = acc_row(r, ln >> 5);
  if (__builtin_expect(__ballot(!(x1 <= 3.0e38f)) != 0ull, 0) && ln == 0) atomicOr(&c.cnt[h * kCoopCtrWords + 16], 1u);
  WvShared* sh = c.sh;
  const int sl = idx & 1;
  // plain LDS reads behind compiler barriers: an atomic load here would make
  // the compiler wait for the direct loads in flight into the tile ring
  asm volatile("" ::: "memory");
  if (__builtin_expect(!p.gave_up && sh->mtag[sl] != idx, 0)) {
    // the slot still holds the workgroup's head before last (its merge is pending)
    unsigned polls = 0;
    bool late;
    do {
      __builtin_amdgcn_s_sleep(1);
      wait_vm_all();
      wv_service(c, p, ln);
      asm volatile("" ::: "memory");
      late = sh->mtag[sl] != idx;
    } while (late && ++polls < c.spin);
    if (late) {
      p.gave_up = true;
      if (ln == 0) __hip_atomic_store(c.status, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if ((ln & 16) == 0) sh->lslot[sl][c.wave][row] = x1;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the sums are in LDS before the count says so
  if (ln == 0) lds_add(&sh->mcnt[sl], 1);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  // the merging wave is (idx + g) % kWvWaves: a wave merges sequence index
  // idx again only at idx + kWvWaves, and before that, at idx + 2, its
  // slot's wait has needed the merge of idx done, so a wave never owes two
  // merges (with the head in place of idx, a head that advances by a multiple
  // of kWvWaves from one round to the next would give one wave both merges)
  if (c.wave == ((idx + c.g) & (kWvWaves - 1))) {
    p.merge_head = h;
    p.merge_idx = idx;
    wv_try_merge(c, p, ln);
  }
}

// A wave's first tile of a head: the head's query fragments from query slot
// seq & 1, once the queries have landed there (bounded wait), where seq is the
// head's index in the workgroup's sequence of heads (every head in order, or
// one head per round when heads are shorter than a round). Every wave of a
// workgroup works on the same head in a round (tile counts are padded to
// whole groups of kWvWaves), so a workgroup loads each head's queries once;
// the last of its waves to read them loads, into the same slot, the queries
// of the head two on in the sequence, and marks them landed at the start of
// its next round.
template <int D>
__device__ __forceinline__ void wv_take_q(const WvCtx& c, WvPipe& p, const WvPos& pos, const WvPos& nxt, int r,
                                          bf16x8_t (&qf)[D / 16], int lane) {
  using Ly = WvLayout<D>;
  constexpr int KS = D / 16;
  const int seq = c.small ? r : pos.head;
  const int sl = seq & 1;
  WvShared* sh = c.sh;
  // plain LDS reads behind compiler barriers (see wv_head_end)
  asm volatile("" ::: "memory");
  if (__builtin_expect(!p.gave_up && sh->qtag[sl] != seq, 0)) {
    unsigned polls = 0;
    bool late;
    do {
      __builtin_amdgcn_s_sleep(1);
      wait_vm_all();
      wv_service(c, p, lane);
      asm volatile("" ::: "memory");
      late = sh->qtag[sl] != seq;
    } while (late && ++polls < c.spin);
    if (late) {
      p.gave_up = true;
      if (lane == 0) __hip_atomic_store(c.status, 5u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const unsigned char* qt = c.qs + sl * Ly::kTileB;
  const int col = lane & 31, half = lane >> 5;
  const unsigned A = static_cast<unsigned>(col * Ly::kRowB) +
                     (static_cast<unsigned>((half * (Ly::kP / 2)) ^ (col & (Ly::kP - 1))) << 4);
#pragma unroll
  for (int s = 0; s < KS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(qt + (A ^ static_cast<unsigned>(s << 4))));
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the slot can be refilled
  p.qhead = pos.head;
  int before = 0;
  if (lane == 0) before = lds_add_rtn_i(&sh->qreads[sl], 1);
  before = __builtin_amdgcn_readfirstlane(before);
  if (before == kWvWaves - 1) {
    // every wave has read them: the slot takes the queries of sequence index seq + 2
    if (lane == 0) sh->qreads[sl] = 0;
    const int nseq = seq + 2;
    if (c.small ? r + 2 < c.rounds : nseq < c.BH) {
      // heads shorter than a round: the head of round r + 2, one round past nxt
      const int nhead = c.small ? nxt.head + c.wq + (nxt.t + c.wr >= c.nt ? 1 : 0) : nseq;
      wv_issue_q<D>(c, wv_q_base(c, nhead), c.qs + sl * Ly::kTileB, lane);
      p.qpub = nseq;
    }
  }
}

template <int D, int BANK, int PAR>
__device__ __forceinline__ void wv_round(const WvCtx& c, WvPipe& p, WvPos& pos, f32x16_t (&sc)[kWvBanks],
                                         f32x16_t& ls, bf16x8_t (&qf)[D / 16], unsigned char* ring0,
                                         unsigned char* ring1, int r) {
  using Ly = WvLayout<D>;
  constexpr int KS = D / 16;
  // BANK = r % kWvBanks, PAR = r % 2 (the ring slot and prefetch parity)
  if (r >= c.rounds + kWvBanks) return;  // past the last votes
  const bool do_a = r < c.rounds;
  const bool do_b = r >= kWvBanks && r - kWvBanks < c.rounds;
  // this round's tile, Q and reference score, and everything issued last round
  wait_vm_all();
  const int lane = opaque(lane_id());
  if (__builtin_expect(p.fin_head < c.BH &&
                           static_cast<unsigned>(__builtin_amdgcn_readfirstlane(p.fin_cnt)) ==
                               static_cast<unsigned>(c.tgt), 0))
    wv_finish(c, p, lane);
  const WvPos nxt = wv_next(c, pos);
  const bool more = r + 1 < c.rounds;
  if (p.qpub >= 0) {
    // the queries this wave loaded into a query slot last round have landed
    // (the wait above): mark them for the workgroup
    if (lane == 0) c.sh->qtag[p.qpub & 1] = p.qpub;
    p.qpub = -1;
  }
  if (more) wv_issue_k<D>(c, nxt, PAR ? ring0 : ring1, lane);
  if (do_a && pos.head != p.qhead) wv_take_q<D>(c, p, pos, nxt, r, qf, lane);
  // the tile whose votes come next round: tile r - 8 (tile 0 before round 9)
  int vn_head = p.vhead, vn_t = p.vtile;
  if (r >= kWvBanks) wv_next_ht(c, vn_head, vn_t);
  // the votes of the tile of round r - 9 first, from the bank this round's
  // MFMAs then write; then the next round's prefetches (the weights read a
  // whole round before their votes); then this tile's MFMAs, the e_ij and the
  // row sums
  if (do_b) wv_votes(c, p, p.pre[PAR], sc[BANK], p.vhead, wv_rot(c, p.vhead, p.vtile), lane);
  if (r >= kWvBanks) {
    p.vhead = vn_head;
    p.vtile = vn_t;
  }
  wv_prefetch<PAR>(c, p, min(vn_head, c.BH - 1), min(more ? nxt.head : pos.head, c.BH - 1), lane);
  // the count of the head this wave finishes, once the wave has reached it
  if (p.fin_head < c.BH && (pos.head >= p.fin_head || !do_a))
    p.fin_cnt = __hip_atomic_load(&c.cnt[p.fin_head * kCoopCtrWords], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (do_a) {
    f32x16_t acc = {};
    const int col = lane & 31, half = lane >> 5;
    // fragment k-step s of row col: piece half*kP/2 + s at slot piece ^ (col & (kP-1)),
    // i.e. address A ^ (s << 4) (the tile's rows start at multiples of 256 bytes)
    const unsigned char* tile = PAR ? ring1 : ring0;
    const unsigned A = static_cast<unsigned>(col * Ly::kRowB) +
                       (static_cast<unsigned>((half * (Ly::kP / 2)) ^ (col & (Ly::kP - 1))) << 4);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t kf =
          __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(tile + (A ^ static_cast<unsigned>(s << 4))));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[s], kf, acc, 0, 0, 0);
      if (s % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // bound the fragments in flight
    }
    float* rs = c.sh->s_wr[c.wave];  // the votes above have read their weights
    if (half == 0) rs[col] = p.rref[PAR];  // R_i of this tile's head, read back per register below
    // e_ij = 2^(s_ij - R_i) for key j = key0 + col and the lane's 16 rows i
    const int key0 = pos.a * kTile;
    const bool full = key0 + kTile <= c.t0;  // every row sees every key of the tile
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4_t rr = *reinterpret_cast<const f32x4_t*>(rs + 8 * a + 4 * half);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * a + e;
        float x = fast_exp2(fmaf(acc[i], c.scale_log2, -rr[e]));
        if (__builtin_expect(!full, 0)) {
          const int j = key0 + col;
          x = (j < c.L && j <= c.t0 + acc_row(i, half)) ? x : 0.f;
        }
        sc[BANK][i] = x;
        ls[i] += x;
      }
    }
    if (!more || nxt.head != pos.head) wv_head_end(c, p, pos.head, c.small ? r : pos.head, ls, lane);
  }
  pos = nxt;
  // a merge still owed after a full wait (the next round starts with that
  // wait anyway: it only comes earlier)
  if (__builtin_expect(p.merge_head >= 0, 0)) {
    wait_vm_all();
    wv_try_merge(c, p, lane);
  }
}

// SHORT: heads shorter than a round (a compile-time choice, so that the
// long-head kernel carries none of the short-head code)
template <int D, bool SHORT>
__global__ __launch_bounds__(kWvThreads, 1) void snap_wave_bf16(
    const uint16_t* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qst, int qrow0,
    const uint16_t* __restrict__ k, int64_t ksb, int64_t ksh, int64_t kst, int H, int L, int w, int nt,
    int total_tiles, int BH, float scale_log2, const float* __restrict__ ref, unsigned long long* __restrict__ acc,
    unsigned* __restrict__ cnt, uint2* __restrict__ stat, unsigned* __restrict__ status, float* __restrict__ vote,
    unsigned* __restrict__ gate, unsigned gate_target, unsigned gate_spin, unsigned wait_spin) {
  using Ly = WvLayout<D>;
  // the two tile slots of every wave's ring, as two arrays: the reads of one
  // slot are then known not to alias the direct loads in flight into the other
  __shared__ __attribute__((aligned(1024))) unsigned char ring_even[kWvWaves * Ly::kTileB];
  __shared__ __attribute__((aligned(1024))) unsigned char ring_odd[kWvWaves * Ly::kTileB];
  // the workgroup's two query slots (slot s at s * kTileB), an array of their own
  __shared__ __attribute__((aligned(1024))) unsigned char qslot[2 * Ly::kTileB];
  __shared__ __attribute__((aligned(16))) WvShared sh;
  __shared__ __attribute__((aligned(16))) WvFin fin[kWvFinBufs];

  WvCtx c;
  c.q = q; c.qsb = qsb; c.qsh = qsh; c.qst = qst; c.qrow0 = qrow0;
  c.k = k; c.ksb = ksb; c.ksh = ksh; c.kst = kst;
  c.H = H; c.L = L; c.w = w; c.t0 = L - w; c.nt = nt; c.BH = BH;
  c.fin = fin;
  c.G = static_cast<int>(gridDim.x); c.g = static_cast<int>(blockIdx.x); c.W = c.G * kWvWaves;
  c.small = SHORT;
  c.wq = SHORT ? c.W / nt : 0;
  c.wr = SHORT ? c.W - c.wq * nt : 0;
  c.h_rcp = static_cast<unsigned>(
      min((0x100000000ull + static_cast<unsigned long long>(H) - 1) / static_cast<unsigned long long>(H),
          0xFFFFFFFFull));
  c.tgt = SHORT ? nt / kWvWaves : c.G;
  c.rounds = (total_tiles - c.g * kWvWaves + c.W - 1) / c.W;  // the same for the workgroup's waves
  c.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  c.tile_b = static_cast<int64_t>(kTile) * kst * 2;
  c.dk_head = ksh * 2;
  c.dk_batch = (ksb - H * ksh) * 2;
  c.spin = wait_spin;
  c.scale_log2 = scale_log2;
  c.ref = ref; c.acc = acc; c.cnt = cnt; c.stat = stat; c.status = status; c.vote = vote;
  c.sh = &sh;
  c.qs = qslot;
  unsigned char* ring0 = ring_even + c.wave * Ly::kTileB;
  unsigned char* ring1 = ring_odd + c.wave * Ly::kTileB;
  if (threadIdx.x == 0) {
    sh.mcnt[0] = sh.mcnt[1] = 0;
    sh.mtag[0] = 0;  // a workgroup's heads in order (all heads, or one per round for short heads)
    sh.mtag[1] = 1;
    sh.qtag[0] = sh.qtag[1] = -1;
    sh.qreads[0] = sh.qreads[1] = 0;
  }
  if (threadIdx.x < kWvFinBufs) sh.fin_owner[threadIdx.x] = -1;
  WvPipe p;
  p.merge_head = p.merge_idx = -1;
  p.fin_head = c.g + c.G * c.wave;
  p.fin_cnt = 0u;
  p.pre[0] = p.pre[1] = make_uint2(0u, 0u);
  p.rref[0] = p.rref[1] = 0.f;
  p.gave_up = false;
  p.qhead = -1;
  p.qpub = -1;
  // round 0: tile v (of head 0 unless heads are shorter than a round)
  WvPos pos;
  {
    const int v = c.g * kWvWaves + c.wave;
    pos.head = SHORT ? v / nt : 0;
    pos.t = v - pos.head * nt;
    const int b = pos.head / H;
    pos.h = pos.head - b * H;
    pos.kh = reinterpret_cast<const char*>(k + b * ksb + pos.h * ksh);
    pos.a = wv_rot(c, pos.head, pos.t);
    pos.kt = pos.kh + static_cast<int64_t>(pos.a) * c.tile_b;
  }
  p.vhead = pos.head;
  p.vtile = pos.t;
  bf16x8_t qf[D / 16];
  if (c.rounds > 0) {
    const int lane = lane_id();
    wv_issue_k<D>(c, pos, ring0, lane);
    // the queries of the workgroup's first two heads (sequence indices 0 and
    // 1) into the query slots, by waves 0 and 1
    if (c.wave < 2 && (SHORT ? c.wave < c.rounds : c.wave < BH)) {
      const int head = SHORT ? (c.g * kWvWaves + c.wave * c.W) / nt : c.wave;
      wv_issue_q<D>(c, wv_q_base(c, head), qslot + c.wave * Ly::kTileB, lane);
      p.qpub = c.wave;
    }
    p.rref[0] = ref[pos.head * 32 + (lane & 31)];
  }
  // Residency check, in place of a launch that guarantees it (its wait
  // overlaps the first tile's loads): the waits below need every workgroup
  // resident at once. Each workgroup counts itself in on gate[0]; the one
  // whose count reaches gate_target opens the pass (gate[1]: 0 -> 1). A
  // workgroup still waiting after gate_spin polls closes it instead (0 -> 2):
  // some workgroups could not start while the others held the compute units.
  // One compare-and-swap decides, so every workgroup, late ones included,
  // takes the same branch; when the pass is closed every head is flagged and
  // the pooling kernel computes all votes exactly.
  __shared__ unsigned s_gate;
  if (threadIdx.x == 0) {
    if (atomicAdd(&gate[0], 1u) + 1u == gate_target) atomicCAS(&gate[1], 0u, 1u);
    unsigned st = __hip_atomic_load(&gate[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (unsigned polls = 0; st == 0u && polls < gate_spin; ++polls) {
      __builtin_amdgcn_s_sleep(2);
      st = __hip_atomic_load(&gate[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (st == 0u) {
      const unsigned prev = atomicCAS(&gate[1], 0u, 2u);
      st = prev == 0u ? 2u : prev;
    }
    if (st != 1u)
      for (int h = 0; h < BH; ++h) atomicOr(&cnt[h * kCoopCtrWords + 16], 1u);
    s_gate = st;
  }
  __syncthreads();  // also: the slot counters are set
  if (s_gate != 1u) {
    wait_vm_all();  // no direct load may still be landing in LDS when the wave ends
    return;
  }

  f32x16_t sc[kWvBanks];
  f32x16_t ls = {};
  static_assert(kWvBanks == 9, "the round loop below is unrolled over the register banks and ring slots");
  // the last tile's votes fall in round rounds - 1 + kWvBanks, and the last
  // head's publication a few rounds after its last tile; the loop body is
  // 18 rounds (bank r % 9, ring slot r % 2)
  for (int r0 = 0; r0 < c.rounds + kWvBanks; r0 += 2 * kWvBanks) {
    wv_round<D, 0, 0>(c, p, pos, sc, ls, qf, ring0, ring1, r0);
    wv_round<D, 1, 1>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 1);
    wv_round<D, 2, 0>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 2);
    wv_round<D, 3, 1>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 3);
    wv_round<D, 4, 0>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 4);
    wv_round<D, 5, 1>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 5);
    wv_round<D, 6, 0>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 6);
    wv_round<D, 7, 1>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 7);
    wv_round<D, 8, 0>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 8);
    wv_round<D, 0, 1>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 9);
    wv_round<D, 1, 0>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 10);
    wv_round<D, 2, 1>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 11);
    wv_round<D, 3, 0>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 12);
    wv_round<D, 4, 1>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 13);
    wv_round<D, 5, 0>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 14);
    wv_round<D, 6, 1>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 15);
    wv_round<D, 7, 0>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 16);
    wv_round<D, 8, 1>(c, p, pos, sc, ls, qf, ring0, ring1, r0 + 17);
  }
  // work still owed after the last round: a pending merge, heads still to
  // finish (bounded)
  for (unsigned t = 0; (p.merge_head >= 0 || p.fin_head < c.BH) && !p.gave_up && t < c.spin; ++t) {
    wait_vm_all();
    __builtin_amdgcn_s_sleep(2);
    wv_service(c, p, lane_id());
  }
  // a finisher that ran out of time here (a wait that gave up earlier has
  // recorded its own code already)
  if (p.fin_head < c.BH && !p.gave_up && lane_id() == 0)
    __hip_atomic_store(status, 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exact votes of the heads the single pass flagged (a score more than 2^127
// above its row's reference; every head when the independent-wave kernel's
// workgroups could not all be resident, or when a bounded wait of a score
// kernel ran out, which leaves a non-zero status word), recomputed in fp32 by the pooling
// kernel's workgroups, each for the positions it pools: one plain pass over
// the head's keys gives every window row's (max, sum of 2^(s - m)), then the
// vote of a position is sum_i 2^(s_i - c_i) with c_i = m_i + log2 sum_i.
// Every workgroup of a flagged head repeats the first pass: a fallback for
// inputs far outside the usual range, not a fast path.
struct ExactArgs {
  const uint16_t* q;
  int64_t qsb, qsh, qst;
  int qrow0;
  const uint16_t* k;
  int64_t ksb, ksh, kst;
  int H, L, w, D;
  float scale_log2;
  const unsigned* flags;   // per head at word 16 of its counters; NULL: no head is flagged
  const unsigned* status;  // the score kernel's failure code (non-zero: every head flagged); NULL: none
};

constexpr int kExactMaxWaves = 16;  // the largest workgroup that computes exact votes (1024 threads)

struct ExactShared {
  float qs[kMaxWindow][128];
  float red_m[kExactMaxWaves][kMaxWindow], red_l[kExactMaxWaves][kMaxWindow];
  float cst[kMaxWindow];
};

// A pooling workgroup's LDS: the histogram, or (before it, for a flagged
// head) the exact recomputation's rows and statistics.
union PoolShared {
  unsigned sh[kHistBins];
  ExactShared es;
};

__device__ __forceinline__ bool exact_flagged(const ExactArgs& a, int bh) {
  return (a.status && a.status[0] != 0u) || (a.flags && a.flags[bh * kCoopCtrWords + 16] != 0u);
}

// Rows 8g .. 8g+7 of the window's fp32 scores against key j (rows past w
// are zero rows). Eight rows at a time keep the fallback's registers few: the
// pooling kernels that carry it must keep their occupancy.
constexpr int kExactRows = 8;

__device__ __forceinline__ void exact_scores(const ExactShared& e, const ExactArgs& a, const uint16_t* kb, int j,
                                             int g, float (&s)[kExactRows]) {
#pragma unroll
  for (int i = 0; i < kExactRows; ++i) s[i] = 0.f;
  for (int d = 0; d < a.D; ++d) {
    const float kv = bf16_to_f32(kb[static_cast<int64_t>(j) * a.kst + d]);
#pragma unroll
    for (int i = 0; i < kExactRows; ++i) s[i] = fmaf(e.qs[g * kExactRows + i][d], kv, s[i]);
  }
}

// The head's window rows into LDS, then c_i from one pass over its keys per
// group of rows (every thread of the workgroup calls it).
__device__ void exact_prepare(ExactShared& e, const ExactArgs& a, int bh) {
  // any workgroup of whole waves up to kExactMaxWaves of them
  const int nthreads = static_cast<int>(blockDim.x), nwaves = nthreads / kWave;
  const int b = bh / a.H, h = bh - b * a.H, t0 = a.L - a.w, wave = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kMaxWindow * a.D; i += nthreads) {
    const int rr = i / a.D, d = i - rr * a.D;
    e.qs[rr][d] = rr < a.w ? bf16_to_f32(a.q[b * a.qsb + h * a.qsh + static_cast<int64_t>(a.qrow0 + rr) * a.qst + d])
                           : 0.f;
  }
  __syncthreads();
  const uint16_t* kb = a.k + b * a.ksb + h * a.ksh;
#pragma unroll 1
  for (int g = 0; g < kMaxWindow / kExactRows; ++g) {
    float m[kExactRows], l[kExactRows];
#pragma unroll
    for (int i = 0; i < kExactRows; ++i) {
      m[i] = kNegBig;
      l[i] = 0.f;
    }
    for (int j = threadIdx.x; j < a.L; j += nthreads) {
      float s[kExactRows];
      exact_scores(e, a, kb, j, g, s);
#pragma unroll
      for (int i = 0; i < kExactRows; ++i) {
        const int row = g * kExactRows + i;
        if (row < a.w && j <= t0 + row) lse2_merge(m[i], l[i], s[i] * a.scale_log2, 1.f);
      }
    }
#pragma unroll
    for (int i = 0; i < kExactRows; ++i) {
      lse2_merge(m[i], l[i], lane_xor<32>(m[i]), lane_xor<32>(l[i]));
      lse2_merge(m[i], l[i], lane_xor<16>(m[i]), lane_xor<16>(l[i]));
      lse2_merge(m[i], l[i], lane_xor<8>(m[i]), lane_xor<8>(l[i]));
      lse2_merge(m[i], l[i], lane_xor<4>(m[i]), lane_xor<4>(l[i]));
      lse2_merge(m[i], l[i], lane_xor<2>(m[i]), lane_xor<2>(l[i]));
      lse2_merge(m[i], l[i], lane_xor<1>(m[i]), lane_xor<1>(l[i]));
      if (lane_id() == 0) {
        e.red_m[wave][g * kExactRows + i] = m[i];
        e.red_l[wave][g * kExactRows + i] = l[i];
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < kMaxWindow) {
    float mm = e.red_m[0][threadIdx.x], ll = e.red_l[0][threadIdx.x];
    for (int wv = 1; wv < nwaves; ++wv) lse2_merge(mm, ll, e.red_m[wv][threadIdx.x], e.red_l[wv][threadIdx.x]);
    e.cst[threadIdx.x] = mm + __builtin_amdgcn_logf(ll);
  }
  __syncthreads();
}

// The exact vote of prefix position j of head bh (after exact_prepare).
__device__ float exact_vote(const ExactShared& e, const ExactArgs& a, int bh, int j) {
  const int b = bh / a.H, h = bh - b * a.H;
  const uint16_t* kb = a.k + b * a.ksb + h * a.ksh;
  float v = 0.f;
#pragma unroll 1
  for (int g = 0; g < kMaxWindow / kExactRows; ++g) {
    float s[kExactRows];
    exact_scores(e, a, kb, j, g, s);
#pragma unroll
    for (int i = 0; i < kExactRows; ++i)
      if (g * kExactRows + i < a.w) v += fast_exp2(s[i] * a.scale_log2 - e.cst[g * kExactRows + i]);
  }
  return v;
}

// Max- or average-pool of raw votes (neighbours beyond the prefix ignored) and
// the per-head 12-bit histogram of the pooled scores, after the single pass. A
// thread pools kPoolPer consecutive positions from a register window of their
// votes with a halo of R on each side (rounded up to whole 16-byte pieces);
// neighbouring pooled scores often share a histogram bin, so each run of equal
// bins is one LDS add.
constexpr int kPoolPer = 16;
constexpr int kPoolChunk = kThreads * kPoolPer;
constexpr int kPoolBigThreads = 1024;  // the large-layer form: 4x the positions per histogram
constexpr int kPoolBigChunk = kPoolBigThreads * kPoolPer;
constexpr int kPoolRegRadius = 7;  // larger radii pool from LDS (snap_pool_lds)

template <int R, bool VEC, int THREADS>
__global__ __launch_bounds__(THREADS) void snap_pool(float* __restrict__ vote, float* __restrict__ pooled,
                                                     unsigned* __restrict__ hist, int N, int avg,
                                                     const ExactArgs ea) {
  // pooled may be NULL: then only the histogram is produced
  constexpr int kHalo = (R + 3) / 4 * 4;
  constexpr int kX = kPoolPer + 2 * kHalo;
  __shared__ PoolShared ps;
  unsigned* sh = ps.sh;
  const int bh = blockIdx.y;
  const int j0 = (static_cast<int>(blockIdx.x) * THREADS + static_cast<int>(threadIdx.x)) * kPoolPer;
  float* vb = vote + static_cast<int64_t>(bh) * N;
  float x[kX];
  // the votes are loaded before the head's flag is known (its load would
  // otherwise delay theirs); a flagged head's exact votes replace them
  const bool vec_body = VEC && j0 >= kHalo && j0 + kPoolPer + kHalo <= N;
  if (vec_body) {
#pragma unroll
    for (int p = 0; p < kX / 4; ++p) {
      const f32x4_t f = *reinterpret_cast<const f32x4_t*>(vb + j0 - kHalo + 4 * p);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * p + e] = f[e];
    }
  }
  if (exact_flagged(ea, bh)) {
    // exact votes (halo included) for a flagged head; the thread's own
    // positions go back to the vote buffer, where the selection and the
    // caller read them
    exact_prepare(ps.es, ea, bh);
    for (int i = 0; i < kX; ++i) {
      const int j = j0 - kHalo + i;
      x[i] = j >= 0 && j < N ? exact_vote(ps.es, ea, bh, j) : -__builtin_huge_valf();
      if (i >= kHalo && i < kHalo + kPoolPer && j < N) vb[j] = x[i];
    }
    __syncthreads();  // the rows are read before the histogram reuses their LDS
  } else if (!vec_body) {
#pragma unroll
    for (int i = 0; i < kX; ++i) {
      const int j = j0 - kHalo + i;
      x[i] = j >= 0 && j < N ? vb[j] : -__builtin_huge_valf();
    }
  }
  for (int i = threadIdx.x; i < kHistBins; i += THREADS) sh[i] = 0;
  float o[kPoolPer];
  if (avg) {
    // the mean of the in-range neighbours j-R .. j+R (summed in position order)
#pragma unroll
    for (int i = 0; i < kPoolPer; ++i) {
      const int j = j0 + i;
      float m = 0.f;
#pragma unroll
      for (int d = 0; d <= 2 * R; ++d) {
        const int jd = j - R + d;
        m += jd >= 0 && jd < N ? x[i + kHalo - R + d] : 0.f;
      }
      o[i] = m / static_cast<float>(min(j + R, N - 1) - max(j - R, 0) + 1);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPoolPer; ++i) {
      float m = x[i + kHalo - R];
#pragma unroll
      for (int d = 1; d <= 2 * R; ++d) m = fmaxf(m, x[i + kHalo - R + d]);
      o[i] = m;
    }
  }
  if (pooled) {  // the pooled scores are stored only when something reads them
    float* pr = pooled + static_cast<int64_t>(bh) * N + j0;
    if (VEC && j0 + kPoolPer <= N) {
#pragma unroll
      for (int p = 0; p < kPoolPer / 4; ++p) {
        f32x4_t f;
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = o[4 * p + e];
        *reinterpret_cast<f32x4_t*>(pr + 4 * p) = f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPoolPer; ++i)
        if (j0 + i < N) pr[i] = o[i];
    }
  }
  __syncthreads();  // histogram cleared
  unsigned run_bin = 0, run = 0;
#pragma unroll
  for (int i = 0; i < kPoolPer; ++i) {
    const unsigned bin = (__float_as_uint(o[i]) >> kHistShift) & (kHistBins - 1);
    if (j0 + i < N) {
      if (run && bin != run_bin) {
        atomicAdd(&sh[run_bin], run);
        run = 0;
      }
      run_bin = bin;
      ++run;
    }
  }
  if (run) atomicAdd(&sh[run_bin], run);
  __syncthreads();
  flush_hist(sh, hist + static_cast<int64_t>(bh) * kHistBins);
}

// The same for pooling radii beyond kPoolRegRadius: the chunk's votes and halo
// staged in LDS, one output position per thread and step.
__global__ __launch_bounds__(kThreads) void snap_pool_lds(float* __restrict__ vote, float* __restrict__ pooled,
                                                          unsigned* __restrict__ hist, int N, int r, int avg,
                                                          const ExactArgs ea) {
  __shared__ float sv[kPoolChunk + 2 * kMaxPoolRadius];
  __shared__ PoolShared ps;
  unsigned* sh = ps.sh;
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int c0 = chunk * kPoolChunk, c1 = min(N, c0 + kPoolChunk);
  const int e0 = max(0, c0 - r), e1 = min(N, c1 + r);
  float* vb = vote + static_cast<int64_t>(bh) * N;
  if (exact_flagged(ea, bh)) {  // exact votes of a flagged head, as in snap_pool
    exact_prepare(ps.es, ea, bh);
    for (int j = e0 + static_cast<int>(threadIdx.x); j < e1; j += kThreads) {
      sv[j - e0] = exact_vote(ps.es, ea, bh, j);
      if (j >= c0 && j < c1) vb[j] = sv[j - e0];
    }
    __syncthreads();  // the rows are read before the histogram reuses their LDS
  } else {
    for (int j = e0 + static_cast<int>(threadIdx.x); j < e1; j += kThreads) sv[j - e0] = vb[j];
  }
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) sh[i] = 0;
  __syncthreads();
  pool_and_count(sv, e0, e1, c0, c1, r, avg, pooled + static_cast<int64_t>(bh) * N, sh);
  __syncthreads();
  flush_hist(sh, hist + static_cast<int64_t>(bh) * kHistBins);
}

// ------------------------------------------------------------ selection
//
// The kk kept prefix positions of a head are those with the largest pooled
// scores, ties going to the lower position, written in ascending order. A
// position's key is its score's bits (scores are non-negative, so their bits
// order like their values) above its inverted position. Each head's prefix is
// split into kSelChunk-position ranges, one workgroup each:
//  1. every workgroup finds, from the head's 12-bit histogram, the bin b*
//     holding the kk-th largest key and the number `rem` of picks left among
//     that bin's members;
//  2. it classifies its range: positions in bins above b* become bits of the
//     head's bitmap (whole words, each stored once), members of b* go to the
//     head's candidate list (one slot reservation per workgroup); both are
//     stored at device scope and complete before the workgroup counts itself
//     finished;
//  3. the head's last workgroup to finish loads the bitmap and the
//     candidates, finds the rem-th largest candidate key (8-bit radix passes
//     below the bits b* fixes while more than a wave's worth of candidates
//     share the prefix, each digit found by one wave, then a direct rank
//     within one wave), adds the bits of the candidates at or above it and
//     compacts the bitmap into ascending positions.
// A head of at most one range is selected by one workgroup alone
// (snap_select_head): the same steps with the bitmap and candidates in LDS
// throughout, and no exchange through device memory.
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
static_assert(kSelWaves <= kExactMaxWaves, "exact votes may be computed by a workgroup of the selection's size");
static_assert(kHistBins >= kSelThreads, "the compaction keeps one run start per thread in the histogram's LDS");
constexpr int kSelPer = 4;                            // 16-byte score pieces per thread
constexpr int kSelChunk = kSelThreads * kSelPer * 4;  // positions per workgroup
constexpr int kCandLds = 4096;                        // candidates a workgroup holds in LDS
constexpr int kBitmapLds = 16384;                     // bitmap words kept in LDS (N <= 524288)
constexpr int kKeyFixed = 51;                         // key bits 63..51: the sign (clear) and the bin
constexpr int kSelMaxRad = 4;                         // pooling radius the selection applies to raw votes
constexpr unsigned kSelHistSpin = 1u << 14;           // polls for a head's histogram before counting it alone

__device__ __forceinline__ unsigned long long sel_key(unsigned u, unsigned j) {
  return (static_cast<unsigned long long>(u & 0x7FFFFFFFu) << 32) | static_cast<unsigned long long>(~j);
}

__device__ __forceinline__ unsigned load_word(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_word(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS fetch-and-add by each active lane, as written (no wave-level rewrite).
__device__ __forceinline__ unsigned lds_add_rtn(unsigned* p, unsigned v) {
  const unsigned a = static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned*)p));
  unsigned r;
  asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(a), "v"(v) : "memory");
  return r;
}

// Exclusive prefix sum over the block with one barrier; *total gets the block
// sum. `wsum` (kSelWaves words) may be written again only after a barrier.
__device__ __forceinline__ unsigned sel_block_scan(unsigned x, unsigned* wsum, unsigned* total) {
  const int w = static_cast<int>(threadIdx.x) / kWave;
  const unsigned incl = wave_incl_scan(x);
  if (lane_id() == kWave - 1) wsum[w] = incl;
  __syncthreads();
  unsigned before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const unsigned v = wsum[i];
    all += v;
    before += i < w ? v : 0u;
  }
  *total = all;
  return before + incl - x;
}

// The bin b holding the kk-th largest member of the LDS histogram h:
// count(bins > b) < kk <= count(bins >= b). Every thread calls it; *bin and
// *above are written before its closing barrier (left as they were if h holds
// fewer than kk members).
__device__ void sel_find_bin(const unsigned* h, unsigned kk, unsigned* wsum, unsigned* bin, unsigned* above) {
  constexpr int kPer = kHistBins / kSelThreads;
  const int t = threadIdx.x;
  unsigned c[kPer], sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    c[i] = h[t * kPer + i];
    sum += c[i];
  }
  unsigned total;
  const unsigned pre = sel_block_scan(sum, wsum, &total);
  const unsigned higher = total - pre - sum;  // members of bins owned by higher threads
  if (higher < kk && higher + sum >= kk) {
    unsigned run = higher;
#pragma unroll
    for (int i = kPer - 1; i >= 0; --i) {
      if (run + c[i] >= kk) {
        *bin = t * kPer + i;
        *above = run;
        break;
      }
      run += c[i];
    }
  }
  __syncthreads();
}

struct SelShared {
  unsigned bm[kBitmapLds];
  uint2 cand[kCandLds];
  unsigned sh[kHistBins];
  alignas(16) unsigned long long mem[kWave];
  unsigned wsum[kSelWaves];
  unsigned long long thr;
  unsigned bin, above, nloc, base, last, nmem, hist_in;
};

// A candidate found by this workgroup: held in LDS while there is room, else
// listed in the head's workspace list at once.
__device__ __forceinline__ void sel_add_cand(SelShared& s, unsigned* ctr_head, uint2* cand_g, int N, unsigned u,
                                             unsigned j, unsigned slot) {
  const uint2 c = make_uint2(u, j);
  if (slot < static_cast<unsigned>(kCandLds)) {
    s.cand[slot] = c;
  } else {
    const unsigned g = atomicAdd(&ctr_head[0], 1u);
    if (g < static_cast<unsigned>(N)) st_agent_u2(&cand_g[g], c);
  }
}

// OR over the 8 lanes of each aligned lane octet.
__device__ __forceinline__ unsigned octet_or(unsigned m) {
  m |= static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  m |= static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  m |= static_cast<unsigned>(__builtin_amdgcn_mov_dpp(static_cast<int>(m), 0x141, 0xF, 0xF, false));  // half-row mirror
  return m;
}

// One 16-byte piece f of scores (positions 4f .. 4f+3) per lane. The wave's
// pieces are consecutive and start at a multiple of 64, so the lanes of an
// octet hold the 32 positions of bitmap word f >> 3, which one of them stores.
__device__ __forceinline__ void sel_piece(SelShared& s, unsigned* bm_g, unsigned* ctr_head, uint2* cand_g, int N,
                                          f32x4_t x, int f, bool valid, unsigned bstar) {
  const int lane = lane_id();
  unsigned m = 0, nc = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const unsigned bin = (__float_as_uint(x[e]) >> kHistShift) & (kHistBins - 1);
    m |= static_cast<unsigned>(valid && bin > bstar) << e;
    nc += valid && bin == bstar;
  }
  m = octet_or(m << (4 * (lane & 7)));
  if (valid && (lane & 7) == 0) store_word(&bm_g[f >> 3], m);
  if (nc != 0u) {
    unsigned slot = lds_add_rtn(&s.nloc, nc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned u = __float_as_uint(x[e]);
      if (valid && ((u >> kHistShift) & (kHistBins - 1)) == bstar) {
        sel_add_cand(s, ctr_head, cand_g, N, u, static_cast<unsigned>(4 * f + e), slot);
        ++slot;
      }
    }
  }
}

// Whether a wave's 64 consecutive pieces can hold anything in bin b* or above:
// the largest raw vote (or pooled score) among its pieces and the pieces either
// side of each (`edge` holds a neighbouring piece for every lane) bounds every
// pooled score of the wave's positions, since pooling reaches at most
// kSelMaxRad <= 4 positions, one piece, away. A wave below b* has no bitmap bit
// and no candidate, so its classification reduces to storing zero words.
__device__ __forceinline__ bool sel_wave_reaches(f32x4_t cur, f32x4_t edge, unsigned bstar) {
  float m = fmaxf(fmaxf(fmaxf(cur[0], cur[1]), fmaxf(cur[2], cur[3])),
                  fmaxf(fmaxf(edge[0], edge[1]), fmaxf(edge[2], edge[3])));
  m = fmaxf(m, lane_xor<1>(m));
  m = fmaxf(m, lane_xor<2>(m));
  m = fmaxf(m, lane_xor<4>(m));
  m = fmaxf(m, lane_xor<8>(m));
  m = fmaxf(m, lane_xor<16>(m));
  m = fmaxf(m, lane_xor<32>(m));
  return ((__float_as_uint(m) >> kHistShift) & (kHistBins - 1)) >= bstar;
}

// The max-pool (radius rad <= kSelMaxRad, neighbours past the prefix ignored)
// of piece f of a row of raw votes, from the lane's piece `cur`, its wave
// neighbours' pieces (DPP wave shifts) and, for the wave's first and last lane,
// the piece beyond the wave (`edge`: piece f - 1 for lane 0, f + 1 for lane 63).
__device__ __forceinline__ f32x4_t sel_pool_piece(f32x4_t cur, f32x4_t edge, int f, int nf, int rad) {
  if (rad == 0) return cur;
  const float ninf = -__builtin_huge_valf();
  float x[12];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // wave_shr:1 gives lane l the value of lane l - 1 (lane 0 keeps `old`); wave_shl:1 of lane l + 1
    x[e] = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(edge[e]), __float_as_int(cur[e]), 0x138, 0xF,
                                                      0xF, false));
    x[4 + e] = cur[e];
    x[8 + e] = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(edge[e]), __float_as_int(cur[e]), 0x130, 0xF,
                                                          0xF, false));
  }
  if (f == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = ninf;
  }
  if (f + 1 >= nf) {  // past the row (the lanes there hold clamped copies)
#pragma unroll
    for (int e = 0; e < 4; ++e) x[8 + e] = ninf;
  }
  f32x4_t out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float m = x[4 + e];
#pragma unroll
    for (int d = 1; d <= kSelMaxRad; ++d)
      if (d <= rad) m = fmaxf(m, fmaxf(x[4 + e - d], x[4 + e + d]));
    out[e] = m;
  }
  return out;
}

// A piece's four pooled scores counted in the LDS histogram `sh` (a run of
// equal bins one add) and, if out is not NULL, stored there.
__device__ __forceinline__ void sel_count_piece(unsigned* sh, f32x4_t p, float* out) {
  unsigned run_bin = (__float_as_uint(p[0]) >> kHistShift) & (kHistBins - 1), run = 1;
#pragma unroll
  for (int e = 1; e < 4; ++e) {
    const unsigned bin = (__float_as_uint(p[e]) >> kHistShift) & (kHistBins - 1);
    if (bin != run_bin) {
      atomicAdd(&sh[run_bin], run);
      run_bin = bin;
      run = 0;
    }
    ++run;
  }
  atomicAdd(&sh[run_bin], run);
  if (out) *reinterpret_cast<f32x4_t*>(out) = p;
}

// The exact votes of piece f (positions 4f .. 4f + 3) of head bh.
__device__ f32x4_t sel_exact_piece(const ExactShared& e, const ExactArgs& a, int bh, int f) {
  f32x4_t x;
#pragma unroll 1
  for (int i = 0; i < 4; ++i) x[i] = exact_vote(e, a, bh, 4 * f + i);
  return x;
}

// The max-pool (radius rad) of position j of a row of N raw votes, one by one.
__device__ __forceinline__ float sel_pool_at(const float* pb, int j, int N, int rad) {
  float m = pb[j];
  for (int d = 1; d <= rad; ++d) {
    if (j - d >= 0) m = fmaxf(m, pb[j - d]);
    if (j + d < N) m = fmaxf(m, pb[j + d]);
  }
  return m;
}

// The head's kk kept positions once all its positions are classified: the
// bitmap holds the positions above the threshold bin bstar (in LDS s.bm when
// lds_bm, else bm_g), the bin's n_cand members are candidates (s.cand when
// in_lds, else cand_g), of which the rem with the largest keys are kept. One
// workgroup: the rem-th largest candidate key (8-bit radix passes below the
// bits bstar fixes while more than a wave's worth share the prefix, then a
// direct rank in one wave), the kept candidates' bits added, and the bitmap
// compacted into ascending positions.
__device__ void sel_rank_compact(SelShared& s, unsigned bstar, unsigned rem, unsigned n_cand, bool in_lds,
                                 const uint2* __restrict__ cand_g, unsigned* __restrict__ bm_g, bool lds_bm,
                                 int words, int N, int kk, int* __restrict__ out) {
  const int tid = threadIdx.x;
  unsigned long long prefix = static_cast<unsigned long long>(bstar) << kKeyFixed;
  unsigned long long pmask = ~0ull << kKeyFixed;
  unsigned long long thr = prefix;  // candidate keys >= thr are kept
  unsigned members = n_cand;        // candidates whose key matches prefix under pmask
  unsigned pass = 0;
  __syncthreads();
  for (int lo = kKeyFixed; members != rem && lo > 0;) {
    if (members <= static_cast<unsigned>(kWave)) {
      // direct rank of the few members left, by one wave: each lane counts
      // the members above its own, reading 16 keys per step (the unused slots
      // hold 0, below every key)
      if (tid == 0) {
        s.nmem = 0;
        s.thr = prefix;
      }
      if (tid < kWave) s.mem[tid] = 0ull;
      __syncthreads();
      for (unsigned i = tid; i < n_cand; i += kSelThreads) {
        const uint2 c = in_lds ? s.cand[i] : ld_agent_u2(&cand_g[i]);
        const unsigned long long key = sel_key(c.x, c.y);
        if ((key & pmask) == prefix) {
          const unsigned slot = lds_add_rtn(&s.nmem, 1u);
          if (slot < static_cast<unsigned>(kWave)) s.mem[slot] = key;
        }
      }
      __syncthreads();
      const unsigned nm = min(s.nmem, static_cast<unsigned>(kWave));
      if (static_cast<unsigned>(tid) < nm) {
        const unsigned long long mine = s.mem[tid];
        unsigned greater = 0;
        for (unsigned i = 0; i < nm; i += 16) {
          u64x2_t kv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) kv[e] = *reinterpret_cast<const u64x2_t*>(&s.mem[i + 2 * e]);
#pragma unroll
          for (int e = 0; e < 8; ++e) greater += (kv[e][0] > mine) + (kv[e][1] > mine);
        }
        if (greater + 1u == rem) s.thr = mine;  // keys are distinct: one lane at most
      }
      __syncthreads();
      thr = s.thr;
      break;
    }
    // an 8-bit digit: 256 bins, which one wave scans (4 per lane); the
    // passes alternate between two bin arrays, so that a pass's clear needs no
    // barrier after the previous pass's reads
    const int nb = lo >= 8 ? 8 : lo;
    lo -= nb;
    const unsigned dmask = (1u << nb) - 1u;
    unsigned* hb = s.sh + (pass++ & 1) * 256;
    if (tid < 256) hb[tid] = 0;
    if (tid == 0) {
      s.bin = 0;
      s.above = 0;
    }
    __syncthreads();
    for (unsigned i = tid; i < n_cand; i += kSelThreads) {
      const uint2 c = in_lds ? s.cand[i] : ld_agent_u2(&cand_g[i]);
      const unsigned long long key = sel_key(c.x, c.y);
      if ((key & pmask) == prefix) atomicAdd(&hb[static_cast<unsigned>(key >> lo) & dmask], 1u);
    }
    __syncthreads();
    if (tid < kWave) {  // wave 0: the digit holding the rem-th largest member
      unsigned c[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hb[4 * tid + i];
        sum += c[i];
      }
      const unsigned incl = wave_incl_scan(sum);
      const unsigned higher =
          static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1)) - incl;
      if (higher < rem && higher + sum >= rem) {
        unsigned run = higher;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          if (run + c[i] >= rem) {
            s.bin = 4 * tid + i;
            s.above = run;
            break;
          }
          run += c[i];
        }
      }
    }
    __syncthreads();
    const unsigned d = s.bin;
    rem -= s.above;
    members = hb[d];
    prefix |= static_cast<unsigned long long>(d) << lo;
    pmask |= static_cast<unsigned long long>(dmask) << lo;
    thr = prefix;
  }
  for (unsigned i = tid; i < n_cand; i += kSelThreads) {
    const uint2 c = in_lds ? s.cand[i] : ld_agent_u2(&cand_g[i]);
    if (sel_key(c.x, c.y) >= thr && c.y < static_cast<unsigned>(N)) {
      if (lds_bm)
        atomicOr(&s.bm[c.y >> 5], 1u << (c.y & 31));
      else
        atomicOr(&bm_g[c.y >> 5], 1u << (c.y & 31));
    }
  }
  __syncthreads();

  // ordered compaction of the bitmap into ascending positions: each thread
  // counts a run of wpt consecutive words and a block scan gives every run's
  // first output slot. With the bitmap in LDS, every output slot t then finds
  // its wave from the waves' first slots, its run by binary search over that
  // wave's 64 runs, its word by a scan of at most wpt popcounts and its bit by
  // halving popcounts, so that all lanes do the same work; else each thread
  // writes its own run's positions.
  const int wpt = (words + kSelThreads - 1) / kSelThreads;
  const int w0 = min(words, tid * wpt), w1 = min(words, w0 + wpt);
  unsigned cnt = 0;
  for (int i = w0; i < w1; ++i) cnt += __popc(lds_bm ? s.bm[i] : load_word(&bm_g[i]));
  unsigned total;
  unsigned run = sel_block_scan(cnt, s.wsum, &total);
  if (lds_bm) {
    unsigned* first = s.sh;  // kSelThreads run starts (the histogram is no longer needed)
    first[tid] = run;
    // the waves' first output slots: wave w's runs start at wstart[w] (wsum
    // holds the waves' totals after the scan)
    unsigned wstart[kSelWaves];
    {
      unsigned acc = 0;
#pragma unroll
      for (int i = 0; i < kSelWaves; ++i) {
        wstart[i] = acc;
        acc += s.wsum[i];
      }
    }
    __syncthreads();
    const unsigned n_out = min(total, static_cast<unsigned>(kk));
    for (unsigned t = tid; t < n_out; t += kSelThreads) {
      // the last wave starting at or before t holds slot t (an empty wave
      // shares its start with the next one), then its 64 runs by halving:
      // first[lo] <= t < first[hi], first[kSelThreads] standing for the total
      int w = 0;
#pragma unroll
      for (int i = 1; i < kSelWaves; ++i) w += wstart[i] <= t ? 1 : 0;
      int lo = w * kWave, hi = lo + kWave;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (first[mid] <= t)
          lo = mid;
        else
          hi = mid;
      }
      unsigned r = t - first[lo];
      int wi = lo * wpt;  // run lo's words (a run with no set bit is never found)
      unsigned x = s.bm[wi];
      for (unsigned c = __popc(x); r >= c; c = __popc(x)) {
        r -= c;
        x = s.bm[++wi];
      }
      int pos = 0;
#pragma unroll
      for (int sh = 16; sh; sh >>= 1) {
        const unsigned c = __popc(x & ((1u << sh) - 1u));
        if (r >= c) {
          r -= c;
          x >>= sh;
          pos += sh;
        }
      }
      out[t] = wi * 32 + pos;
    }
  } else {
    for (int i = w0; i < w1; ++i) {
      unsigned x = load_word(&bm_g[i]);
      while (x) {
        if (run < static_cast<unsigned>(kk)) out[run] = i * 32 + __ffs(x) - 1;
        ++run;
        x &= x - 1;
      }
    }
  }
}

// src: per head N pooled scores (rad = 0) or raw votes (pooled here with radius rad)
__global__ __launch_bounds__(kSelThreads) void snap_select(const float* __restrict__ src, int vec, int rad, int skip,
                                                           unsigned* __restrict__ hist, int N, int kk,
                                                           unsigned* __restrict__ ctr, uint2* __restrict__ cand_ws,
                                                           unsigned* __restrict__ bitmap_ws,
                                                           int* __restrict__ idx_out, int self_hist,
                                                           float* __restrict__ pooled_out, const ExactArgs ea,
                                                           unsigned spin) {
  __shared__ SelShared s;
  __shared__ ExactShared es;
  const int blk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = lane_id();
  const float* pb = src + static_cast<int64_t>(bh) * N;
  const int words = (N + 31) >> 5;
  unsigned* bm_g = bitmap_ws + static_cast<int64_t>(bh) * words;
  uint2* cand_g = cand_ws + static_cast<int64_t>(bh) * N;
  unsigned* ctr_head = ctr + bh * kSelCtrWords;
  unsigned* hb = hist + static_cast<int64_t>(bh) * kHistBins;
  const int c0 = blk * kSelChunk, c1 = min(N, c0 + kSelChunk);

  // 1. the range's scores on their way (off the 16-byte path the loads read,
  // and ignore, the histogram row), then the threshold bin
  constexpr int kHistPer = kHistBins / kSelThreads;
  unsigned hv[kHistPer];
  if (!self_hist) {
#pragma unroll
    for (int r = 0; r < kHistPer; ++r) hv[r] = hb[tid + r * kSelThreads];
  }
  const int nf = vec ? N >> 2 : 1;
  const int fb = vec ? c0 >> 2 : 0;
  const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(vec ? static_cast<const void*>(pb) : static_cast<const void*>(hb));
  f32x4_t xb[kSelPer], xe[kSelPer];
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    const int f = fb + tid + k * kSelThreads;
    xb[k] = pv[min(f, nf - 1)];
    // the piece just beyond the wave, for lanes 0 and 63 (a clamped copy for the others)
    xe[k] = pv[min(max((lane == 0 ? f - 1 : f + 1), 0), nf - 1)];
  }
  const bool exact = self_hist && exact_flagged(ea, bh);
  if (exact) {
    // the exact votes of the range's pieces and of the pieces beyond the
    // waves' edges (those of a neighbouring range computed here too, so that
    // no workgroup reads another's); the range's own go back to the vote buffer
    exact_prepare(es, ea, bh);
    float* vb = const_cast<float*>(pb);
#pragma unroll 1
    for (int k = 0; k < kSelPer; ++k) {
      const int f = fb + tid + k * kSelThreads;
      xb[k] = sel_exact_piece(es, ea, bh, min(f, nf - 1));
      if (lane == 0 || lane == kWave - 1) xe[k] = sel_exact_piece(es, ea, bh, min(max((lane == 0 ? f - 1 : f + 1), 0), nf - 1));
      if (f < nf) *reinterpret_cast<f32x4_t*>(vb + 4 * f) = xb[k];
    }
  }
  f32x4_t pp[kSelPer];
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) pp[k] = vec ? sel_pool_piece(xb[k], xe[k], fb + tid + k * kSelThreads, nf, rad) : xb[k];
#pragma unroll
  for (int r = 0; r < kHistPer; ++r) s.sh[tid + r * kSelThreads] = self_hist ? 0u : hv[r];
  if (tid == 0) {
    s.bin = 0;
    s.above = 0;
    s.nloc = 0;
  }
  __syncthreads();
  if (self_hist) {
    // the range's histogram into the head's row, then the head's once all its
    // workgroups have added theirs (bounded wait), else counted here
#pragma unroll
    for (int k = 0; k < kSelPer; ++k) {
      const int f = fb + tid + k * kSelThreads;
      if (f < nf) sel_count_piece(s.sh, pp[k], pooled_out ? pooled_out + static_cast<int64_t>(bh) * N + 4 * f : nullptr);
    }
    __syncthreads();
    flush_hist(s.sh, hb);
    // this thread's device-scope adds are complete before the workgroup counts
    // itself in (a wait, not a fence: an agent-scope release fence would write
    // back the L2 for every wave)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      atomicAdd(&ctr_head[2], 1u);
      unsigned n = load_word(&ctr_head[2]);
      for (unsigned polls = 0; n < gridDim.x && polls < spin; ++polls) {
        __builtin_amdgcn_s_sleep(2);
        n = load_word(&ctr_head[2]);
      }
      s.hist_in = n >= gridDim.x;
    }
    __syncthreads();
    if (s.hist_in) {
      // (agent-scope loads: they read the adds where they were made)
#pragma unroll
      for (int r = 0; r < kHistPer; ++r) s.sh[tid + r * kSelThreads] = load_word(&hb[tid + r * kSelThreads]);
    } else {
      // some of the head's workgroups were not resident: every piece of the
      // head pooled and counted here (exact votes again for a flagged head)
#pragma unroll
      for (int r = 0; r < kHistPer; ++r) s.sh[tid + r * kSelThreads] = 0;
      __syncthreads();
#pragma unroll 1
      for (int f0 = 0; f0 < nf; f0 += kSelThreads) {
        const int f = f0 + tid, fe = min(max((lane == 0 ? f - 1 : f + 1), 0), nf - 1);
        f32x4_t x = pv[min(f, nf - 1)], y = pv[fe];
        if (exact) {
          x = sel_exact_piece(es, ea, bh, min(f, nf - 1));
          if (lane == 0 || lane == kWave - 1) y = sel_exact_piece(es, ea, bh, fe);
        }
        const f32x4_t p = sel_pool_piece(x, y, f, nf, rad);
        if (f < nf) sel_count_piece(s.sh, p, nullptr);
      }
    }
    __syncthreads();
  }
  sel_find_bin(s.sh, static_cast<unsigned>(kk), s.wsum, &s.bin, &s.above);
  const unsigned bstar = s.bin;
  unsigned rem = static_cast<unsigned>(kk) - s.above;

  // 2. classification of [c0, c1)
  if (vec) {
#pragma unroll
    for (int k = 0; k < kSelPer; ++k) {
      const int f = fb + tid + k * kSelThreads;
      if (!skip || sel_wave_reaches(xb[k], xe[k], bstar))
        sel_piece(s, bm_g, ctr_head, cand_g, N, pp[k], f, f < nf, bstar);
      else if (f < nf && (lane_id() & 7) == 0)
        store_word(&bm_g[f >> 3], 0u);
    }
  } else {
    for (int w = (c0 >> 5) + tid; w < ((c1 + 31) >> 5); w += kSelThreads) {
      unsigned bits = 0;
      for (int b = 0; b < 32; ++b) {
        const int j = w * 32 + b;
        if (j >= c1) break;
        const unsigned u = __float_as_uint(sel_pool_at(pb, j, N, rad));
        const unsigned bin = (u >> kHistShift) & (kHistBins - 1);
        bits |= static_cast<unsigned>(bin > bstar) << b;
        if (bin == bstar) sel_add_cand(s, ctr_head, cand_g, N, u, static_cast<unsigned>(j), lds_add_rtn(&s.nloc, 1u));
      }
      store_word(&bm_g[w], bits);
    }
  }
  __syncthreads();
  const unsigned nl = min(s.nloc, static_cast<unsigned>(kCandLds));
  if (tid == 0) s.base = nl ? atomicAdd(&ctr_head[0], nl) : 0u;
  __syncthreads();
  for (unsigned i = tid; i < nl; i += kSelThreads)
    if (s.base + i < static_cast<unsigned>(N)) st_agent_u2(&cand_g[s.base + i], s.cand[i]);
  // this thread's device-scope stores are complete before the workgroup counts
  // itself finished
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s.last = atomicAdd(&ctr_head[1], 1u) == gridDim.x - 1u;
  __syncthreads();
  if (!s.last) return;

  // 3. the head's last workgroup: candidates and bitmap, ranking, compaction
  const unsigned n_cand = min(load_word(&ctr_head[0]), static_cast<unsigned>(N));
  const bool in_lds = n_cand <= static_cast<unsigned>(kCandLds);
  const bool lds_bm = words <= kBitmapLds;
  // every load in flight before the first LDS store (one round trip)
  constexpr int kCandPer = kCandLds / kSelThreads, kBmPer = kBitmapLds / kSelThreads;
  uint2 cv[kCandPer];
  unsigned bv[kBmPer];
#pragma unroll
  for (int r = 0; r < kBmPer; ++r) {
    const int i = tid + r * kSelThreads;
    if (lds_bm && i < words) bv[r] = load_word(&bm_g[i]);
  }
#pragma unroll
  for (int r = 0; r < kCandPer; ++r) {
    const unsigned i = static_cast<unsigned>(tid + r * kSelThreads);
    if (in_lds && i < n_cand) cv[r] = ld_agent_u2(&cand_g[i]);
  }
#pragma unroll
  for (int r = 0; r < kBmPer; ++r) {
    const int i = tid + r * kSelThreads;
    if (lds_bm && i < words) s.bm[i] = bv[r];
  }
#pragma unroll
  for (int r = 0; r < kCandPer; ++r) {
    const unsigned i = static_cast<unsigned>(tid + r * kSelThreads);
    if (in_lds && i < n_cand) s.cand[i] = cv[r];
  }
  sel_rank_compact(s, bstar, rem, n_cand, in_lds, cand_g, bm_g, lds_bm, words, N, kk,
                   idx_out + static_cast<int64_t>(bh) * kk);
}

// The classification of sel_piece with the bitmap word kept in LDS.
__device__ __forceinline__ void sel_piece_lds(SelShared& s, unsigned* ctr_head, uint2* cand_g, int N, f32x4_t x,
                                              int f, bool valid, unsigned bstar) {
  const int lane = lane_id();
  unsigned m = 0, nc = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const unsigned bin = (__float_as_uint(x[e]) >> kHistShift) & (kHistBins - 1);
    m |= static_cast<unsigned>(valid && bin > bstar) << e;
    nc += valid && bin == bstar;
  }
  m = octet_or(m << (4 * (lane & 7)));
  if (valid && (lane & 7) == 0) s.bm[f >> 3] = m;
  if (nc != 0u) {
    unsigned slot = lds_add_rtn(&s.nloc, nc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned u = __float_as_uint(x[e]);
      if (valid && ((u >> kHistShift) & (kHistBins - 1)) == bstar) {
        sel_add_cand(s, ctr_head, cand_g, N, u, static_cast<unsigned>(4 * f + e), slot);
        ++slot;
      }
    }
  }
}

// The whole selection of one head in one workgroup, for heads of at most
// kSelChunk positions (one workgroup's range; N % 4 == 0, 16-byte aligned
// rows): the same threshold bin, classification, ranking and compaction as
// snap_select, with the head's bitmap and candidates in LDS from the start,
// so that no workgroup waits for another's results through device memory.
// Longer heads go to snap_select: one workgroup walking them range by range
// would wait for each range's loads in turn.
//
// With self_hist (single pass, raw votes max-pooled here) the workgroup also
// does the pooling kernel's work for its head, which is then not launched:
// the exact votes of a flagged head (ea, as the pooling kernel), the head's
// 12-bit histogram of pooled scores (in LDS, from the pooled pieces the
// classification uses) and, if pooled_out is not NULL, the pooled scores.
// `hist` is not read then.
__global__ __launch_bounds__(kSelThreads) void snap_select_head(const float* __restrict__ src, int rad, int skip,
                                                                const unsigned* __restrict__ hist, int N, int kk,
                                                                unsigned* __restrict__ ctr,
                                                                uint2* __restrict__ cand_ws,
                                                                int* __restrict__ idx_out, int self_hist,
                                                                float* __restrict__ pooled_out, const ExactArgs ea) {
  __shared__ SelShared s;
  __shared__ ExactShared es;
  const int bh = blockIdx.x, tid = threadIdx.x, lane = lane_id();
  const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(src + static_cast<int64_t>(bh) * N);
  const int nf = N >> 2;
  const int words = (N + 31) >> 5;
  uint2* cand_g = cand_ws + static_cast<int64_t>(bh) * N;
  unsigned* ctr_head = ctr + bh * kSelCtrWords;
  const unsigned* hb = hist + static_cast<int64_t>(bh) * kHistBins;

  // the histogram row (or the head's flag) and the head's pieces in flight together
  constexpr int kHistPer = kHistBins / kSelThreads;
  unsigned hv[kHistPer];
  if (!self_hist) {
#pragma unroll
    for (int r = 0; r < kHistPer; ++r) hv[r] = hb[tid + r * kSelThreads];
  }
  f32x4_t xb[kSelPer], xe[kSelPer];
  auto load_pieces = [&]() {
#pragma unroll
    for (int k = 0; k < kSelPer; ++k) {
      const int f = tid + k * kSelThreads;
      xb[k] = pv[min(f, nf - 1)];
      // the piece just beyond the wave, for lanes 0 and 63 (a clamped copy for the others)
      xe[k] = pv[min(max(lane == 0 ? f - 1 : f + 1, 0), nf - 1)];
    }
  };
  load_pieces();
  if (self_hist && exact_flagged(ea, bh)) {
    // the head's exact votes (the pieces just loaded are discarded), written
    // back where the caller reads them, then read again from L2
    float* vb = const_cast<float*>(src) + static_cast<int64_t>(bh) * N;
    exact_prepare(es, ea, bh);
    for (int j = tid; j < N; j += kSelThreads) vb[j] = exact_vote(es, ea, bh, j);
    __threadfence();
    __syncthreads();
    __threadfence();
    load_pieces();
  }
  f32x4_t pp[kSelPer];
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) pp[k] = sel_pool_piece(xb[k], xe[k], tid + k * kSelThreads, nf, rad);
  if (self_hist) {
#pragma unroll
    for (int r = 0; r < kHistPer; ++r) s.sh[tid + r * kSelThreads] = 0;
  } else {
#pragma unroll
    for (int r = 0; r < kHistPer; ++r) s.sh[tid + r * kSelThreads] = hv[r];
  }
  if (tid == 0) {
    s.bin = 0;
    s.above = 0;
    s.nloc = 0;
  }
  __syncthreads();
  if (self_hist) {
#pragma unroll
    for (int k = 0; k < kSelPer; ++k) {
      const int f = tid + k * kSelThreads;
      if (f < nf) sel_count_piece(s.sh, pp[k], pooled_out ? pooled_out + static_cast<int64_t>(bh) * N + 4 * f : nullptr);
    }
    __syncthreads();
  }
  sel_find_bin(s.sh, static_cast<unsigned>(kk), s.wsum, &s.bin, &s.above);
  const unsigned bstar = s.bin;
  const unsigned rem = static_cast<unsigned>(kk) - s.above;
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    const int f = tid + k * kSelThreads;
    if (!skip || sel_wave_reaches(xb[k], xe[k], bstar))
      sel_piece_lds(s, ctr_head, cand_g, N, pp[k], f, f < nf, bstar);
    else if (f < nf && (lane & 7) == 0)
      s.bm[f >> 3] = 0u;
  }
  __syncthreads();
  // candidates past the LDS list went to the head's workspace list as they
  // were found; then the LDS ones join them there
  const unsigned nloc = s.nloc;
  const bool in_lds = nloc <= static_cast<unsigned>(kCandLds);
  unsigned n_cand = nloc;
  if (!in_lds) {
    if (tid == 0) s.base = atomicAdd(&ctr_head[0], static_cast<unsigned>(kCandLds));
    __syncthreads();
    for (unsigned i = tid; i < static_cast<unsigned>(kCandLds); i += kSelThreads)
      if (s.base + i < static_cast<unsigned>(N)) st_agent_u2(&cand_g[s.base + i], s.cand[i]);
    __builtin_amdgcn_s_waitcnt(0);  // the stores are complete before any thread reads the list
    n_cand = min(nloc, static_cast<unsigned>(N));
  }
  sel_rank_compact(s, bstar, rem, n_cand, in_lds, cand_g, nullptr, true, words, N, kk,
                   idx_out + static_cast<int64_t>(bh) * kk);
}

// -------------------------------------------------------------- gather

// kGatherPer 16-byte pieces of output rows per thread, K and V together; all
// loads are issued before the stores.
constexpr int kGatherPer = 2;

__global__ __launch_bounds__(kThreads) void snap_gather(const char* __restrict__ k,
                                                        const char* __restrict__ v, int64_t sb,
                                                        int64_t sh, int64_t st, int H, int L, int w,
                                                        int C, int kk, int vec_per_row,
                                                        const int* __restrict__ idx,
                                                        char* __restrict__ k_out,
                                                        char* __restrict__ v_out) {
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * kThreads * kGatherPer + threadIdx.x;
  const int64_t n_pieces = static_cast<int64_t>(C) * vec_per_row;
  const int64_t row_bytes = static_cast<int64_t>(vec_per_row) * 16;
  u32x4_t kx[kGatherPer], vx[kGatherPer];
  int64_t dst[kGatherPer];
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u) {
    const int64_t t = first + static_cast<int64_t>(u) * kThreads;
    dst[u] = -1;
    if (t >= n_pieces) continue;
    const int row = static_cast<int>(t / vec_per_row);
    const int vc = static_cast<int>(t - static_cast<int64_t>(row) * vec_per_row);
    int src = row < kk ? idx[static_cast<int64_t>(bh) * kk + row] : (L - w + (row - kk));
    src = min(max(src, 0), L - 1);
    const int64_t so = b * sb + h * sh + static_cast<int64_t>(src) * st + static_cast<int64_t>(vc) * 16;
    kx[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(k + so));
    vx[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(v + so));
    dst[u] = (static_cast<int64_t>(bh) * C + row) * row_bytes + static_cast<int64_t>(vc) * 16;
  }
#pragma unroll
  for (int u = 0; u < kGatherPer; ++u) {
    if (dst[u] < 0) continue;
    __builtin_nontemporal_store(kx[u], reinterpret_cast<u32x4_t*>(k_out + dst[u]));
    __builtin_nontemporal_store(vx[u], reinterpret_cast<u32x4_t*>(v_out + dst[u]));
  }
}

// ------------------------------------------------------ workspace layout

struct SnapLayout {
  int64_t BH;
  int N, kk, nchunk, words, nunit;
  size_t hist, sel_ctr;
  size_t part, rowstat, pooled, cand, bitmap;
  size_t cref, cacc, ccnt, cstat, cpart, cstatus;  // single pass (bf16)
  size_t total;
};

bool snap_layout(int B, int H, int L, int D, int w, int budget, kvc_dtype dt, SnapLayout* o) {
  (void)D;
  if (B <= 0 || H <= 0 || L <= 0 || w <= 0 || budget <= w || budget >= L) return false;
  const int64_t BH = static_cast<int64_t>(B) * H;
  o->BH = BH;
  o->N = L - w;
  o->kk = budget - w;
  const int chunk = dt == KVC_BF16 ? kStatChunkMfma : kChunkF32;
  o->nchunk = (L + chunk - 1) / chunk;
  o->words = (o->N + 31) / 32;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  o->hist = take(static_cast<size_t>(BH) * kHistBins * 4);
  o->sel_ctr = take(static_cast<size_t>(BH) * kSelCtrWords * 4);
  o->part = take(static_cast<size_t>(BH) * o->nchunk * 32 * 8);
  o->rowstat = take(static_cast<size_t>(BH) * 32 * 8);
  o->pooled = take(static_cast<size_t>(BH) * o->N * 4);
  o->cand = take(static_cast<size_t>(BH) * o->N * 8);
  o->bitmap = take(static_cast<size_t>(BH) * o->words * 4);
  o->nunit = (L + kCoopUnit - 1) / kCoopUnit;
  o->cref = o->cacc = o->ccnt = o->cstat = o->cpart = o->cstatus = 0;
  if (dt == KVC_BF16) {
    o->cref = take(static_cast<size_t>(BH) * 32 * 4);
    o->cacc = take(static_cast<size_t>(BH) * kCoopHeadWords * 8);
    o->ccnt = take(static_cast<size_t>(BH) * kCoopCtrWords * 4);
    o->cstat = take(static_cast<size_t>(BH) * 32 * 8);
    o->cpart = take(static_cast<size_t>(BH) * o->nunit * 32 * 8);
    o->cstatus = take(16);  // [0] status, [1] [2] the single pass's residency gate
  }
  o->total = off;
  return true;
}

// Optional per-phase timing events (see kvc_snapkv_set_phase_events).
thread_local hipEvent_t* g_phase_events = nullptr;
thread_local int g_phase_count = 0;

void mark_phase(int i, hipStream_t stream) {
  if (g_phase_events && i < g_phase_count && g_phase_events[i]) (void)hipEventRecord(g_phase_events[i], stream);
}

hipEvent_t phase_event(int i) { return g_phase_events && i < g_phase_count ? g_phase_events[i] : nullptr; }

template <typename... P, typename... A, size_t... I>
hipError_t launch_timed_impl(void (*kern)(P...), dim3 grid, dim3 block, hipStream_t stream, hipEvent_t start,
                             hipEvent_t stop, std::index_sequence<I...>, A... a) {
  std::tuple<P...> args(a...);  // every argument as the kernel's own parameter type
  void* ptrs[] = {static_cast<void*>(&std::get<I>(args))...};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, 0, stream, start, stop, 0);
}

// A launch whose start and stop events are recorded by the dispatch itself,
// at the kernel's start and end, instead of by separate records around it
// (each of which costs a few microseconds of GPU time between the kernels).
template <typename... P, typename... A>
hipError_t launch_timed(void (*kern)(P...), dim3 grid, dim3 block, hipStream_t stream, hipEvent_t start,
                        hipEvent_t stop, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
  return launch_timed_impl(kern, grid, block, stream, start, stop, std::index_sequence_for<P...>{}, a...);
}

template <int D>
void launch_stats(const SnapLayout& lay, const uint16_t* q, kvc_strides qs, int qrow0, const uint16_t* k,
                  kvc_strides kvs, int H, int L, int w, float scale_log2, char* ws, hipStream_t stream) {
  const dim3 g(lay.nchunk, static_cast<unsigned>(lay.BH));
  snap_stats_bf16<D><<<g, kThreads, 0, stream>>>(q, qs.b, qs.h, qs.t, qrow0, k, kvs.b, kvs.h, kvs.t, H, L, w,
                                                lay.nchunk, scale_log2, reinterpret_cast<float2*>(ws + lay.part),
                                                reinterpret_cast<unsigned*>(ws + lay.hist),
                                                reinterpret_cast<unsigned*>(ws + lay.sel_ctr));
}

template <int D>
void launch_stats(const SnapLayout& lay, const float* q, kvc_strides qs, int qrow0, const float* k,
                  kvc_strides kvs, int H, int L, int w, float scale_log2, char* ws, hipStream_t stream) {
  const dim3 g(lay.nchunk, static_cast<unsigned>(lay.BH));
  snap_stats_f32<D><<<g, kThreads, 0, stream>>>(q, qs.b, qs.h, qs.t, qrow0, k, kvs.b, kvs.h, kvs.t, H, L, w,
                                               lay.nchunk, scale_log2, reinterpret_cast<float2*>(ws + lay.part),
                                               reinterpret_cast<unsigned*>(ws + lay.hist),
                                               reinterpret_cast<unsigned*>(ws + lay.sel_ctr));
}

template <int D>
void launch_votes(const SnapLayout& lay, const uint16_t* q, kvc_strides qs, int qrow0, const uint16_t* k,
                  kvc_strides kvs, int H, int L, int w, int r, int avg, float scale_log2, char* ws, float* vote,
                  float* pooled, hipStream_t stream) {
  const dim3 g((lay.N + kChunkMfma - 1) / kChunkMfma, static_cast<unsigned>(lay.BH));
  snap_votes_bf16<D><<<g, kThreads, 0, stream>>>(q, qs.b, qs.h, qs.t, qrow0, k, kvs.b, kvs.h, kvs.t, H, L, w, r, avg,
                                                scale_log2, reinterpret_cast<const float2*>(ws + lay.rowstat),
                                                vote, pooled, reinterpret_cast<unsigned*>(ws + lay.hist));
}

template <int D>
void launch_votes(const SnapLayout& lay, const float* q, kvc_strides qs, int qrow0, const float* k,
                  kvc_strides kvs, int H, int L, int w, int r, int avg, float scale_log2, char* ws, float* vote,
                  float* pooled, hipStream_t stream) {
  const dim3 g((lay.N + kChunkF32 - 1) / kChunkF32, static_cast<unsigned>(lay.BH));
  snap_votes_f32<D><<<g, kThreads, 0, stream>>>(q, qs.b, qs.h, qs.t, qrow0, k, kvs.b, kvs.h, kvs.t, H, L, w, r, avg,
                                               scale_log2, reinterpret_cast<const float2*>(ws + lay.rowstat),
                                               vote, pooled, reinterpret_cast<unsigned*>(ws + lay.hist));
}

// Pass 1 (row statistics; it also clears the histograms and counters), the
// merge of each head's statistics, then pass 2 (votes, pooling and the
// histogram), with phase marks 2, 3 and 4.
template <typename T>
void launch_score_passes(const SnapLayout& lay, const T* q, kvc_strides qs, int qrow0, const T* k,
                         kvc_strides kvs, int H, int L, int D, int w, int r, int avg, float scale_log2, char* ws,
                         float* vote, float* pooled, hipStream_t stream) {
  if (D == 128)
    launch_stats<128>(lay, q, qs, qrow0, k, kvs, H, L, w, scale_log2, ws, stream);
  else
    launch_stats<64>(lay, q, qs, qrow0, k, kvs, H, L, w, scale_log2, ws, stream);
  mark_phase(2, stream);
  snap_stats_merge<<<static_cast<unsigned>(lay.BH), kThreads, 0, stream>>>(
      reinterpret_cast<const float2*>(ws + lay.part), lay.nchunk, reinterpret_cast<float2*>(ws + lay.rowstat));
  mark_phase(3, stream);
  if (D == 128)
    launch_votes<128>(lay, q, qs, qrow0, k, kvs, H, L, w, r, avg, scale_log2, ws, vote, pooled, stream);
  else
    launch_votes<64>(lay, q, qs, qrow0, k, kvs, H, L, w, r, avg, scale_log2, ws, vote, pooled, stream);
  mark_phase(4, stream);
}

thread_local int g_schedule = KVC_SNAPKV_AUTO;
thread_local int g_last_schedule = 0;

// Per device: cooperative launch support, compute units and resident
// single-pass workgroups per compute unit (index 0: D = 64, 1: D = 128).
struct CoopCaps {
  bool queried = false, coop = false;
  int cus = 0, per_cu[2] = {0, 0}, wv_per_cu[2] = {0, 0};
  int sel_per_cu = 0;  // split selection workgroups per compute unit
};

const CoopCaps& coop_caps() {
  static std::mutex mu;
  static CoopCaps caps[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    static const CoopCaps none;
    return none;
  }
  std::lock_guard<std::mutex> lock(mu);
  CoopCaps& c = caps[dev];
  if (!c.queried) {
    c.queried = true;
    int coop = 0, cus = 0, n64 = 0, n128 = 0, w64 = 0, w128 = 0, sel = 0;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&n64, snap_coop_bf16<64>, kCoopThreads, 0) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&n128, snap_coop_bf16<128>, kCoopThreads, 0) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&w64, snap_wave_bf16<64, false>, kWvThreads, 0) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&w128, snap_wave_bf16<128, false>, kWvThreads, 0) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&sel, snap_select, kSelThreads, 0) == hipSuccess) {
      c.coop = coop != 0;
      c.cus = cus;
      c.per_cu[0] = n64;
      c.per_cu[1] = n128;
      c.wv_per_cu[0] = w64;
      c.wv_per_cu[1] = w128;
      c.sel_per_cu = sel;
    }
    (void)hipGetLastError();
  }
  return c;
}

// Grid of the single pass for these sizes, 0 when it cannot run. The votes of
// a round-r unit wait (in round r + kCoopLag) for its head's normaliser,
// which the finishing workgroup publishes three rounds after the head's last
// unit; with a head spanning at most kCoopLag - 3 consecutive rounds every
// such wait depends only on heads that started in earlier rounds, so all of
// them end.
int coop_grid(const SnapLayout& lay, int D) {
  const CoopCaps& c = coop_caps();
  if (!c.coop || c.cus <= 0) return 0;
  const int per_cu = c.per_cu[D == 128 ? 1 : 0];
  if (per_cu <= 0) return 0;
  const int64_t total = lay.BH * lay.nunit;
  const int G = static_cast<int>(std::min<int64_t>(static_cast<int64_t>(per_cu) * c.cus, total));
  if (lay.nunit > (kCoopLag - 3) * G) return 0;
  for (int64_t bh = 0; bh < lay.BH; ++bh) {
    const int64_t u0 = bh * lay.nunit, u1 = u0 + lay.nunit - 1;
    if (u1 / G - u0 / G > kCoopLag - 4) return 0;
  }
  return G;
}

// Tiles per head of the independent-wave single pass: 32-key tiles, padded to
// a multiple of kWvWaves.
int64_t wave_tiles(int L) { return ((L + kTile - 1) / kTile + kWvWaves - 1) / kWvWaves * kWvWaves; }

// Grid of the independent-wave single pass (one workgroup per resident slot,
// which the kernel checks at its start), 0 when it cannot run. Either every
// workgroup has tiles in every head (a head's padded tile count is at least
// the worker count W), or heads are shorter than a round and each workgroup
// takes one head per round (nt / kWvWaves workgroups contribute to each);
// a head may span at most kWvMaxSpan rounds
// beyond its first: a vote waits (in round r) for the normaliser of a tile
// of round r - kWvBanks, whose head's last tile was then scored by round
// r - 3 at the latest, so every such wait depends only on heads that every
// wave has finished, and all of them end.
int wave_grid(const SnapLayout& lay, int D, int L, int64_t kst, int64_t qst) {
  const CoopCaps& c = coop_caps();
  if (c.cus <= 0) return 0;
  const int per_cu = c.wv_per_cu[D == 128 ? 1 : 0];
  if (per_cu <= 0) return 0;
  const int64_t G = static_cast<int64_t>(per_cu) * c.cus, W = G * kWvWaves, nt = wave_tiles(L);
  if (lay.BH * nt > INT32_MAX) return 0;
  // heads shorter than a round: each workgroup takes one head per round, so
  // only when the layer fills enough rounds for the votes' lag to pay off
  if (nt < W && lay.BH * nt < static_cast<int64_t>(kWvMinRounds) * W) return 0;
  if (kst * 2 * 8 >= (int64_t(1) << 32) || qst * 2 * 32 >= (int64_t(1) << 32)) return 0;  // 32-bit lane offsets
  for (int64_t bh = 0; bh < lay.BH; ++bh) {
    const int64_t r0 = bh * nt / W, r1 = ((bh + 1) * nt - 1) / W;
    if (r1 - r0 > kWvMaxSpan) return 0;
  }
  return static_cast<int>(G);
}

thread_local const char* g_last_kernel = "";
thread_local bool g_force_residency_fail = false;
thread_local bool g_force_wait_timeout = false;
thread_local int g_force_split_select = 0;  // 1: split selection, 2: split selection and the pooling kernel
thread_local const char* g_last_select = "";
thread_local const char* g_last_pool = "";

template <int R>
void launch_pool_r(float* vote, float* pooled, unsigned* hist, int BH, int N, int avg, const ExactArgs& ea,
                   hipStream_t stream) {
  const bool vec = N % 4 == 0 && aligned16(vote) && (!pooled || aligned16(pooled));
  // a layer that fills the GPU with workgroups of 16384 positions takes those:
  // the histogram's clear and its flush into the head's row (device atomics)
  // are then paid once per 16384 positions instead of once per 4096
  const int64_t big_groups = static_cast<int64_t>(BH) * ((N + kPoolBigChunk - 1) / kPoolBigChunk);
  if (vec && big_groups >= coop_caps().cus) {
    const dim3 g((N + kPoolBigChunk - 1) / kPoolBigChunk, static_cast<unsigned>(BH));
    snap_pool<R, true, kPoolBigThreads><<<g, kPoolBigThreads, 0, stream>>>(vote, pooled, hist, N, avg, ea);
    return;
  }
  const dim3 g((N + kPoolChunk - 1) / kPoolChunk, static_cast<unsigned>(BH));
  if (vec)
    snap_pool<R, true, kThreads><<<g, kThreads, 0, stream>>>(vote, pooled, hist, N, avg, ea);
  else
    snap_pool<R, false, kThreads><<<g, kThreads, 0, stream>>>(vote, pooled, hist, N, avg, ea);
}

// Max-pool of the raw votes with the histogram of the results (pooled scores
// stored if `pooled` is not NULL; radii beyond kPoolRegRadius always store them).
void launch_pool(float* vote, float* pooled, unsigned* hist, int BH, int N, int r, int avg, const ExactArgs& ea,
                 hipStream_t stream) {
  static_assert(kPoolRegRadius == 7, "the cases below cover radii 0 .. kPoolRegRadius");
  switch (r) {
    case 0: return launch_pool_r<0>(vote, pooled, hist, BH, N, avg, ea, stream);
    case 1: return launch_pool_r<1>(vote, pooled, hist, BH, N, avg, ea, stream);
    case 2: return launch_pool_r<2>(vote, pooled, hist, BH, N, avg, ea, stream);
    case 3: return launch_pool_r<3>(vote, pooled, hist, BH, N, avg, ea, stream);
    case 4: return launch_pool_r<4>(vote, pooled, hist, BH, N, avg, ea, stream);
    case 5: return launch_pool_r<5>(vote, pooled, hist, BH, N, avg, ea, stream);
    case 6: return launch_pool_r<6>(vote, pooled, hist, BH, N, avg, ea, stream);
    case 7: return launch_pool_r<7>(vote, pooled, hist, BH, N, avg, ea, stream);
    default: {
      const dim3 g((N + kPoolChunk - 1) / kPoolChunk, static_cast<unsigned>(BH));
      snap_pool_lds<<<g, kThreads, 0, stream>>>(vote, pooled, hist, N, r, avg, ea);
    }
  }
}

// Single pass: the per-head preparation (reference scores, cleared state),
// the score pass (raw votes to `vote`; the independent-wave kernel, else the
// cooperative one), then pooling + histogram (pooled scores to `pooled`
// unless it is NULL; after the independent-wave kernel, exact votes of any
// flagged head first). Phase marks 1 to 4.
template <int D>
kvc_status launch_single_pass(const SnapLayout& lay, int Gw, int Gc, const uint16_t* q, kvc_strides qs, int qrow0,
                              const uint16_t* k, kvc_strides kvs, int H, int L, int w, int r, int avg,
                              float scale_log2, char* ws, float* vote, float* pooled, ExactArgs* fused, hipStream_t stream) {
  float* ref = reinterpret_cast<float*>(ws + lay.cref);
  unsigned long long* acc = reinterpret_cast<unsigned long long*>(ws + lay.cacc);
  unsigned* cnt = reinterpret_cast<unsigned*>(ws + lay.ccnt);
  uint2* stat = reinterpret_cast<uint2*>(ws + lay.cstat);
  float2* part = reinterpret_cast<float2*>(ws + lay.cpart);
  unsigned* status = reinterpret_cast<unsigned*>(ws + lay.cstatus);
  unsigned* hist = reinterpret_cast<unsigned*>(ws + lay.hist);
  unsigned* gate = status + 1;
  snap_coop_prep<D><<<static_cast<unsigned>(lay.BH), kThreads, 0, stream>>>(
      q, qs.b, qs.h, qs.t, qrow0, k, kvs.b, kvs.h, kvs.t, H, L, w, scale_log2, ref, acc, cnt, stat, hist,
      reinterpret_cast<unsigned*>(ws + lay.sel_ctr), status);
  // phase marks 1 and 2 around the independent-wave kernel come from its own
  // dispatch when both are set
  const hipEvent_t ev1 = phase_event(1), ev2 = phase_event(2);
  const bool timed = Gw > 0 && ev1 && ev2;
  if (!timed) mark_phase(1, stream);
  int64_t qsb = qs.b, qsh = qs.h, qst = qs.t, ksb = kvs.b, ksh = kvs.h, kst = kvs.t;
  const float* cref = ref;
  hipError_t e = hipErrorInvalidValue;
  // the pooling kernel reads the status word after either score kernel: a
  // wait that ran out leaves it non-zero, and every head's votes are then
  // recomputed exactly
  ExactArgs ea{q, qsb, qsh, qst, qrow0, k, ksb, ksh, kst, H, L, w, D, scale_log2, nullptr, status};
  if (Gw > 0) {
    // an ordinary launch: the kernel checks residency itself (a cooperative
    // launch would guarantee it, at ~10 us of extra queue work on each side)
    const int nt = static_cast<int>(wave_tiles(L)), total = static_cast<int>(lay.BH * nt);
    const unsigned target = static_cast<unsigned>(Gw) + (g_force_residency_fail ? 1u : 0u);
    const unsigned spin = g_force_residency_fail ? 16u : kWvGateSpin;
    const unsigned wait_spin = g_force_wait_timeout ? kWvSpinForced : kWvSpin;
    const int bhi = static_cast<int>(lay.BH);
    auto kern = nt < Gw * kWvWaves ? snap_wave_bf16<D, true> : snap_wave_bf16<D, false>;
    if (timed) {
      e = launch_timed(kern, dim3(Gw), dim3(kWvThreads), stream, ev1, ev2, q, qsb, qsh, qst, qrow0, k, ksb, ksh, kst,
                       H, L, w, nt, total, bhi, scale_log2, cref, acc, cnt, stat, status, vote, gate, target, spin,
                       wait_spin);
    } else {
      kern<<<dim3(Gw), dim3(kWvThreads), 0, stream>>>(q, qsb, qsh, qst, qrow0, k, ksb, ksh, kst, H, L, w, nt, total,
                                                      bhi, scale_log2, cref, acc, cnt, stat, status, vote, gate,
                                                      target, spin, wait_spin);
      e = hipSuccess;
    }
    const hipError_t le = hipGetLastError();
    if (e == hipSuccess) e = le;
    if (e == hipSuccess) {
      g_last_kernel = "snap_wave_bf16";
      if (!timed) mark_phase(2, stream);
      ea.flags = cnt;  // the pooling kernel recomputes the votes of flagged heads exactly
    } else {
      (void)hipGetLastError();
    }
  }
  if (e != hipSuccess && Gc > 0) {
    int nunit = lay.nunit, total_units = static_cast<int>(lay.BH * lay.nunit);
    void* args[] = {&q,     &qsb,         &qsh,        &qst,  &qrow0, &k,   &ksb,  &ksh,  &kst,    &H,   &L, &w,
                    &nunit, &total_units, &scale_log2, &cref, &acc,   &cnt, &stat, &part, &status, &vote};
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(snap_coop_bf16<D>), dim3(Gc), dim3(kCoopThreads),
                                   args, 0, stream);
    if (e == hipSuccess) {
      g_last_kernel = "snap_coop_bf16";
      mark_phase(2, stream);
    }
  }
  if (e != hipSuccess) return fail(KVC_ERR_HIP, "snapkv single pass launch: %s", hipGetErrorString(e));
  mark_phase(3, stream);
  if (fused)
    *fused = ea;  // the per-head selection pools, counts and recomputes flagged heads itself
  else
    launch_pool(vote, pooled, hist, static_cast<int>(lay.BH), lay.N, r, avg, ea, stream);
  mark_phase(4, stream);
  return KVC_OK;
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" int kvc_snapkv_set_schedule(int schedule) {
  if (schedule != KVC_SNAPKV_AUTO && schedule != KVC_SNAPKV_TWO_PASS && schedule != KVC_SNAPKV_SINGLE_PASS)
    return -1;
  const int prev = g_schedule;
  g_schedule = schedule;
  return prev;
}

extern "C" int kvc_snapkv_last_schedule(void) { return g_last_schedule; }

extern "C" const char* kvc_snapkv_last_score_kernel(void) { return g_last_kernel; }

extern "C" int kvc_snapkv_force_residency_fallback(int on) {
  const int prev = g_force_residency_fail ? 1 : 0;
  g_force_residency_fail = on != 0;
  return prev;
}

extern "C" int kvc_snapkv_force_wait_timeout(int on) {
  const int prev = g_force_wait_timeout ? 1 : 0;
  g_force_wait_timeout = on != 0;
  return prev;
}

extern "C" int kvc_snapkv_force_split_select(int on) {
  const int prev = g_force_split_select;
  g_force_split_select = on == 2 ? 2 : on != 0 ? 1 : 0;
  return prev;
}

extern "C" const char* kvc_snapkv_last_select_kernel(void) { return g_last_select; }

extern "C" const char* kvc_snapkv_last_pool_kernel(void) { return g_last_pool; }

extern "C" size_t kvc_snapkv_workspace_bytes(int B, int H, int L, int D, int window, int budget,
                                             int pool_kernel, kvc_dtype dt) {
  (void)pool_kernel;
  SnapLayout lay;
  if (!snap_layout(B, H, L, D, window, budget, dt, &lay)) return 0;
  return lay.total;
}

extern "C" int64_t kvc_snapkv_status_offset(int B, int H, int L, int D, int window, int budget, int pool_kernel,
                                           kvc_dtype dt) {
  (void)pool_kernel;
  SnapLayout lay;
  if (!snap_layout(B, H, L, D, window, budget, dt, &lay) || lay.cstatus == 0) return -1;
  return static_cast<int64_t>(lay.cstatus);
}

namespace kvc {
namespace {

// Host checks of one layer's arguments (everything but the workspace).
kvc_status snap_validate(const void* q, int q_len, kvc_strides qs, const void* k, const void* v, kvc_strides kvs,
                         int B, int H, int L, int D, int window, int budget, int pool_kernel, int pool_type,
                         kvc_dtype dt, const void* k_out, const void* v_out, const int32_t* idx_out) {
  if (!q || !k || !v || !k_out || !v_out || !idx_out)
    return fail(KVC_ERR_INVALID_ARG, "snapkv: q, k, v, k_out, v_out and idx_out must be non-NULL");
  if (dt != KVC_BF16 && dt != KVC_F32) return fail(KVC_ERR_INVALID_ARG, "snapkv: unknown dtype %d", (int)dt);
  if (B <= 0 || H <= 0 || L <= 0) return fail(KVC_ERR_INVALID_ARG, "snapkv: B, H, L must be positive");
  if (static_cast<int64_t>(B) * H > 65535) return fail(KVC_ERR_UNSUPPORTED, "snapkv: B*H must be <= 65535");
  if (window < 1 || window >= budget || budget >= L)
    return fail(KVC_ERR_INVALID_ARG, "snapkv: need 1 <= window < budget < L (window=%d budget=%d L=%d)",
                window, budget, L);
  if (window > kMaxWindow) return fail(KVC_ERR_UNSUPPORTED, "snapkv: window %d > %d", window, kMaxWindow);
  if (pool_kernel < 1 || pool_kernel % 2 == 0)
    return fail(KVC_ERR_INVALID_ARG, "snapkv: pool_kernel must be odd and >= 1 (got %d)", pool_kernel);
  if (pool_kernel / 2 > kMaxPoolRadius)
    return fail(KVC_ERR_UNSUPPORTED, "snapkv: pool_kernel %d > %d", pool_kernel, 2 * kMaxPoolRadius + 1);
  if (pool_type != KVC_POOL_MAX && pool_type != KVC_POOL_AVG)
    return fail(KVC_ERR_INVALID_ARG, "snapkv: unknown pool type %d", pool_type);
  if (q_len < window) return fail(KVC_ERR_INVALID_ARG, "snapkv: q_len %d < window %d", q_len, window);
  if (D != 64 && D != 128) return fail(KVC_ERR_UNSUPPORTED, "snapkv: head_dim %d not in {64, 128}", D);
  const int64_t es = dt == KVC_BF16 ? 2 : 4;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out))
    return fail(KVC_ERR_INVALID_ARG, "snapkv: device pointers must be 16-byte aligned");
  const int64_t strides[6] = {qs.b, qs.h, qs.t, kvs.b, kvs.h, kvs.t};
  for (int64_t st : strides)
    if (st < 0 || (st * es) % 16 != 0)
      return fail(KVC_ERR_INVALID_ARG, "snapkv: strides must be non-negative and multiples of 16 bytes");
  if (kvs.t < D || qs.t < D)
    return fail(KVC_ERR_INVALID_ARG, "snapkv: row strides must be >= head_dim (D axis contiguous)");
  return KVC_OK;
}

// One validated launch sequence over B*H heads of length L: the score
// schedule, the selection and the gather.
kvc_status snap_core(const void* q, int q_len, kvc_strides qs, const void* k, const void* v, kvc_strides kvs,
                     int B, int H, int L, int D, int window, int budget, int pool_kernel, int avg, kvc_dtype dt,
                     void* k_out, void* v_out, int32_t* idx_out, float* pooled_out, float* vote_out, char* ws,
                     hipStream_t stream) {
  SnapLayout lay;
  snap_layout(B, H, L, D, window, budget, dt, &lay);
  const int64_t es = dt == KVC_BF16 ? 2 : 4;
  const float scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(D)));
  float* vote = vote_out;  // votes are written only when asked for
  unsigned* hist = reinterpret_cast<unsigned*>(ws + lay.hist);
  float* pooled = pooled_out ? pooled_out : reinterpret_cast<float*>(ws + lay.pooled);
  const int qrow0 = q_len - window;

  // AUTO takes the single pass where the independent-wave kernel runs (it
  // reads K once and measures faster there on MI355X), else two passes: the
  // lockstep single-pass kernel that covers shorter heads measures slower than
  // two passes (16K-key heads: 0.156 against 0.125 ms per call), so only an
  // explicit SINGLE_PASS takes it. A failed single-pass launch under AUTO
  // falls back to two passes.
  const bool try_single = dt == KVC_BF16 && g_schedule != KVC_SNAPKV_TWO_PASS;
  const int Gw = try_single ? wave_grid(lay, D, L, kvs.t, qs.t) : 0;
  const int Gc = try_single && (g_schedule == KVC_SNAPKV_SINGLE_PASS || Gw > 0) ? coop_grid(lay, D) : 0;
  int schedule = KVC_SNAPKV_TWO_PASS;
  mark_phase(0, stream);
  // what the selection reads: the pooled scores, or (single pass, max-pool of
  // a small radius) the raw votes, which it then pools itself
  const float* sel_src = pooled;
  int sel_rad = 0;
  bool self_hist = false;
  ExactArgs fused_ea{};
  if (Gw > 0 || Gc > 0) {
    // Raw votes go to the caller's buffer, else to the pooled-score area when
    // the selection pools them (nothing else is stored there then), else to
    // the candidate area, which is free until the selection starts (the
    // pooling kernel has read them by then). The pooling kernel stores pooled
    // scores only if the caller asked for them or the selection reads them.
    const int r = pool_kernel / 2;
    // the selection pools the raw votes itself (max-pool of a small radius),
    // else it reads the pooling kernel's stored scores
    const bool sel_pools = !avg && r <= kSelMaxRad;
    float* vraw = vote ? vote : reinterpret_cast<float*>(ws + (sel_pools ? lay.pooled : lay.cand));
    float* pooled_dst = pooled_out ? pooled_out : sel_pools ? nullptr : pooled;
    const uint16_t* qb = static_cast<const uint16_t*>(q);
    const uint16_t* kb = static_cast<const uint16_t*>(k);
    // The selection also does the pooling kernel's work (histogram, pooled
    // output, exact votes of flagged heads), which is then not launched: one
    // workgroup per head where a head is at most one workgroup's range, else
    // the head's workgroups together (they meet on the head's histogram)
    // where the whole selection grid is resident at once.
    const bool sel_vec = lay.N % 4 == 0 && aligned16(vraw) && (!pooled_out || aligned16(pooled_out));
    const bool per_head = lay.N <= kSelChunk && !g_force_split_select;
    const CoopCaps& caps = coop_caps();
    const int64_t sel_grid = static_cast<int64_t>((lay.N + kSelChunk - 1) / kSelChunk) * lay.BH;
    const bool fuse = sel_pools && sel_vec &&
                      (per_head || (g_force_split_select != 2 && sel_grid <= static_cast<int64_t>(caps.sel_per_cu) * caps.cus));
    ExactArgs* fused_arg = fuse ? &fused_ea : nullptr;
    kvc_status st = D == 128 ? launch_single_pass<128>(lay, Gw, Gc, qb, qs, qrow0, kb, kvs, H, L, window, r, avg,
                                                       scale_log2, ws, vraw, pooled_dst, fused_arg, stream)
                             : launch_single_pass<64>(lay, Gw, Gc, qb, qs, qrow0, kb, kvs, H, L, window, r, avg,
                                                      scale_log2, ws, vraw, pooled_dst, fused_arg, stream);
    if (st == KVC_OK) {
      schedule = KVC_SNAPKV_SINGLE_PASS;
      self_hist = fuse;
      g_last_pool = fuse ? (per_head ? "snap_select_head" : "snap_select")
                         : r <= kPoolRegRadius ? "snap_pool" : "snap_pool_lds";
      if (sel_pools) {
        sel_src = vraw;
        sel_rad = r;
      }
    } else if (g_schedule == KVC_SNAPKV_SINGLE_PASS) {
      return st;
    } else {
      clear_error();
      (void)hipGetLastError();
    }
  }
  if (schedule == KVC_SNAPKV_TWO_PASS) {
    mark_phase(1, stream);  // counters and histograms are cleared by the statistics pass
    g_last_kernel = dt == KVC_BF16 ? "snap_stats_bf16+snap_votes_bf16" : "snap_stats_f32+snap_votes_f32";
    g_last_pool = dt == KVC_BF16 ? "snap_votes_bf16" : "snap_votes_f32";
    if (dt == KVC_BF16)
      launch_score_passes<uint16_t>(lay, static_cast<const uint16_t*>(q), qs, qrow0,
                                    static_cast<const uint16_t*>(k), kvs, H, L, D, window, pool_kernel / 2, avg,
                                    scale_log2, ws, vote, pooled, stream);
    else
      launch_score_passes<float>(lay, static_cast<const float*>(q), qs, qrow0, static_cast<const float*>(k), kvs, H,
                                 L, D, window, pool_kernel / 2, avg, scale_log2, ws, vote, pooled, stream);
  }
  kvc_status st = check_launch("snapkv score passes");
  if (st != KVC_OK) return st;

  const int vec = lay.N % 4 == 0 && aligned16(sel_src);
  // a wave checks whether its range can reach the threshold bin before it
  // classifies only where few positions are kept (the check costs more than
  // it saves where most waves hold a kept position)
  const int skip = static_cast<int64_t>(lay.kk) * 128 < lay.N ? 1 : 0;
  if (vec && lay.N <= kSelChunk && !g_force_split_select) {
    // one workgroup per head (a head of at most one workgroup's range): no
    // exchange between workgroups
    snap_select_head<<<static_cast<unsigned>(lay.BH), kSelThreads, 0, stream>>>(
        sel_src, sel_rad, skip, hist, lay.N, lay.kk, reinterpret_cast<unsigned*>(ws + lay.sel_ctr),
        reinterpret_cast<uint2*>(ws + lay.cand), idx_out, self_hist ? 1 : 0, self_hist ? pooled_out : nullptr,
        fused_ea);
    g_last_select = "snap_select_head";
  } else {
    const dim3 gs((lay.N + kSelChunk - 1) / kSelChunk, static_cast<unsigned>(lay.BH));
    snap_select<<<gs, kSelThreads, 0, stream>>>(sel_src, vec, sel_rad, skip, hist, lay.N, lay.kk,
                                                reinterpret_cast<unsigned*>(ws + lay.sel_ctr),
                                                reinterpret_cast<uint2*>(ws + lay.cand),
                                                reinterpret_cast<unsigned*>(ws + lay.bitmap), idx_out,
                                                self_hist ? 1 : 0, self_hist ? pooled_out : nullptr, fused_ea,
                                                g_force_wait_timeout ? kWvSpinForced : kSelHistSpin);
    g_last_select = "snap_select";
  }
  mark_phase(5, stream);
  st = check_launch("snapkv selection");
  if (st != KVC_OK) return st;

  const int vec_per_row = static_cast<int>(D * es / 16);  // 16-byte pieces per row
  const int64_t pieces = static_cast<int64_t>(budget) * vec_per_row;
  const int64_t per_block = static_cast<int64_t>(kThreads) * kGatherPer;
  const dim3 gg(static_cast<unsigned>((pieces + per_block - 1) / per_block), static_cast<unsigned>(lay.BH));
  snap_gather<<<gg, kThreads, 0, stream>>>(static_cast<const char*>(k), static_cast<const char*>(v),
                                           kvs.b * es, kvs.h * es, kvs.t * es, H, L, window, budget, lay.kk,
                                           vec_per_row, idx_out, static_cast<char*>(k_out),
                                           static_cast<char*>(v_out));
  mark_phase(6, stream);
  st = check_launch("snapkv gather");
  if (st == KVC_OK) g_last_schedule = schedule;
  return st;
}

}  // namespace
}  // namespace kvc

extern "C" kvc_status kvc_snapkv_compress(const void* q, int q_len, kvc_strides qs, const void* k,
                                          const void* v, kvc_strides kvs, int B, int H, int L, int D,
                                          int window, int budget, int pool_kernel, kvc_dtype dt,
                                          void* k_out, void* v_out, int32_t* idx_out,
                                          float* pooled_out, float* vote_out, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  kvc_status st = snap_validate(q, q_len, qs, k, v, kvs, B, H, L, D, window, budget, pool_kernel, KVC_POOL_MAX, dt,
                                k_out, v_out, idx_out);
  if (st != KVC_OK) return st;
  SnapLayout lay;
  snap_layout(B, H, L, D, window, budget, dt, &lay);
  if (!workspace || workspace_bytes < lay.total)
    return fail(KVC_ERR_WORKSPACE, "snapkv: workspace of %zu bytes needed, got %zu", lay.total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(KVC_ERR_INVALID_ARG, "snapkv: workspace must be 16-byte aligned");
  return snap_core(q, q_len, qs, k, v, kvs, B, H, L, D, window, budget, pool_kernel, 0, dt, k_out, v_out, idx_out,
                   pooled_out, vote_out, static_cast<char*>(workspace), stream);
}

extern "C" size_t kvc_snapkv_workspace_bytes_ex(int n_layers, int B, int H, int L, int D, int window, int budget,
                                                int pool_kernel, kvc_dtype dt, int ragged) {
  (void)pool_kernel;
  if (n_layers < 1 || B < 1) return 0;
  // a ragged batch runs one sequence of one layer per launch sequence; else
  // the layers run together as one batch of n_layers * B (or one by one)
  const int64_t Bc = ragged ? 1 : static_cast<int64_t>(n_layers) * B;
  if (Bc > INT32_MAX) return 0;
  SnapLayout lay;
  if (!snap_layout(static_cast<int>(Bc), H, L, D, window, budget, dt, &lay)) return 0;
  return lay.total;
}

extern "C" kvc_status kvc_snapkv_compress_ex(const void* q, int q_len, kvc_strides qs, int64_t q_layer_stride,
                                             const void* k, const void* v, kvc_strides kvs,
                                             int64_t kv_layer_stride, int n_layers, int B, int H, int L, int D,
                                             const int32_t* lengths, int window, int budget, int pool_kernel,
                                             int pool_type, kvc_dtype dt, void* k_out, void* v_out,
                                             int32_t* idx_out, float* pooled_out, float* vote_out,
                                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  if (n_layers < 1) return fail(KVC_ERR_INVALID_ARG, "snapkv: n_layers must be >= 1 (got %d)", n_layers);
  kvc_status st = snap_validate(q, q_len, qs, k, v, kvs, B, H, L, D, window, budget, pool_kernel, pool_type, dt,
                                k_out, v_out, idx_out);
  if (st != KVC_OK) return st;
  const int64_t es = dt == KVC_BF16 ? 2 : 4;
  if (n_layers > 1 && (q_layer_stride < 0 || kv_layer_stride < 0 || (q_layer_stride * es) % 16 != 0 ||
                       (kv_layer_stride * es) % 16 != 0))
    return fail(KVC_ERR_INVALID_ARG, "snapkv: layer strides must be non-negative and multiples of 16 bytes");
  if (static_cast<int64_t>(n_layers) * B * H > INT32_MAX)
    return fail(KVC_ERR_UNSUPPORTED, "snapkv: n_layers * B * H too large");
  if (lengths)
    for (int b = 0; b < B; ++b)
      if (lengths[b] <= budget || lengths[b] > L)
        return fail(KVC_ERR_INVALID_ARG, "snapkv: lengths[%d] = %d must satisfy budget (%d) < length <= L (%d)", b,
                    lengths[b], budget, L);
  const size_t need = kvc_snapkv_workspace_bytes_ex(n_layers, B, H, L, D, window, budget, pool_kernel, dt,
                                                    lengths != nullptr);
  if (need == 0) return fail(KVC_ERR_UNSUPPORTED, "snapkv: sizes out of range");
  if (!workspace || workspace_bytes < need)
    return fail(KVC_ERR_WORKSPACE, "snapkv: workspace of %zu bytes needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(KVC_ERR_INVALID_ARG, "snapkv: workspace must be 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  const int avg = pool_type == KVC_POOL_AVG;
  const int kk = budget - window;
  const int64_t out_bh = static_cast<int64_t>(budget) * D * es;  // output bytes per head
  char* ko = static_cast<char*>(k_out);
  char* vo = static_cast<char*>(v_out);
  const char* qc = static_cast<const char*>(q);
  const char* kc = static_cast<const char*>(k);
  const char* vc = static_cast<const char*>(v);
  if (!lengths) {
    const int64_t N = L - window;
    const bool fold = n_layers == 1 || (q_layer_stride == static_cast<int64_t>(B) * qs.b &&
                                        kv_layer_stride == static_cast<int64_t>(B) * kvs.b);
    if (fold) {  // the layers are one batch of n_layers * B sequences
      if (static_cast<int64_t>(n_layers) * B * H > 65535)
        return fail(KVC_ERR_UNSUPPORTED, "snapkv: n_layers * B * H must be <= 65535");
      return snap_core(q, q_len, qs, k, v, kvs, n_layers * B, H, L, D, window, budget, pool_kernel, avg, dt, k_out,
                       v_out, idx_out, pooled_out, vote_out, ws, stream);
    }
    for (int l = 0; l < n_layers; ++l) {  // layer by layer, one workspace reused in stream order
      const int64_t bh0 = static_cast<int64_t>(l) * B * H;
      st = snap_core(qc + l * q_layer_stride * es, q_len, qs, kc + l * kv_layer_stride * es,
                     vc + l * kv_layer_stride * es, kvs, B, H, L, D, window, budget, pool_kernel, avg, dt,
                     ko + bh0 * out_bh, vo + bh0 * out_bh, idx_out + bh0 * kk, pooled_out ? pooled_out + bh0 * N : nullptr,
                     vote_out ? vote_out + bh0 * N : nullptr, ws, stream);
      if (st != KVC_OK) return st;
    }
    return KVC_OK;
  }
  // ragged: sequence b of layer l is its own launch sequence over its
  // lengths[b] keys; pooled / vote rows are packed per (l, b) in that order,
  // H rows of lengths[b] - window each
  int64_t packed = 0;
  for (int l = 0; l < n_layers; ++l) {
    for (int b = 0; b < B; ++b) {
      const int Lb = lengths[b];
      const int64_t bh0 = (static_cast<int64_t>(l) * B + b) * H;
      st = snap_core(qc + (l * q_layer_stride + b * qs.b) * es, q_len, qs,
                     kc + (l * kv_layer_stride + b * kvs.b) * es, vc + (l * kv_layer_stride + b * kvs.b) * es, kvs, 1,
                     H, Lb, D, window, budget, pool_kernel, avg, dt, ko + bh0 * out_bh, vo + bh0 * out_bh,
                     idx_out + bh0 * kk, pooled_out ? pooled_out + packed : nullptr,
                     vote_out ? vote_out + packed : nullptr, ws, stream);
      if (st != KVC_OK) return st;
      packed += static_cast<int64_t>(H) * (Lb - window);
    }
  }
  return KVC_OK;
}

extern "C" void kvc_snapkv_set_phase_events(hipEvent_t* events, int n_events) {
  g_phase_events = n_events > 0 ? events : nullptr;
  g_phase_count = n_events > 0 ? n_events : 0;
}

