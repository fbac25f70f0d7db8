// H2O heavy-hitter + recent KV-cache step on gfx950.
//
// The method (abeam.tech summary of "H2O: Heavy-Hitter Oracle for Efficient
// Generative Inference of Large Language Models", section 技術の仕組み,
// subsections 処理の流れ and 何を残すのか): every decode step, the new query's
// attention probabilities are added to each cached token's running score; when
// the cache is over budget, the most recent tokens stay and the rest of the
// budget goes to the tokens with the largest running score.
//
// One workgroup per (batch, head). The step is HBM-bound: it streams the K
// rows once for the scores (and the V rows once when the attention output is
// requested); everything else lives in LDS. Per-slot state (score, position)
// is held in LDS for the whole step, so the cache capacity is bounded by LDS.
#include <math.h>

#include "common.hpp"

namespace kvc {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxCap = 8192;  // 12 bytes of LDS per slot

__device__ __forceinline__ float block_max(float x, float* red) {
  x = wave_max(x);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) red[w] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) red[w] = x;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) r += red[i];
  __syncthreads();
  return r;
}

// Eviction order key: smaller score first, then older position first.
__device__ __forceinline__ unsigned long long evict_key(float acc, int pos) {
  return (static_cast<unsigned long long>(__float_as_uint(acc)) << 32) | static_cast<unsigned>(pos);
}

// The smallest (score, position) key among slots j < N whose position is
// below rthr: evict_threshold for E = 1 (the usual decode step), by one
// block-wide minimum. red: kWaves words of LDS. Every thread calls it.
__device__ unsigned long long evict_min(const float* s_val, const int* s_pos, int N, int rthr,
                                        unsigned long long* red) {
  unsigned long long m = ~0ull;
  for (int j = threadIdx.x; j < N; j += blockDim.x)
    if (s_pos[j] < rthr) m = min(m, evict_key(s_val[j], s_pos[j]));
  m = min(m, lane_xor_u64<32>(m));
  m = min(m, lane_xor_u64<16>(m));
  m = min(m, lane_xor_u64<8>(m));
  m = min(m, lane_xor_u64<4>(m));
  m = min(m, lane_xor_u64<2>(m));
  m = min(m, lane_xor_u64<1>(m));
  if (lane_id() == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  unsigned long long r = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = min(r, red[i]);
  __syncthreads();
  return r;
}

// Key of the E-th smallest (score, position) among slots j < N whose position
// is below rthr (the non-recent tokens): radix select, 8 bits at a time from the
// top. Slots with a key <= the result are exactly the E to evict (keys are
// distinct). dh: 256 LDS counters. Every thread of the block calls it.
__device__ unsigned long long evict_threshold(const float* s_val, const int* s_pos, int N, int rthr,
                                              unsigned E, unsigned* dh) {
  __shared__ unsigned s_digit, s_below;
  unsigned rem = E;
  unsigned long long prefix = 0, pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) dh[i] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < N; j += blockDim.x) {
      if (s_pos[j] >= rthr) continue;
      const unsigned long long key = evict_key(s_val[j], s_pos[j]);
      if ((key & pmask) == prefix) atomicAdd(&dh[(key >> shift) & 255], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      unsigned c4[4], c = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c4[i] = dh[4 * threadIdx.x + i];
        c += c4[i];
      }
      const unsigned incl = wave_incl_scan(c);
      const unsigned lower = incl - c;  // digits owned by lower lanes
      if (lower < rem && lower + c >= rem) {
        unsigned run = lower;
        for (int i = 0; i < 4; ++i) {
          if (run + c4[i] >= rem) {
            s_digit = 4 * threadIdx.x + i;
            s_below = run;
            break;
          }
          run += c4[i];
        }
      }
    }
    __syncthreads();
    rem -= s_below;
    prefix |= static_cast<unsigned long long>(s_digit) << shift;
    pmask |= 0xFFull << shift;
    __syncthreads();
  }
  return prefix;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads, 8) void h2o_step_kernel(
    char* __restrict__ kc, char* __restrict__ vc, int* __restrict__ pos_g, float* __restrict__ acc_g,
    int cap, int n, int new_pos, const char* __restrict__ q, const char* __restrict__ kn,
    const char* __restrict__ vn, int n_heavy, int n_recent, float scale_log2, float* __restrict__ out) {
  constexpr int VE = Vec16<T>::kN;             // elements per 16-byte piece
  constexpr int LPR = D / VE;                  // lanes per row
  constexpr int RPW = kWave / LPR;             // rows per wave instruction
  constexpr int RB = D * static_cast<int>(sizeof(T));  // row bytes
  extern __shared__ unsigned char smem[];
  const int N = n + 1;
  float* s_val = reinterpret_cast<float*>(smem);           // scores, then running scores
  int* s_pos = reinterpret_cast<int*>(s_val + N);          // positions
  int* s_list = s_pos + N;                                 // holes from the front, movers from the back
  __shared__ float red[kWaves];
  __shared__ float ored[kWaves][D];
  __shared__ unsigned dh[256];
  __shared__ unsigned scratch[kWaves + 1];

  const int bh = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int sub = lane % LPR, grp = lane / LPR;
  const int64_t slot0 = static_cast<int64_t>(bh) * cap;
  char* kb = kc + slot0 * RB;
  char* vb = vc + slot0 * RB;
  const char* knr = kn + static_cast<int64_t>(bh) * RB;
  const char* vnr = vn + static_cast<int64_t>(bh) * RB;

  // Append the new token in slot n (its K/V row; score and position go to LDS).
  for (int i = threadIdx.x; i < RB / 16; i += kThreads) {
    *reinterpret_cast<u32x4_t*>(kb + static_cast<int64_t>(n) * RB + i * 16) =
        *reinterpret_cast<const u32x4_t*>(knr + i * 16);
    *reinterpret_cast<u32x4_t*>(vb + static_cast<int64_t>(n) * RB + i * 16) =
        *reinterpret_cast<const u32x4_t*>(vnr + i * 16);
  }
  float qv[VE];
  Vec16<T>::load(q + static_cast<int64_t>(bh) * RB + sub * 16, qv);
  // The slots' positions and running scores, loaded now so that they arrive
  // while the scores are computed (the first kPre * kThreads slots).
  constexpr int kPre = 4;
  int pre_pos[kPre];
  float pre_acc[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int j = threadIdx.x + u * kThreads;
    pre_pos[u] = j < n ? pos_g[slot0 + j] : new_pos;
    pre_acc[u] = j < n ? acc_g[slot0 + j] : 0.f;
  }

  // Scores of all N slots; the new token's key is read from k_new. kStepRows
  // row groups per iteration, their loads all issued before any is used.
  constexpr int kStepRows = D >= 128 ? 3 : 2;
  float lmax = -INFINITY;
  for (int j0 = wave * RPW; j0 < N; j0 += kWaves * RPW * kStepRows) {
    float kx[kStepRows][VE];
#pragma unroll
    for (int u = 0; u < kStepRows; ++u) {
      const int j = j0 + u * kWaves * RPW + grp;
      if (j < N) Vec16<T>::load((j < n ? kb + static_cast<int64_t>(j) * RB : knr) + sub * 16, kx[u]);
    }
#pragma unroll
    for (int u = 0; u < kStepRows; ++u) {
      const int j = j0 + u * kWaves * RPW + grp;
      float dot = 0.f;
      if (j < N) {
#pragma unroll
        for (int e = 0; e < VE; ++e) dot += qv[e] * kx[u][e];
      }
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) dot += lane_xor_n(dot, o);
      if (j < N && sub == 0) {
        const float s2 = dot * scale_log2;
        s_val[j] = s2;
        lmax = fmaxf(lmax, s2);
      }
    }
  }
  // positions to LDS, running scores parked in the eviction list's space
  // until the update below
  float* s_acc = reinterpret_cast<float*>(s_list);
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int j = threadIdx.x + u * kThreads;
    if (j < N) {
      s_pos[j] = pre_pos[u];
      s_acc[j] = pre_acc[u];
    }
  }
  for (int j = threadIdx.x + kPre * kThreads; j < N; j += kThreads) {
    s_pos[j] = j < n ? pos_g[slot0 + j] : new_pos;
    s_acc[j] = j < n ? acc_g[slot0 + j] : 0.f;
  }
  __syncthreads();
  const float m2 = block_max(lmax, red);
  float lsum = 0.f;
  for (int j = threadIdx.x; j < N; j += kThreads) lsum += fast_exp2(s_val[j] - m2);
  const float inv = 1.f / block_sum(lsum, red);

  // Optional attention output o = sum_j p_j v_j (before eviction).
  if (out) {
    float ov[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) ov[e] = 0.f;
    for (int j0 = wave * RPW; j0 < N; j0 += kWaves * RPW * kStepRows) {
      float vx[kStepRows][VE];
#pragma unroll
      for (int u = 0; u < kStepRows; ++u) {
        const int j = j0 + u * kWaves * RPW + grp;
        if (j < N) Vec16<T>::load((j < n ? vb + static_cast<int64_t>(j) * RB : vnr) + sub * 16, vx[u]);
      }
#pragma unroll
      for (int u = 0; u < kStepRows; ++u) {
        const int j = j0 + u * kWaves * RPW + grp;
        if (j < N) {
          const float p = fast_exp2(s_val[j] - m2) * inv;
#pragma unroll
          for (int e = 0; e < VE; ++e) ov[e] += p * vx[u][e];
        }
      }
    }
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1)
#pragma unroll
      for (int e = 0; e < VE; ++e) ov[e] += lane_xor_n(ov[e], o);
    if (grp == 0)
#pragma unroll
      for (int e = 0; e < VE; ++e) ored[wave][sub * VE + e] = ov[e];
  }
  __syncthreads();
  if (out && threadIdx.x < D) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) s += ored[i][threadIdx.x];
    out[static_cast<int64_t>(bh) * D + threadIdx.x] = s;
  }

  // Running scores: acc += p (the new token starts from 0).
  for (int j = threadIdx.x; j < N; j += kThreads) {
    const float p = fast_exp2(s_val[j] - m2) * inv;
    s_val[j] = s_acc[j] + p;
  }
  __syncthreads();

  const int budget = n_heavy + n_recent;
  int n_keep = N;
  if (N > budget) {
    // Evict the E smallest (score, position) keys among the non-recent tokens.
    const int length = new_pos + 1;
    const int rthr = length - n_recent;  // positions >= rthr are recent
    const int E = N - budget;
    n_keep = budget;
    __shared__ unsigned long long red64[kWaves];
    const unsigned long long prefix = E == 1 ? evict_min(s_val, s_pos, N, rthr, red64)
                                             : evict_threshold(s_val, s_pos, N, rthr, static_cast<unsigned>(E), dh);
    // prefix = key of the last evicted token. Holes: evicted slots below
    // n_keep; movers: kept slots at or above n_keep. Pair them by rank.
    const int seg = (N + kThreads - 1) / kThreads;
    const int a0 = min(N, static_cast<int>(threadIdx.x) * seg), a1 = min(N, a0 + seg);
    unsigned nh = 0, nm = 0;
    for (int j = a0; j < a1; ++j) {
      const bool ev = s_pos[j] < rthr && evict_key(s_val[j], s_pos[j]) <= prefix;
      nh += (ev && j < n_keep);
      nm += (!ev && j >= n_keep);
    }
    unsigned th, tm;
    unsigned oh = block_excl_scan<kThreads>(nh, scratch, &th);
    unsigned om = block_excl_scan<kThreads>(nm, scratch, &tm);
    for (int j = a0; j < a1; ++j) {
      const bool ev = s_pos[j] < rthr && evict_key(s_val[j], s_pos[j]) <= prefix;
      if (ev && j < n_keep) s_list[oh++] = j;
      if (!ev && j >= n_keep) s_list[N - 1 - static_cast<int>(om++)] = j;
    }
    __syncthreads();
    const int moves = static_cast<int>(min(th, tm));
    // move K/V rows: one 16-byte piece per thread per iteration
    for (int i = threadIdx.x; i < moves * (RB / 16); i += kThreads) {
      const int r = i / (RB / 16), c = i - r * (RB / 16);
      const int dst = s_list[r], src = s_list[N - 1 - r];
      *reinterpret_cast<u32x4_t*>(kb + static_cast<int64_t>(dst) * RB + c * 16) =
          *reinterpret_cast<const u32x4_t*>(kb + static_cast<int64_t>(src) * RB + c * 16);
      *reinterpret_cast<u32x4_t*>(vb + static_cast<int64_t>(dst) * RB + c * 16) =
          *reinterpret_cast<const u32x4_t*>(vb + static_cast<int64_t>(src) * RB + c * 16);
    }
    __syncthreads();
    for (int r = threadIdx.x; r < moves; r += kThreads) {
      const int dst = s_list[r], src = s_list[N - 1 - r];
      s_val[dst] = s_val[src];
      s_pos[dst] = s_pos[src];
    }
    __syncthreads();
  }
  for (int j = threadIdx.x; j < n_keep; j += kThreads) {
    acc_g[slot0 + j] = s_val[j];
    pos_g[slot0 + j] = s_pos[j];
  }
}

template <typename T, int D>
kvc_status launch_h2o(kvc_h2o_cache* c, const void* q, const void* kn, const void* vn, int n_heavy,
                      int n_recent, float* out, hipStream_t stream) {
  const int N = c->n + 1;
  const size_t smem = static_cast<size_t>(N) * 12;
  const float scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(D)));
  const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(c->B) * c->H);
  h2o_step_kernel<T, D><<<grid, kThreads, smem, stream>>>(
      static_cast<char*>(c->k), static_cast<char*>(c->v), c->pos, c->acc, c->cap, c->n,
      static_cast<int>(c->len), static_cast<const char*>(q), static_cast<const char*>(kn),
      static_cast<const char*>(vn), n_heavy, n_recent, scale_log2, out);
  return check_launch("h2o step");
}

// ------------------------------------------------------------------ prefill
//
// Initial scores after the prompt (H2O page: local statistics are the
// attention observed so far): score of prompt token j = sum over prompt
// queries i >= j of the causal softmax weight P[i, j]. Pass 1 gives every
// query row its (max, 1/sum) (a workgroup owns 32 whole rows); pass 2 sums
// each key column over the rows that see it (a workgroup owns 32 whole
// columns); pass 3 applies the heavy + recent eviction at length = prompt
// length and writes the kept tokens into the cache in position order.

constexpr int kPTile = 32;
constexpr float kNegBig = -1.0e30f;

template <int D>
__device__ __forceinline__ void load_frag(const uint16_t* p, bf16x8_t (&f)[D / 16]) {
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = __builtin_bit_cast(bf16x8_t, src[s]);
}

__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// bf16 passes: a workgroup owns kWaves consecutive 32-row tiles (one per wave)
// of its head and streams the other operand's tiles through a double-buffered
// LDS ring, so each streamed tile is read from L2 once per workgroup instead of
// once per wave. Rows in LDS are padded by 16 bytes: a wave's 16-byte fragment
// reads (32 rows at one column offset) then spread over all LDS banks.
template <int D>
constexpr int kPRow = D + 8;  // LDS row stride in bf16 elements

// Block id -> (head, group) so that the groups of one head run on one XCD
// (workgroups are dealt to the 8 XCDs round-robin by linear id): a head's K and
// Q stay in that XCD's L2 while its groups run. Heavier groups (more tiles in
// the causal triangle) are issued first. Any bijection is correct.
__device__ __forceinline__ void xcd_group(int64_t id, int64_t total, int nb, bool heavy_last, int& bh, int& g) {
  const int64_t x = id & 7, slot = id >> 3, q = total >> 3, r = total & 7;
  const int64_t lin = x * q + (x < r ? x : r) + slot;
  bh = static_cast<int>(lin / nb);
  const int i = static_cast<int>(lin - static_cast<int64_t>(bh) * nb);
  g = heavy_last ? nb - 1 - i : i;
}

// Global -> registers part of staging one 32-row tile (rows clamped to Lp - 1):
// 16-byte pieces, consecutive threads on consecutive pieces of a row.
template <int D>
__device__ __forceinline__ void tile_load(const uint16_t* base, int64_t st, int row0, int Lp,
                                          u32x4_t (&r)[D / 64]) {
  constexpr int kChunks = D / 8;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const int p = static_cast<int>(threadIdx.x) + i * kThreads;
    const int row = p / kChunks, c = p - row * kChunks;
    r[i] = *reinterpret_cast<const u32x4_t*>(base + static_cast<int64_t>(min(row0 + row, Lp - 1)) * st + c * 8);
  }
}

template <int D>
__device__ __forceinline__ void tile_store(uint16_t* t, const u32x4_t (&r)[D / 64]) {
  constexpr int kChunks = D / 8;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const int p = static_cast<int>(threadIdx.x) + i * kThreads;
    const int row = p / kChunks, c = p - row * kChunks;
    *reinterpret_cast<u32x4_t*>(t + row * kPRow<D> + c * 8) = r[i];
  }
}

// MFMA operand of lane (col, half): row col, elements [half*D/2, half*D/2 + D/2)
// (the same permutation of the head dimension on both operands).
template <int D>
__device__ __forceinline__ void frag_lds(const uint16_t* t, int col, int half, bf16x8_t (&f)[D / 16]) {
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(t + col * kPRow<D> + half * (D / 2));
#pragma unroll
  for (int s = 0; s < D / 16; ++s) f[s] = __builtin_bit_cast(bf16x8_t, src[s]);
}

// Pass 1, output S^T (lane = query row): per-row running max/sum over the key
// tiles up to the row's own (the diagonal tile is the only one that needs the
// causal mask; rows past Lp in the last tile are not written).
template <int D>
__global__ __launch_bounds__(kThreads) void h2o_prefill_stats_bf16(
    const uint16_t* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qst, const uint16_t* __restrict__ k,
    int64_t ksb, int64_t ksh, int64_t kst, int H, int Lp, int nb, float scale_log2, float2* __restrict__ stat) {
  constexpr int KS = D / 16;
  __shared__ __align__(16) uint16_t ring[2][kPTile * kPRow<D>];
  int bh, g;
  xcd_group(blockIdx.x, gridDim.x, nb, true, bh, g);
  const int b = bh / H, h = bh - b * H;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int col = lane & 31, half = lane >> 5;
  const int nqt = (Lp + kPTile - 1) / kPTile;
  const int qt = g * kWaves + wave;
  const int qi = qt * kPTile + col;
  const int last = min(g * kWaves + kWaves - 1, nqt - 1);
  bf16x8_t qf[KS];
  load_frag<D>(q + b * qsb + h * qsh + static_cast<int64_t>(min(qi, Lp - 1)) * qst + half * (D / 2), qf);
  const uint16_t* kb = k + b * ksb + h * ksh;
  u32x4_t stage[D / 64];
  tile_load<D>(kb, kst, 0, Lp, stage);
  tile_store<D>(ring[0], stage);
  __syncthreads();
  float m_run = kNegBig, l_run = 0.f;
  for (int kt = 0; kt <= last; ++kt) {
    if (kt < last) tile_load<D>(kb, kst, (kt + 1) * kPTile, Lp, stage);
    if (kt <= qt && qt < nqt) {
      bf16x8_t kf[KS];
      frag_lds<D>(ring[kt & 1], col, half, kf);
      f32x16_t acc = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], acc, 0, 0, 0);
      if (kt == qt) {
        // -inf, not a large finite value: a half-wave whose rows are all masked
        // then adds exactly 0 (fma(-big, scale, -m) can round to a large positive).
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * kPTile + acc_row(r, half) > qi) acc[r] = -__builtin_inff();
      }
      float tmax = acc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, acc[r]);
      const float mnew = fmaxf(m_run, tmax * scale_log2);
      float add = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) add += fast_exp2(fmaf(acc[r], scale_log2, -mnew));
      l_run = l_run * fast_exp2(m_run - mnew) + add;
      m_run = mnew;
    }
    if (kt < last) tile_store<D>(ring[(kt + 1) & 1], stage);
    __syncthreads();
  }
  lse2_merge(m_run, l_run, lane_xor<32>(m_run), lane_xor<32>(l_run));
  if (half == 0 && qi < Lp) stat[static_cast<int64_t>(bh) * Lp + qi] = make_float2(m_run, 1.f / l_run);
}

// Pass 2, output S (lane = key column): column sums of the normalised weights
// over the query tiles from the column's own to the last. With
// c_i = m_i + log2(l_i), each weight is 2^(s*scale - c_i); rows past Lp get
// c = +1e30 (weight 0), so only the diagonal tile needs a mask.
template <int D>
__global__ __launch_bounds__(kThreads) void h2o_prefill_colsum_bf16(
    const uint16_t* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qst, const uint16_t* __restrict__ k,
    int64_t ksb, int64_t ksh, int64_t kst, int H, int Lp, int nb, float scale_log2,
    const float2* __restrict__ stat, float* __restrict__ colsum) {
  constexpr int KS = D / 16;
  __shared__ __align__(16) uint16_t ring[2][kPTile * kPRow<D>];
  __shared__ __align__(16) float cring[2][kPTile];
  int bh, g;
  xcd_group(blockIdx.x, gridDim.x, nb, false, bh, g);
  const int b = bh / H, h = bh - b * H;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int col = lane & 31, half = lane >> 5;
  const int nqt = (Lp + kPTile - 1) / kPTile;
  const int kt = g * kWaves + wave;
  const int kj = kt * kPTile + col;
  const int first = g * kWaves;
  bf16x8_t kf[KS];
  load_frag<D>(k + b * ksb + h * ksh + static_cast<int64_t>(min(kj, Lp - 1)) * kst + half * (D / 2), kf);
  const uint16_t* qb = q + b * qsb + h * qsh;
  const float2* sb = stat + static_cast<int64_t>(bh) * Lp;
  u32x4_t stage[D / 64];
  float cst = 0.f;
  auto load_c = [&](int qt) {
    if (threadIdx.x < kPTile) {
      const int i = qt * kPTile + static_cast<int>(threadIdx.x);
      cst = 1.0e30f;
      if (i < Lp) {
        const float2 v = sb[i];
        cst = v.x - __builtin_amdgcn_logf(v.y);
      }
    }
  };
  tile_load<D>(qb, qst, first * kPTile, Lp, stage);
  load_c(first);
  tile_store<D>(ring[0], stage);
  if (threadIdx.x < kPTile) cring[0][threadIdx.x] = cst;
  __syncthreads();
  float csum = 0.f;
  for (int qt = first; qt < nqt; ++qt) {
    const int cur = (qt - first) & 1;
    if (qt + 1 < nqt) {
      tile_load<D>(qb, qst, (qt + 1) * kPTile, Lp, stage);
      load_c(qt + 1);
    }
    if (qt >= kt) {
      bf16x8_t qf[KS];
      frag_lds<D>(ring[cur], col, half, qf);
      f32x16_t acc = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[s], kf[s], acc, 0, 0, 0);
      float cr[16];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float4 c4 = *reinterpret_cast<const float4*>(&cring[cur][8 * gq + 4 * half]);
        cr[4 * gq] = c4.x; cr[4 * gq + 1] = c4.y; cr[4 * gq + 2] = c4.z; cr[4 * gq + 3] = c4.w;
      }
      if (qt == kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_row(r, half) < col) cr[r] = 1.0e30f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) csum += fast_exp2(fmaf(acc[r], scale_log2, -cr[r]));
    }
    if (qt + 1 < nqt) {
      tile_store<D>(ring[cur ^ 1], stage);
      if (threadIdx.x < kPTile) cring[cur ^ 1][threadIdx.x] = cst;
    }
    __syncthreads();
  }
  csum += lane_xor<32>(csum);
  if (half == 0 && kj < Lp) colsum[static_cast<int64_t>(bh) * Lp + kj] = csum;
}

// fp32, VALU: a query row (pass 1) or a key column (pass 2) per thread.
template <int D>
__global__ __launch_bounds__(kThreads) void h2o_prefill_stats_f32(
    const float* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qst, const float* __restrict__ k,
    int64_t ksb, int64_t ksh, int64_t kst, int H, int Lp, float scale_log2, float2* __restrict__ stat) {
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= Lp) return;
  const float* qr = q + b * qsb + h * qsh + static_cast<int64_t>(i) * qst;
  const float* kb = k + b * ksb + h * ksh;
  float m = kNegBig, l = 0.f;
  for (int j = 0; j <= i; ++j) {
    float s = 0.f;
    for (int d = 0; d < D; ++d) s += qr[d] * kb[static_cast<int64_t>(j) * kst + d];
    s *= scale_log2;
    const float mn = fmaxf(m, s);
    l = l * fast_exp2(m - mn) + fast_exp2(s - mn);
    m = mn;
  }
  stat[static_cast<int64_t>(bh) * Lp + i] = make_float2(m, 1.f / l);
}

template <int D>
__global__ __launch_bounds__(kThreads) void h2o_prefill_colsum_f32(
    const float* __restrict__ q, int64_t qsb, int64_t qsh, int64_t qst, const float* __restrict__ k,
    int64_t ksb, int64_t ksh, int64_t kst, int H, int Lp, float scale_log2, const float2* __restrict__ stat,
    float* __restrict__ colsum) {
  const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int j = blockIdx.x * kThreads + threadIdx.x;
  if (j >= Lp) return;
  const float* kr = k + b * ksb + h * ksh + static_cast<int64_t>(j) * kst;
  const float* qb = q + b * qsb + h * qsh;
  float c = 0.f;
  for (int i = j; i < Lp; ++i) {
    float s = 0.f;
    for (int d = 0; d < D; ++d) s += qb[static_cast<int64_t>(i) * qst + d] * kr[d];
    const float2 st = stat[static_cast<int64_t>(bh) * Lp + i];
    c += fast_exp2(s * scale_log2 - st.x) * st.y;
  }
  colsum[static_cast<int64_t>(bh) * Lp + j] = c;
}

// Pass 3: eviction at length = Lp, then the kept tokens go to slots 0..n-1 in
// ascending position order. Dynamic LDS: scores, positions and the slot map
// (12 bytes per prompt token).
template <int RB>
__global__ __launch_bounds__(kThreads) void h2o_prefill_evict(
    const char* __restrict__ k, const char* __restrict__ v, int64_t sb, int64_t sh, int64_t st, int H, int Lp,
    int n_heavy, int n_recent, const float* __restrict__ colsum, char* __restrict__ kc, char* __restrict__ vc,
    int* __restrict__ pos_g, float* __restrict__ acc_g, int cap) {
  extern __shared__ unsigned char smem[];
  float* s_val = reinterpret_cast<float*>(smem);
  int* s_pos = reinterpret_cast<int*>(s_val + Lp);
  int* s_map = s_pos + Lp;
  __shared__ unsigned dh[256];
  __shared__ unsigned scratch[kWaves + 1];
  const int bh = blockIdx.x, b = bh / H, h = bh - b * H;
  for (int j = threadIdx.x; j < Lp; j += kThreads) {
    s_val[j] = colsum[static_cast<int64_t>(bh) * Lp + j];
    s_pos[j] = j;
  }
  __syncthreads();
  const int budget = n_heavy + n_recent;
  const int rthr = Lp - n_recent;
  unsigned long long prefix = 0;
  const bool evicting = Lp > budget;
  if (evicting) prefix = evict_threshold(s_val, s_pos, Lp, rthr, static_cast<unsigned>(Lp - budget), dh);
  const int seg = (Lp + kThreads - 1) / kThreads;
  const int a0 = min(Lp, static_cast<int>(threadIdx.x) * seg), a1 = min(Lp, a0 + seg);
  unsigned cnt = 0;
  for (int j = a0; j < a1; ++j)
    cnt += !(evicting && j < rthr && evict_key(s_val[j], j) <= prefix);
  unsigned total;
  unsigned slot = block_excl_scan<kThreads>(cnt, scratch, &total);
  for (int j = a0; j < a1; ++j)
    if (!(evicting && j < rthr && evict_key(s_val[j], j) <= prefix)) s_map[slot++] = j;
  __syncthreads();
  const int n = static_cast<int>(min(total, static_cast<unsigned>(cap)));
  const int64_t slot0 = static_cast<int64_t>(bh) * cap;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    pos_g[slot0 + i] = s_map[i];
    acc_g[slot0 + i] = s_val[s_map[i]];
  }
  constexpr int kPieces = RB / 16;
  const int64_t base = b * sb + h * sh;
  for (int i = threadIdx.x; i < n * kPieces; i += kThreads) {
    const int r = i / kPieces, c = i - r * kPieces;
    const int64_t src = base + static_cast<int64_t>(s_map[r]) * st + c * 16;
    const int64_t dst = (slot0 + r) * RB + c * 16;
    *reinterpret_cast<u32x4_t*>(kc + dst) = *reinterpret_cast<const u32x4_t*>(k + src);
    *reinterpret_cast<u32x4_t*>(vc + dst) = *reinterpret_cast<const u32x4_t*>(v + src);
  }
}

template <int D>
void launch_prefill_passes(const uint16_t* q, kvc_strides qs, const uint16_t* k, kvc_strides kvs, int H,
                           int64_t BH, int Lp, float scale_log2, float2* stat, float* colsum, hipStream_t stream) {
  const int nqt = (Lp + kPTile - 1) / kPTile;
  const int nb = (nqt + kWaves - 1) / kWaves;
  const unsigned g = static_cast<unsigned>(BH * nb);
  h2o_prefill_stats_bf16<D><<<g, kThreads, 0, stream>>>(q, qs.b, qs.h, qs.t, k, kvs.b, kvs.h, kvs.t, H, Lp, nb,
                                                       scale_log2, stat);
  h2o_prefill_colsum_bf16<D><<<g, kThreads, 0, stream>>>(q, qs.b, qs.h, qs.t, k, kvs.b, kvs.h, kvs.t, H, Lp, nb,
                                                        scale_log2, stat, colsum);
}

template <int D>
void launch_prefill_passes(const float* q, kvc_strides qs, const float* k, kvc_strides kvs, int H, int64_t BH,
                           int Lp, float scale_log2, float2* stat, float* colsum, hipStream_t stream) {
  const dim3 g((Lp + kThreads - 1) / kThreads, static_cast<unsigned>(BH));
  h2o_prefill_stats_f32<D><<<g, kThreads, 0, stream>>>(q, qs.b, qs.h, qs.t, k, kvs.b, kvs.h, kvs.t, H, Lp,
                                                      scale_log2, stat);
  h2o_prefill_colsum_f32<D><<<g, kThreads, 0, stream>>>(q, qs.b, qs.h, qs.t, k, kvs.b, kvs.h, kvs.t, H, Lp,
                                                       scale_log2, stat, colsum);
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" kvc_status kvc_h2o_step(kvc_h2o_cache* c, const void* q, const void* k_new, const void* v_new,
                                   int n_heavy, int n_recent, float* attn_out, hipStream_t stream) {
  clear_error();
  if (!c) return fail(KVC_ERR_INVALID_ARG, "h2o: cache is NULL");
  if (!c->k || !c->v || !c->pos || !c->acc || !q || !k_new || !v_new)
    return fail(KVC_ERR_INVALID_ARG, "h2o: cache arrays, q, k_new and v_new must be non-NULL");
  if (c->dt != KVC_BF16 && c->dt != KVC_F32) return fail(KVC_ERR_INVALID_ARG, "h2o: unknown dtype");
  if (c->B <= 0 || c->H <= 0 || c->cap <= 0) return fail(KVC_ERR_INVALID_ARG, "h2o: B, H, cap must be positive");
  if (c->D != 64 && c->D != 128) return fail(KVC_ERR_UNSUPPORTED, "h2o: head_dim %d not in {64, 128}", c->D);
  if (c->cap > kMaxCap) return fail(KVC_ERR_UNSUPPORTED, "h2o: cap %d > %d", c->cap, kMaxCap);
  if (c->n < 0 || c->n + 1 > c->cap) return fail(KVC_ERR_INVALID_ARG, "h2o: n+1 (%d) exceeds cap %d", c->n + 1, c->cap);
  if (c->len < c->n || c->len >= INT32_MAX) return fail(KVC_ERR_INVALID_ARG, "h2o: len out of range");
  if (n_heavy < 0 || n_recent < 0) return fail(KVC_ERR_INVALID_ARG, "h2o: n_heavy and n_recent must be >= 0");
  if (static_cast<int64_t>(c->B) * c->H > INT32_MAX) return fail(KVC_ERR_UNSUPPORTED, "h2o: too many heads");
  if (!aligned16(c->k) || !aligned16(c->v) || !aligned16(q) || !aligned16(k_new) || !aligned16(v_new))
    return fail(KVC_ERR_INVALID_ARG, "h2o: K/V and q/k/v pointers must be 16-byte aligned");
  kvc_status st;
  if (c->dt == KVC_BF16)
    st = c->D == 128 ? launch_h2o<uint16_t, 128>(c, q, k_new, v_new, n_heavy, n_recent, attn_out, stream)
                     : launch_h2o<uint16_t, 64>(c, q, k_new, v_new, n_heavy, n_recent, attn_out, stream);
  else
    st = c->D == 128 ? launch_h2o<float, 128>(c, q, k_new, v_new, n_heavy, n_recent, attn_out, stream)
                     : launch_h2o<float, 64>(c, q, k_new, v_new, n_heavy, n_recent, attn_out, stream);
  if (st != KVC_OK) return st;
  const int budget = n_heavy + n_recent;
  c->n = c->n + 1 > budget ? budget : c->n + 1;
  c->len += 1;
  return KVC_OK;
}

extern "C" size_t kvc_h2o_prefill_workspace_bytes(int B, int H, int prompt_len) {
  if (B <= 0 || H <= 0 || prompt_len <= 0) return 0;
  return align_up(static_cast<size_t>(B) * H * prompt_len * 8, 256) +
         align_up(static_cast<size_t>(B) * H * prompt_len * 4, 256);
}

extern "C" kvc_status kvc_h2o_prefill(kvc_h2o_cache* c, const void* q, kvc_strides qs, const void* k,
                                      const void* v, kvc_strides kvs, int prompt_len, int n_heavy, int n_recent,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  if (!c) return fail(KVC_ERR_INVALID_ARG, "h2o prefill: cache is NULL");
  if (!c->k || !c->v || !c->pos || !c->acc || !q || !k || !v)
    return fail(KVC_ERR_INVALID_ARG, "h2o prefill: cache arrays, q, k and v must be non-NULL");
  if (c->dt != KVC_BF16 && c->dt != KVC_F32) return fail(KVC_ERR_INVALID_ARG, "h2o prefill: unknown dtype");
  if (c->B <= 0 || c->H <= 0 || c->cap <= 0) return fail(KVC_ERR_INVALID_ARG, "h2o prefill: B, H, cap must be positive");
  if (c->D != 64 && c->D != 128) return fail(KVC_ERR_UNSUPPORTED, "h2o prefill: head_dim %d not in {64, 128}", c->D);
  if (static_cast<int64_t>(c->B) * c->H > 65535) return fail(KVC_ERR_UNSUPPORTED, "h2o prefill: B*H must be <= 65535");
  if (prompt_len < 1) return fail(KVC_ERR_INVALID_ARG, "h2o prefill: prompt_len must be >= 1");
  if (prompt_len > kMaxCap) return fail(KVC_ERR_UNSUPPORTED, "h2o prefill: prompt_len %d > %d", prompt_len, kMaxCap);
  if (n_heavy < 0 || n_recent < 0) return fail(KVC_ERR_INVALID_ARG, "h2o prefill: n_heavy and n_recent must be >= 0");
  const int64_t budget = static_cast<int64_t>(n_heavy) + n_recent;
  const int keep = static_cast<int>(prompt_len < budget ? prompt_len : budget);
  if (keep > c->cap) return fail(KVC_ERR_INVALID_ARG, "h2o prefill: %d kept tokens exceed cap %d", keep, c->cap);
  const int64_t es = c->dt == KVC_BF16 ? 2 : 4;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(c->k) || !aligned16(c->v))
    return fail(KVC_ERR_INVALID_ARG, "h2o prefill: K/V and q/k/v pointers must be 16-byte aligned");
  const int64_t strides[6] = {qs.b, qs.h, qs.t, kvs.b, kvs.h, kvs.t};
  for (int64_t s : strides)
    if (s < 0 || (s * es) % 16 != 0)
      return fail(KVC_ERR_INVALID_ARG, "h2o prefill: strides must be non-negative and multiples of 16 bytes");
  if (qs.t < c->D || kvs.t < c->D) return fail(KVC_ERR_INVALID_ARG, "h2o prefill: row strides must be >= head_dim");
  const size_t need = kvc_h2o_prefill_workspace_bytes(c->B, c->H, prompt_len);
  if (!workspace || workspace_bytes < need)
    return fail(KVC_ERR_WORKSPACE, "h2o prefill: workspace of %zu bytes needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  const int64_t BH = static_cast<int64_t>(c->B) * c->H;
  float2* stat = static_cast<float2*>(workspace);
  float* colsum = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           align_up(static_cast<size_t>(BH) * prompt_len * 8, 256));
  const float scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(c->D)));
  if (c->dt == KVC_BF16) {
    if (c->D == 128)
      launch_prefill_passes<128>(static_cast<const uint16_t*>(q), qs, static_cast<const uint16_t*>(k), kvs, c->H, BH,
                                 prompt_len, scale_log2, stat, colsum, stream);
    else
      launch_prefill_passes<64>(static_cast<const uint16_t*>(q), qs, static_cast<const uint16_t*>(k), kvs, c->H, BH,
                                prompt_len, scale_log2, stat, colsum, stream);
  } else {
    if (c->D == 128)
      launch_prefill_passes<128>(static_cast<const float*>(q), qs, static_cast<const float*>(k), kvs, c->H, BH,
                                 prompt_len, scale_log2, stat, colsum, stream);
    else
      launch_prefill_passes<64>(static_cast<const float*>(q), qs, static_cast<const float*>(k), kvs, c->H, BH,
                                prompt_len, scale_log2, stat, colsum, stream);
  }
  const size_t smem = static_cast<size_t>(prompt_len) * 12;
  const int rb = static_cast<int>(c->D * es);
  const unsigned grid = static_cast<unsigned>(BH);
  const char* kb = static_cast<const char*>(k);
  const char* vb = static_cast<const char*>(v);
  char* kc = static_cast<char*>(c->k);
  char* vc = static_cast<char*>(c->v);
  if (rb == 128)
    h2o_prefill_evict<128><<<grid, kThreads, smem, stream>>>(kb, vb, kvs.b * es, kvs.h * es, kvs.t * es, c->H,
                                                            prompt_len, n_heavy, n_recent, colsum, kc, vc, c->pos,
                                                            c->acc, c->cap);
  else if (rb == 256)
    h2o_prefill_evict<256><<<grid, kThreads, smem, stream>>>(kb, vb, kvs.b * es, kvs.h * es, kvs.t * es, c->H,
                                                            prompt_len, n_heavy, n_recent, colsum, kc, vc, c->pos,
                                                            c->acc, c->cap);
  else
    h2o_prefill_evict<512><<<grid, kThreads, smem, stream>>>(kb, vb, kvs.b * es, kvs.h * es, kvs.t * es, c->H,
                                                            prompt_len, n_heavy, n_recent, colsum, kc, vc, c->pos,
                                                            c->acc, c->cap);
  const kvc_status st = check_launch("h2o prefill");
  if (st != KVC_OK) return st;
  c->n = keep;
  c->len = prompt_len;
  return KVC_OK;
}
