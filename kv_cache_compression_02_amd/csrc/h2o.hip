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

template <typename T>
struct Vec16;  // a 16-byte piece of a row as float lanes
template <>
struct Vec16<uint16_t> {
  static constexpr int kN = 8;
  __device__ static void load(const void* p, float (&x)[8]) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct Vec16<float> {
  static constexpr int kN = 4;
  __device__ static void load(const void* p, float (&x)[4]) {
    const f32x4_t u = *reinterpret_cast<const f32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = u[i];
  }
};

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

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void h2o_step_kernel(
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
  __shared__ unsigned s_digit, s_below;

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

  // Scores of all N slots; the new token's key is read from k_new.
  float lmax = -INFINITY;
  for (int j0 = wave * RPW; j0 < N; j0 += kWaves * RPW) {
    const int j = j0 + grp;
    float dot = 0.f;
    if (j < N) {
      float kx[VE];
      Vec16<T>::load((j < n ? kb + static_cast<int64_t>(j) * RB : knr) + sub * 16, kx);
#pragma unroll
      for (int e = 0; e < VE; ++e) dot += qv[e] * kx[e];
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
    if (j < N && sub == 0) {
      const float s2 = dot * scale_log2;
      s_val[j] = s2;
      lmax = fmaxf(lmax, s2);
    }
  }
  for (int j = threadIdx.x; j < N; j += kThreads) s_pos[j] = j < n ? pos_g[slot0 + j] : new_pos;
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
    for (int j0 = wave * RPW; j0 < N; j0 += kWaves * RPW) {
      const int j = j0 + grp;
      if (j < N) {
        const float p = fast_exp2(s_val[j] - m2) * inv;
        float vx[VE];
        Vec16<T>::load((j < n ? vb + static_cast<int64_t>(j) * RB : vnr) + sub * 16, vx);
#pragma unroll
        for (int e = 0; e < VE; ++e) ov[e] += p * vx[e];
      }
    }
#pragma unroll
    for (int o = LPR; o < kWave; o <<= 1)
#pragma unroll
      for (int e = 0; e < VE; ++e) ov[e] += __shfl_xor(ov[e], o);
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
    s_val[j] = (j < n ? acc_g[slot0 + j] : 0.f) + p;
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
    unsigned rem = static_cast<unsigned>(E);
    unsigned long long prefix = 0, pmask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      dh[threadIdx.x] = 0;  // kThreads == 256 digits
      __syncthreads();
      for (int j = threadIdx.x; j < N; j += kThreads) {
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
