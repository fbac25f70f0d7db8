// Decode-time attention over a compacted or windowed KV cache (gfx950).
//
// After SnapKV compression every later generation step attends over the
// compressed cache only (SnapKV page, 技術の仕組み, processing flow step 4), and
// a StreamingLLM step attends over the sink and recent tokens only
// (StreamingLLM page, 推論の流れ). Both are one query per head against the n
// cached rows: o = sum_j softmax_j(q.k_j / sqrt(D)) v_j. No positional
// re-encoding happens inside the cache, so the rows may sit in any order (a
// ring, a compacted prefix + window, an H2O slot list).
//
// A single query against n rows is a GEMV: every K and V byte is used once,
// so the kernel is bound by HBM, not by MFMA. Split-K: a workgroup takes a
// chunk of kChunk rows of one head (kChunkSmall when a short cache of few
// heads would otherwise leave the chip underfilled); a wave takes a quarter of
// them with one 16-byte piece of a row per lane (LPR lanes per row, RPW rows per load),
// keeps its rows' scores in registers, then forms exp2(s - m) and the
// weighted V sum. Chunks write (m, l, o[D]) partials that a second kernel
// merges by log-sum-exp; a head of a single chunk writes its output directly.
#include <math.h>

#include <mutex>

#include "common.hpp"

namespace kvc {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kChunk = 256;       // rows per workgroup
constexpr int kChunkSmall = 128;  // rows per workgroup when kChunk would leave the chip underfilled
constexpr int kFillGroups = 512;  // workgroups below which the small chunk is used

// A 16-byte piece as float lanes (bf16: 8 widened by a shift; fp32: 4).
__device__ __forceinline__ void widen16(const u32x4_t& u, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(u[i] << 16);
    x[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void widen16(const u32x4_t& u, float (&x)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(u[i]);
}

template <typename T, int D, int CH>
__global__ __launch_bounds__(kDecThreads) void decode_partial(const T* __restrict__ q, int64_t qsb, int64_t qsh,
                                                               const T* __restrict__ k, const T* __restrict__ v,
                                                               int64_t ksb, int64_t ksh, int64_t kst, int H, int n,
                                                               int nchunk, float scale_log2, float* __restrict__ part,
                                                               float* __restrict__ out) {
  constexpr int VE = Vec16<T>::kN;           // elements per 16-byte piece
  constexpr int LPR = D / VE;                // lanes per row
  constexpr int RPW = kWave / LPR;           // rows per wave load
  constexpr int RW = CH / kDecWaves;         // rows per wave
  constexpr int S = RW / RPW;                // loads per wave
  __shared__ float s_m[kDecWaves], s_l[kDecWaves];
  __shared__ float s_o[kDecWaves][D];

  const int chunk = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh - b * H;
  const int wave = threadIdx.x / kWave, lane = lane_id(), slot = lane / LPR, pc = lane % LPR;
  const int row0 = chunk * CH + wave * RW + slot;
  const T* kb = k + b * ksb + h * ksh + pc * VE;
  const T* vb = v + b * ksb + h * ksh + pc * VE;
  float qv[VE];
  Vec16<T>::load(q + b * qsb + h * qsh + pc * VE, qv);

  // every K and V piece of the wave's rows is requested before any is used:
  // the chunk then costs one memory round trip, not one per load group
  u32x4_t kr[S], vr[S];
#pragma unroll
  for (int st = 0; st < S; ++st)
    kr[st] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t*>(kb + static_cast<int64_t>(min(row0 + st * RPW, n - 1)) * kst));
#pragma unroll
  for (int st = 0; st < S; ++st)
    vr[st] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t*>(vb + static_cast<int64_t>(min(row0 + st * RPW, n - 1)) * kst));
  __builtin_amdgcn_sched_barrier(0);  // (the scheduler would otherwise sink the loads to their uses)
  float sc[S];
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int row = row0 + st * RPW;
    float kv[VE];
    widen16(kr[st], kv);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) d = fmaf(qv[e], kv[e], d);
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) d += lane_xor_n(d, o);  // the row's lanes are adjacent
    sc[st] = row < n ? d * scale_log2 : -INFINITY;
  }
  float m = -INFINITY;
#pragma unroll
  for (int st = 0; st < S; ++st) m = fmaxf(m, sc[st]);
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) m = fmaxf(m, lane_xor_n(m, o));

  float l = 0.f, ov[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) ov[e] = 0.f;
#pragma unroll
  for (int st = 0; st < S; ++st) {
    const int row = row0 + st * RPW;
    float vv[VE];
    widen16(vr[st], vv);
    const float p = row < n ? fast_exp2(sc[st] - m) : 0.f;
    l += p;
#pragma unroll
    for (int e = 0; e < VE; ++e) ov[e] = fmaf(p, vv[e], ov[e]);
  }
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) {
    l += lane_xor_n(l, o);
#pragma unroll
    for (int e = 0; e < VE; ++e) ov[e] += lane_xor_n(ov[e], o);
  }
  if (lane == 0) {
    s_m[wave] = m;
    s_l[wave] = l;
  }
  if (slot == 0) {
#pragma unroll
    for (int e = 0; e < VE; ++e) s_o[wave][pc * VE + e] = ov[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int t = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, s_m[w]);  // finite: every chunk holds a row
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = s_l[w] > 0.f ? fast_exp2(s_m[w] - M) : 0.f;  // a wave past row n adds nothing
      L = fmaf(s_l[w], f, L);
      O = fmaf(s_o[w][t], f, O);
    }
    if (nchunk == 1) {
      out[static_cast<int64_t>(bh) * D + t] = O / L;
    } else {
      float* pp = part + (static_cast<int64_t>(bh) * nchunk + chunk) * (D + 2);
      pp[t] = O;
      if (t == 0) {
        pp[D] = M;
        pp[D + 1] = L;
      }
    }
  }
}

// Log-sum-exp merge of a head's chunk partials: one thread per output element.
template <int D>
__global__ __launch_bounds__(D) void decode_merge(const float* __restrict__ part, int nchunk, float* __restrict__ out) {
  const int bh = blockIdx.x, t = threadIdx.x;
  const float* pb = part + static_cast<int64_t>(bh) * nchunk * (D + 2);
  float M = -INFINITY;
  for (int c = 0; c < nchunk; ++c) M = fmaxf(M, pb[c * (D + 2) + D]);
  float L = 0.f, O = 0.f;
  for (int c = 0; c < nchunk; ++c) {
    const float f = fast_exp2(pb[c * (D + 2) + D] - M);
    L = fmaf(pb[c * (D + 2) + D + 1], f, L);
    O = fmaf(pb[c * (D + 2) + t], f, O);
  }
  out[static_cast<int64_t>(bh) * D + t] = O / L;
}

// Rows per workgroup for these sizes: kChunk, or kChunkSmall when that would
// leave fewer than kFillGroups workgroups (a short cache of few heads).
int decode_chunk(int B, int H, int n) {
  const int64_t groups = static_cast<int64_t>(B) * H * ((n + kChunk - 1) / kChunk);
  return groups < kFillGroups ? kChunkSmall : kChunk;
}

template <typename T, int D, int CH>
void launch_decode_ch(const void* q, kvc_strides qs, const void* k, const void* v, kvc_strides kvs, int B, int H,
                      int n, float* out, float* part, hipStream_t stream) {
  const int nchunk = (n + CH - 1) / CH;
  const float scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(D)));
  const dim3 g(nchunk, B * H);
  decode_partial<T, D, CH><<<g, kDecThreads, 0, stream>>>(static_cast<const T*>(q), qs.b, qs.h,
                                                          static_cast<const T*>(k), static_cast<const T*>(v), kvs.b,
                                                          kvs.h, kvs.t, H, n, nchunk, scale_log2, part, out);
  if (nchunk > 1) decode_merge<D><<<B * H, D, 0, stream>>>(part, nchunk, out);
}

template <typename T, int D>
void launch_decode(const void* q, kvc_strides qs, const void* k, const void* v, kvc_strides kvs, int B, int H, int n,
                   float* out, float* part, hipStream_t stream) {
  if (decode_chunk(B, H, n) == kChunk)
    launch_decode_ch<T, D, kChunk>(q, qs, k, v, kvs, B, H, n, out, part, stream);
  else
    launch_decode_ch<T, D, kChunkSmall>(q, qs, k, v, kvs, B, H, n, out, part, stream);
}

// The allocation-free variant's partials: a file-scope array in device memory
// (each GPU the library runs on holds its own copy until the process ends).
// In host code `scratch` names a host-side stand-in, not a device address:
// kernels get the per-device address from scratch_ptr() instead.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on the current device, looked up once per
// device with that device current; NULL (and *err set) if the lookup fails.
float* scratch_ptr(hipError_t* err) {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return static_cast<float*>(ptrs[dev]);
}

// Validation shared by both entry points; on success *split says whether the
// rows are split over several workgroups per head (partials then merged).
kvc_status decode_check(const void* q, kvc_strides qs, const void* k, const void* v, kvc_strides kvs, int B, int H,
                        int n, int D, kvc_dtype dt, float* out, bool* split) {
  if (!q || !k || !v || !out) return fail(KVC_ERR_INVALID_ARG, "decode_attention: q, k, v and out must be non-NULL");
  if (dt != KVC_BF16 && dt != KVC_F32) return fail(KVC_ERR_INVALID_ARG, "decode_attention: unknown dtype %d", (int)dt);
  if (B <= 0 || H <= 0 || n <= 0) return fail(KVC_ERR_INVALID_ARG, "decode_attention: B, H and n must be positive");
  if (static_cast<int64_t>(B) * H > 65535) return fail(KVC_ERR_UNSUPPORTED, "decode_attention: B*H must be <= 65535");
  if (D != 64 && D != 128) return fail(KVC_ERR_UNSUPPORTED, "decode_attention: head_dim %d not in {64, 128}", D);
  const int64_t es = dt == KVC_BF16 ? 2 : 4;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(KVC_ERR_INVALID_ARG, "decode_attention: device pointers must be 16-byte aligned");
  const int64_t strides[5] = {qs.b, qs.h, kvs.b, kvs.h, kvs.t};
  for (int64_t s : strides)
    if (s < 0 || (s * es) % 16 != 0)
      return fail(KVC_ERR_INVALID_ARG, "decode_attention: strides must be non-negative and multiples of 16 bytes");
  if (kvs.t < D) return fail(KVC_ERR_INVALID_ARG, "decode_attention: row stride must be >= head_dim");
  *split = n > decode_chunk(B, H, n);
  return KVC_OK;
}

void launch_decode_any(const void* q, kvc_strides qs, const void* k, const void* v, kvc_strides kvs, int B, int H,
                       int n, int D, kvc_dtype dt, float* out, float* part, hipStream_t stream) {
  if (dt == KVC_BF16) {
    if (D == 128)
      launch_decode<uint16_t, 128>(q, qs, k, v, kvs, B, H, n, out, part, stream);
    else
      launch_decode<uint16_t, 64>(q, qs, k, v, kvs, B, H, n, out, part, stream);
  } else {
    if (D == 128)
      launch_decode<float, 128>(q, qs, k, v, kvs, B, H, n, out, part, stream);
    else
      launch_decode<float, 64>(q, qs, k, v, kvs, B, H, n, out, part, stream);
  }
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" size_t kvc_decode_attention_workspace_bytes(int B, int H, int n, int D) {
  if (B <= 0 || H <= 0 || n <= 0 || (D != 64 && D != 128)) return 0;
  const int ch = decode_chunk(B, H, n);
  const int64_t nchunk = (n + ch - 1) / ch;
  return nchunk > 1 ? static_cast<size_t>(B) * H * nchunk * (D + 2) * sizeof(float) : 16;
}

extern "C" kvc_status kvc_decode_attention(const void* q, kvc_strides qs, const void* k, const void* v,
                                           kvc_strides kvs, int B, int H, int n, int D, kvc_dtype dt, float* out,
                                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  bool split = false;
  const kvc_status st = decode_check(q, qs, k, v, kvs, B, H, n, D, dt, out, &split);
  if (st != KVC_OK) return st;
  const size_t need = kvc_decode_attention_workspace_bytes(B, H, n, D);
  if (split && (!workspace || workspace_bytes < need))
    return fail(KVC_ERR_WORKSPACE, "decode_attention: workspace of %zu bytes needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (split && !aligned16(workspace))
    return fail(KVC_ERR_INVALID_ARG, "decode_attention: workspace must be 16-byte aligned");
  launch_decode_any(q, qs, k, v, kvs, B, H, n, D, dt, out, static_cast<float*>(workspace), stream);
  return check_launch("decode_attention");
}

extern "C" kvc_status kvc_decode_attention_noalloc(const void* q, kvc_strides qs, const void* k, const void* v,
                                                   kvc_strides kvs, int B, int H, int n, int D, kvc_dtype dt,
                                                   float* out, hipStream_t stream) {
  clear_error();
  bool split = false;
  const kvc_status st = decode_check(q, qs, k, v, kvs, B, H, n, D, dt, out, &split);
  if (st != KVC_OK) return st;
  float* part = nullptr;
  if (split) {
    const size_t need = kvc_decode_attention_workspace_bytes(B, H, n, D);
    if (need > kScratchBytes)
      return fail(KVC_ERR_WORKSPACE,
                  "decode_attention_noalloc: these sizes need %zu bytes of partials, beyond the %zu-byte static "
                  "scratch; use kvc_decode_attention with a workspace",
                  need, kScratchBytes);
    hipError_t e = hipSuccess;
    part = scratch_ptr(&e);
    if (!part) return fail(KVC_ERR_HIP, "decode_attention_noalloc: scratch address: %s", hipGetErrorString(e));
  }
  launch_decode_any(q, qs, k, v, kvs, B, H, n, D, dt, out, part, stream);
  return check_launch("decode_attention_noalloc");
}
