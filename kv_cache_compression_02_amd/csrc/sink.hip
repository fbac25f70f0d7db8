// StreamingLLM sink + recent ring update on gfx950.
//
// The method (abeam.tech summary of "Efficient Streaming Language Models with
// Attention Sinks", section 技術の仕組み, subsections キャッシュ構造 and 推論の流れ):
// the first few tokens stay in the cache for good; every later token enters a
// fixed-length recent window whose oldest member leaves once it is full.
//
// Layout: sink slots 0 .. s-1, then a ring of r slots; position p >= s lives in
// slot s + (p - s) mod r, so a new token overwrites exactly the token that
// leaves the window and nothing else moves.
#include "common.hpp"

namespace kvc {
namespace {

constexpr int kThreads = 256;

// One launch per token: thread t copies 16-byte piece t of the heads' new K
// and V rows into the token's slot (t < n_pieces), writes entry t of the
// ascending list of held positions (t < n_kept, when asked for), and thread 0
// records the slot's new position.
__global__ __launch_bounds__(kThreads) void sink_update(char* __restrict__ rk, char* __restrict__ rv,
                                                        const char* __restrict__ kn, const char* __restrict__ vn,
                                                        int64_t n_pieces, int pieces_per_row, int n_slots, int slot,
                                                        int* __restrict__ slot_pos, int pos,
                                                        int* __restrict__ kept, int n_sinks_held, int n_kept,
                                                        int recent_from) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (t < n_pieces) {
    const int64_t bh = t / pieces_per_row;
    const int c = static_cast<int>(t - bh * pieces_per_row);
    const int64_t row_bytes = static_cast<int64_t>(pieces_per_row) * 16;
    const int64_t dst = (bh * n_slots + slot) * row_bytes + c * 16;
    const int64_t src = bh * row_bytes + c * 16;
    *reinterpret_cast<u32x4_t*>(rk + dst) = *reinterpret_cast<const u32x4_t*>(kn + src);
    *reinterpret_cast<u32x4_t*>(rv + dst) = *reinterpret_cast<const u32x4_t*>(vn + src);
  }
  if (kept && t < n_kept) {
    const int i = static_cast<int>(t);
    kept[i] = i < n_sinks_held ? i : recent_from + (i - n_sinks_held);
  }
  if (t == 0) slot_pos[slot] = pos;
}

// Position inside the cache of each slot's token (its rank among the held
// tokens: sinks first, then the recent window oldest to newest), one slot per
// thread; -1 for a slot that holds no token yet.
__global__ __launch_bounds__(kThreads) void sink_positions(const int* __restrict__ slot_pos, int n_slots, int n_sink,
                                                           int n_sinks_held, int recent_from,
                                                           int* __restrict__ cache_pos) {
  const int t = static_cast<int>(blockIdx.x) * kThreads + static_cast<int>(threadIdx.x);
  if (t >= n_slots) return;
  const int p = slot_pos[t];
  cache_pos[t] = p < 0 ? -1 : p < n_sink ? p : n_sinks_held + (p - recent_from);
}

}  // namespace
}  // namespace kvc

using namespace kvc;

extern "C" kvc_status kvc_sink_cache_positions(const int32_t* slot_pos, int64_t len, int n_sink, int n_recent,
                                               int32_t* cache_pos_out, hipStream_t stream) {
  clear_error();
  if (!slot_pos || !cache_pos_out) return fail(KVC_ERR_INVALID_ARG, "sink positions: NULL pointer");
  if (len < 1 || len > INT32_MAX) return fail(KVC_ERR_INVALID_ARG, "sink positions: len must be in [1, 2^31-1]");
  if (n_sink < 0 || n_recent < 1 || static_cast<int64_t>(n_sink) + n_recent > INT32_MAX)
    return fail(KVC_ERR_INVALID_ARG, "sink positions: need n_sink >= 0 and n_recent >= 1");
  const int n_slots = n_sink + n_recent;
  const int64_t held_sinks = len < n_sink ? len : n_sink;
  const int64_t recent_from = len - n_recent > n_sink ? len - n_recent : n_sink;
  sink_positions<<<static_cast<unsigned>((n_slots + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
      slot_pos, n_slots, n_sink, static_cast<int>(held_sinks), static_cast<int>(recent_from), cache_pos_out);
  return check_launch("sink_cache_positions");
}

extern "C" kvc_status kvc_sink_recent(void* ring_k, void* ring_v, int32_t* slot_pos, const void* k_new,
                                      const void* v_new, int64_t len, int n_sink, int n_recent, int B, int H,
                                      int D, kvc_dtype dt, int32_t* kept_idx_out, hipStream_t stream) {
  clear_error();
  if (!ring_k || !ring_v || !slot_pos || !k_new || !v_new)
    return fail(KVC_ERR_INVALID_ARG, "sink: ring_k, ring_v, slot_pos, k_new, v_new must be non-NULL");
  if (dt != KVC_BF16 && dt != KVC_F32) return fail(KVC_ERR_INVALID_ARG, "sink: unknown dtype");
  if (B <= 0 || H <= 0) return fail(KVC_ERR_INVALID_ARG, "sink: B and H must be positive");
  if (D != 64 && D != 128) return fail(KVC_ERR_UNSUPPORTED, "sink: head_dim %d not in {64, 128}", D);
  if (len < 1 || len > INT32_MAX) return fail(KVC_ERR_INVALID_ARG, "sink: len must be in [1, 2^31-1]");
  if (n_sink < 0 || n_recent < 1 || static_cast<int64_t>(n_sink) + n_recent > INT32_MAX)
    return fail(KVC_ERR_INVALID_ARG, "sink: need n_sink >= 0 and n_recent >= 1");
  if (!aligned16(ring_k) || !aligned16(ring_v) || !aligned16(k_new) || !aligned16(v_new))
    return fail(KVC_ERR_INVALID_ARG, "sink: K/V pointers must be 16-byte aligned");
  const int64_t pos = len - 1;
  const int slot = pos < n_sink ? static_cast<int>(pos)
                                : n_sink + static_cast<int>((pos - n_sink) % n_recent);
  const int n_slots = n_sink + n_recent;
  const int es = dt == KVC_BF16 ? 2 : 4;
  const int ppr = D * es / 16;
  const int64_t pieces = static_cast<int64_t>(B) * H * ppr;
  const int64_t held_sinks = len < n_sink ? len : n_sink;
  const int64_t n_kept = len < n_slots ? len : n_slots;
  const int64_t recent_from = len - n_recent > n_sink ? len - n_recent : n_sink;
  const int64_t threads = pieces > n_kept ? pieces : n_kept;
  sink_update<<<static_cast<unsigned>((threads + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
      static_cast<char*>(ring_k), static_cast<char*>(ring_v), static_cast<const char*>(k_new),
      static_cast<const char*>(v_new), pieces, ppr, n_slots, slot, slot_pos, static_cast<int>(pos), kept_idx_out,
      static_cast<int>(held_sinks), static_cast<int>(n_kept), static_cast<int>(recent_from));
  return check_launch("sink_recent");
}
