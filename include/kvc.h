/*
 * kvc — attention-score-guided KV-cache token selection and compaction on
 * AMD Instinct MI355X (gfx950).
 *
 * Three policies share one library:
 *   - SnapKV prompt compression: the abeam.tech summary of "SnapKV: LLM Knows
 *     What You are Looking for Before Generation", section 技術の仕組み (how it
 *     works), subsection 処理の流れ (processing flow), steps 1-4.
 *   - H2O heavy-hitter + recent eviction during decoding: the abeam.tech summary
 *     of "H2O: Heavy-Hitter Oracle for Efficient Generative Inference of Large
 *     Language Models", section 技術の仕組み, subsections 何を残すのか (what is
 *     kept) and 処理の流れ (processing flow).
 *   - StreamingLLM attention sinks + recent window: the abeam.tech summary of
 *     "Efficient Streaming Language Models with Attention Sinks", section
 *     技術の仕組み, subsections キャッシュ構造 (cache structure) and 推論の流れ
 *     (inference flow).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers; the caller owns every buffer,
 *     including workspaces (size them with the *_workspace_bytes queries). The
 *     library never allocates or frees device memory.
 *   - Work is enqueued on `stream` and runs asynchronously; no entry point
 *     synchronises the host. A device-side fault surfaces as a HIP error at the
 *     caller's next synchronisation.
 *   - Arguments are checked on the host before anything is enqueued. A bad
 *     argument returns a non-OK status, leaves every output untouched and sets
 *     a message readable with kvc_last_error(). No C++ exception crosses the ABI.
 *   - Element types: KVC_BF16 (bfloat16 stored as 16-bit patterns) or KVC_F32.
 *     Arithmetic is float32 with fp32 accumulation in every case.
 *   - head_dim D must be 64 or 128 and is the contiguous (innermost) axis.
 *     Device pointers and the byte size of every row stride must be multiples
 *     of 16.
 *   - Calls on one stream are ordered; concurrent calls that share a workspace
 *     or a cache race.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARG = 1, /* a pointer, size or policy value is out of range      */
  KVC_ERR_UNSUPPORTED = 2, /* valid, but outside what the kernels handle (D, w)     */
  KVC_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query     */
  KVC_ERR_HIP = 4          /* a kernel launch failed; message holds the HIP error  */
} kvc_status;

typedef enum { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

/* Element strides of a [B, H, T, D] tensor whose D axis is contiguous. */
typedef struct {
  int64_t b, h, t;
} kvc_strides;

/* Message describing the last non-OK status returned on the calling thread
 * ("" if none). The pointer stays valid until the next call on that thread. */
const char* kvc_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int kvc_version(void);

/* ------------------------------------------------------------------------- */
/* SnapKV prompt-KV compression (one attention layer, every head).            */
/* ------------------------------------------------------------------------- */

/* Bytes of device workspace kvc_snapkv_compress needs for these sizes
 * (0 if the sizes are invalid). */
size_t kvc_snapkv_workspace_bytes(int B, int H, int L, int D, int window, int budget,
                                  int pool_kernel, kvc_dtype dt);

/* Compress the prompt cache of one layer to `budget` rows per head.
 *
 * For every (b, h), independently (SnapKV page, processing flow):
 *   1. the last `window` prompt queries attend to the prompt keys with scores
 *      q.k / sqrt(D); query i of the window sits at position L-window+i and sees
 *      keys 0 .. L-window+i (causal inside the window); each row's softmax runs
 *      over every key it sees;
 *   2. vote[j] = sum over the window rows of their softmax weight on prefix
 *      position j, j < L-window;
 *   3. pooled = 1D max-pool of vote, odd width pool_kernel, stride 1, neighbours
 *      beyond either end ignored;
 *   4. the budget-window prefix positions with the largest pooled score are kept
 *      (equal scores: lower position first), in ascending order, and their K/V
 *      rows are concatenated with the window's own K/V rows.
 *
 * q        [B, H, q_len, D] queries with strides qs; rows q_len-window .. q_len-1
 *          are the observation window (the rest is not read).
 * k, v     [B, H, L, D] prompt keys and values, both with strides kvs.
 * k_out,   [B, H, budget, D] contiguous outputs: kept prefix rows in ascending
 * v_out    position order, then the window rows L-window .. L-1.
 * idx_out  [B, H, budget-window] int32 kept prefix positions, ascending.
 * pooled_out, vote_out  optional float [B, H, L-window] (NULL = not written).
 * workspace  device buffer of at least kvc_snapkv_workspace_bytes(...) bytes;
 *          its contents on entry do not matter.
 *
 * Requires 1 <= window <= 32, window < budget < L (when L <= budget there is
 * nothing to compress: INVALID_ARG), pool_kernel odd in [1, 65], q_len >= window,
 * D in {64, 128}. Outputs must not overlap the inputs. */
kvc_status kvc_snapkv_compress(const void* q, int q_len, kvc_strides qs,
                               const void* k, const void* v, kvc_strides kvs,
                               int B, int H, int L, int D, int window, int budget,
                               int pool_kernel, kvc_dtype dt,
                               void* k_out, void* v_out, int32_t* idx_out,
                               float* pooled_out, float* vote_out,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Pooling operators of the vote smoothing (SnapKV page, processing flow step
 * 3 says only "1D pooling"):
 *   KVC_POOL_MAX  max over the in-range neighbours j-p/2 .. j+p/2 (the default
 *                 of kvc_snapkv_compress);
 *   KVC_POOL_AVG  their mean: the sum of the in-range neighbours' votes,
 *                 divided by how many are in range (neighbours beyond either end
 *                 of the prefix are ignored, as for the max). */
typedef enum { KVC_POOL_MAX = 0, KVC_POOL_AVG = 1 } kvc_pool_type;

/* Workspace bytes kvc_snapkv_compress_ex needs for these sizes (0 if they are
 * invalid); `ragged` non-zero when a lengths array will be passed. */
size_t kvc_snapkv_workspace_bytes_ex(int n_layers, int B, int H, int L, int D, int window, int budget,
                                     int pool_kernel, kvc_dtype dt, int ragged);

/* kvc_snapkv_compress with three extensions for serving stacks (SnapKV page,
 * limits: per-head selection and gather-based KV reconstruction inside the
 * serving engine; processing flow step 3 for the pooling operator):
 *   - pool_type: KVC_POOL_MAX or KVC_POOL_AVG (see kvc_pool_type);
 *   - n_layers >= 1 layers of one prompt in one call: layer l's queries start
 *     q_layer_stride elements after layer l-1's, its keys and values
 *     kv_layer_stride elements after; each layer is compressed independently
 *     (the method is per layer and per head). Outputs are contiguous over
 *     [n_layers, B, H, ...]. When q_layer_stride == B * qs.b and
 *     kv_layer_stride == B * kvs.b (layers stacked in front of the batch axis)
 *     the layers run as one batch of n_layers * B sequences, which fills the
 *     device for short prompts; otherwise layer by layer;
 *   - lengths: optional HOST array [B] of prompt lengths (a ragged batch
 *     padded to L): sequence b uses keys and values 0 .. lengths[b]-1, its
 *     window is its last `window` positions lengths[b]-window .. lengths[b]-1,
 *     whose queries are q's rows q_len-window .. q_len-1 (the same rows for
 *     every sequence: each sequence's own window queries, aligned at the end
 *     of q); every length must satisfy budget < lengths[b] <= L. Each (layer,
 *     sequence) then runs as its own launch sequence. k_out / v_out / idx_out
 *     keep their fixed shapes; pooled_out and vote_out are packed: for each
 *     layer, then each sequence, H rows of lengths[b] - window values.
 *     NULL lengths: every sequence has length L (pooled / vote
 *     [n_layers, B, H, L - window]).
 * Everything else (arguments, rules, errors, asynchrony) is as in
 * kvc_snapkv_compress; the workspace is sized by kvc_snapkv_workspace_bytes_ex
 * and reused across the launch sequences in stream order. */
kvc_status kvc_snapkv_compress_ex(const void* q, int q_len, kvc_strides qs, int64_t q_layer_stride,
                                  const void* k, const void* v, kvc_strides kvs, int64_t kv_layer_stride,
                                  int n_layers, int B, int H, int L, int D, const int32_t* lengths,
                                  int window, int budget, int pool_kernel, int pool_type, kvc_dtype dt,
                                  void* k_out, void* v_out, int32_t* idx_out, float* pooled_out,
                                  float* vote_out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* Score schedules of kvc_snapkv_compress. Both compute every score in fp32
 * from the same bf16 / fp32 inputs and select by the same rule; they differ in
 * how often K is read and in how each window row's softmax normaliser is
 * formed (so votes may differ in the last bits).
 *   TWO_PASS     row statistics (max, sum) in one pass over K, votes in a
 *                second: K is read twice. Bitwise reproducible.
 *   SINGLE_PASS  bf16 only: one device-wide pass keeps each key tile's
 *                scores in registers until its head's normaliser is complete,
 *                so K is read once. Each row's normaliser is summed exactly in
 *                fixed point, so the result does not depend on the order of
 *                the contributions (bitwise reproducible as well). Two kernels
 *                implement it, and both need all their workgroups resident at
 *                once. snap_wave_bf16, whose waves work independently on
 *                32-key tiles, runs where every workgroup has tiles in every
 *                head and a head spans at most seven of its rounds (on MI355X:
 *                about 64K to 390K keys per head), or where heads are shorter
 *                than one of its rounds (2048 tiles) and the layer fills at
 *                least eight rounds (e.g. 64 heads of 16K keys); it is launched like any
 *                kernel and checks residency at its start: if its workgroups
 *                cannot all start within about a millisecond (other work
 *                holding the compute units), it flags every head and the
 *                pooling kernel computes their votes exactly instead (the
 *                same results, far slower). snap_coop_bf16, whose workgroups step through
 *                128-key units together, covers shorter heads (a head of at
 *                most four device-wide rounds of units) with a cooperative
 *                launch. Where neither can run, the call uses TWO_PASS.
 *   AUTO         the default: SINGLE_PASS where snap_wave_bf16 can run
 *                (there the faster schedule on MI355X), else TWO_PASS (which
 *                measures faster than snap_coop_bf16 on shorter heads); also
 *                TWO_PASS if the single-pass launch fails. */
typedef enum {
  KVC_SNAPKV_AUTO = 0,
  KVC_SNAPKV_TWO_PASS = 1,
  KVC_SNAPKV_SINGLE_PASS = 2
} kvc_snapkv_schedule;

/* Select the schedule for later kvc_snapkv_compress calls on the calling
 * thread. Returns the previous setting, or -1 (and changes nothing) for an
 * unknown value. */
int kvc_snapkv_set_schedule(int schedule);

/* The schedule (TWO_PASS or SINGLE_PASS) the last successful
 * kvc_snapkv_compress call on the calling thread ran, 0 if none. */
int kvc_snapkv_last_schedule(void);

/* Name of the kernel (or kernels, joined by '+') that computed the scores in
 * the last successful kvc_snapkv_compress call on the calling thread: a
 * static string, "" if none. For reports and tests; it does not change. */
const char* kvc_snapkv_last_score_kernel(void);

/* Testing (not part of the method): while `on` is non-zero, the calling
 * thread's single-pass calls run the independent-wave score kernel with a
 * residency check that cannot pass (it waits for one workgroup more than the
 * grid holds, 16 polls), so the kernel takes its fallback: it flags every head
 * and the pooling kernel computes all votes exactly, as when the kernel's
 * workgroups cannot all be resident at once. Returns the previous setting. */
int kvc_snapkv_force_residency_fallback(int on);

/* Testing (not part of the method): while `on` is non-zero, the calling
 * thread's single-pass calls run the independent-wave score kernel with a
 * limit of zero polls on its cross-worker waits (vote weights, merge slots,
 * a head's queries, a head's publication, the work owed after the last
 * round): every wait that
 * would have to wait gives up at once and records a failure code in the
 * status word, exactly as a wait whose normal limit (2^18 polls) runs out.
 * The split selection's wait for its head's histogram also gives up at once
 * (each workgroup then counts the whole head's pooled scores itself).
 * The kernel still exits normally. The pooling kernel reads the status word
 * and recomputes every head's votes exactly, so the results are the same as
 * without the knob (the votes may differ in the last bits). Returns the
 * previous setting. */
int kvc_snapkv_force_wait_timeout(int on);

/* Testing (not part of the method): byte offset, inside a workspace sized by
 * kvc_snapkv_workspace_bytes for the same arguments, of the single pass's
 * three 32-bit status words, or -1 if that layout has none (fp32, or
 * arguments it rejects). After a single-pass kvc_snapkv_compress call has
 * completed, word 0 is 0 when every bounded wait of the score kernel ended
 * in time, else the code of the wait that ran out (1 vote weights, 2 merge
 * slot, 3 a head's publication, 4 a head left unfinished, 5 a head's
 * queries), in which case every
 * head's votes were recomputed exactly; words 1 and 2 are the residency
 * gate's count and state (1: passed). Reading them is the caller's copy. */
int64_t kvc_snapkv_status_offset(int B, int H, int L, int D, int window, int budget, int pool_kernel,
                                 kvc_dtype dt);

/* Testing (not part of the method): while `on` is non-zero, the calling
 * thread's kvc_snapkv_compress calls run the top-k selection as several
 * workgroups per head that classify ranges of the head's positions and leave
 * the ranking and compaction to the head's last workgroup (the form used for
 * heads of more than 16384 prefix positions or rows that are not 16-byte
 * aligned), instead of one workgroup per head. With `on` = 2 the single pass
 * also launches its separate pooling kernel where the split selection would
 * otherwise pool and count the votes itself. The kept positions are the same
 * either way. Returns the previous setting (0, 1 or 2). */
int kvc_snapkv_force_split_select(int on);

/* Name of the selection kernel the last kvc_snapkv_compress call on the
 * calling thread launched ("snap_select_head" or "snap_select"): a static
 * string, "" if none. For reports and tests. */
const char* kvc_snapkv_last_select_kernel(void);

/* Name of the kernel that pooled the votes (max or average) and counted the
 * histogram of pooled scores in the last kvc_snapkv_compress call on the
 * calling thread:
 * "snap_votes_bf16" or "snap_votes_f32" (two passes: the vote pass pools),
 * "snap_pool" or "snap_pool_lds" (single pass: a pooling kernel after the
 * score kernel), "snap_select_head" or "snap_select" (single pass, max-pool
 * of radius at most 4: the selection kernel pools, counts and recomputes
 * flagged heads itself and no pooling kernel is launched; one workgroup per
 * head for heads of at most 16384 prefix positions, else the head's
 * workgroups together where the whole selection grid fits on the GPU at
 * once); a static string, "" if none. For reports and tests. */
const char* kvc_snapkv_last_pool_kernel(void);

/* Instrumentation (not part of the method): while set, every
 * kvc_snapkv_compress call on the calling thread records events[i] on its
 * stream at phase boundary i, for i < n_events (at most 7) and events[i] not
 * NULL (each recorded event costs a few microseconds of GPU time): 0 before the
 * first kernel, then after the workspace clear (1; the single pass's
 * preparation kernel under SINGLE_PASS), the row-statistics pass (2; the
 * single score kernel under SINGLE_PASS), the row-statistics merge (3; nothing
 * under SINGLE_PASS), the vote + pooling + histogram pass (4;
 * pooling + histogram under SINGLE_PASS, nothing where the selection pools),
 * the per-head selection (5) and the gather (6). When events 1 and 2 are both
 * set and the independent-wave score kernel runs, the kernel's own dispatch
 * records them at its start and end (no separate records around it), so that
 * their interval is the kernel's duration. The events are created and owned
 * by the caller; pass NULL or 0 to stop recording. */
void kvc_snapkv_set_phase_events(hipEvent_t* events, int n_events);

/* ------------------------------------------------------------------------- */
/* H2O heavy-hitter + recent cache, one decode step.                          */
/* ------------------------------------------------------------------------- */

/* Cache of one layer. Device arrays are caller-owned; n and len live on the
 * host and are advanced by the library (deterministically, no readback).
 * Every head holds the same number n of valid slots (0 .. n-1); slot order is
 * arbitrary (eviction moves the last slots into the freed ones). */
typedef struct {
  void* k;        /* [B, H, cap, D] cached keys, contiguous                  */
  void* v;        /* [B, H, cap, D] cached values, contiguous                */
  int32_t* pos;   /* [B, H, cap] absolute position of each cached token       */
  float* acc;     /* [B, H, cap] cumulative attention score of each token     */
  int B, H, D, cap;
  int n;          /* valid slots per head                                     */
  int64_t len;    /* tokens seen so far (positions 0 .. len-1)                */
  kvc_dtype dt;
} kvc_h2o_cache;

/* One decode step for every head (H2O page, processing flow and what is kept):
 *   - the new token (position len) is appended with score 0;
 *   - the new query attends, scores q.k / sqrt(D), softmax over all n+1 cached
 *     tokens; each token's probability is added to its score; if attn_out is
 *     not NULL, attn_out = sum_j p_j v_j (float32, [B, H, D], contiguous);
 *   - with length = len+1, tokens at positions >= length - n_recent are recent;
 *     when n+1 > n_heavy + n_recent, every recent token is kept and the rest
 *     of the budget n_heavy + n_recent goes to the other tokens with the
 *     largest score (equal scores: newer position kept).
 * On return c->len has grown by one and c->n = min(n+1, n_heavy + n_recent).
 * q, k_new, v_new: [B, H, D] contiguous, element type c->dt.
 * Requires n+1 <= cap, cap <= 8192, n_heavy >= 0, n_recent >= 0. */
kvc_status kvc_h2o_step(kvc_h2o_cache* c, const void* q, const void* k_new,
                        const void* v_new, int n_heavy, int n_recent,
                        float* attn_out, hipStream_t stream);

/* Bytes of device workspace kvc_h2o_prefill needs (0 if the sizes are invalid). */
size_t kvc_h2o_prefill_workspace_bytes(int B, int H, int prompt_len);

/* Initial H2O state after a prompt (H2O page: the glossary's local statistics,
 * i.e. the attention observed so far, and the what-is-kept subsection):
 *   - the score of prompt token j is the sum, over prompt queries i >= j, of the
 *     causal softmax weight of q_i on k_j (scores q.k / sqrt(D));
 *   - with length = prompt_len, the eviction rule of kvc_h2o_step keeps every
 *     recent token (position >= prompt_len - n_recent) and fills the rest of the
 *     budget n_heavy + n_recent with the highest-scoring other tokens;
 *   - the kept tokens are written to slots 0 .. n-1 in ascending position order
 *     (their K/V rows, positions and scores).
 * q [B, H, prompt_len, D] with strides qs; k, v [B, H, prompt_len, D] with
 * strides kvs (D contiguous), element type c->dt. The cache's previous contents
 * are replaced; on return c->n = min(prompt_len, n_heavy + n_recent) and
 * c->len = prompt_len. Requires prompt_len <= 8192, c->n <= cap after the
 * call, and a workspace of kvc_h2o_prefill_workspace_bytes(...) bytes. */
kvc_status kvc_h2o_prefill(kvc_h2o_cache* c, const void* q, kvc_strides qs, const void* k,
                           const void* v, kvc_strides kvs, int prompt_len, int n_heavy,
                           int n_recent, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* StreamingLLM sink + recent ring, one new token.                            */
/* ------------------------------------------------------------------------- */

/* Write the new token's key/value into the cache and report what it holds
 * (StreamingLLM page, cache structure and inference flow).
 *
 * The cache has n_sink sink slots followed by a ring of n_recent slots; the
 * token at position p lives in slot p if p < n_sink, else in slot
 * n_sink + (p - n_sink) mod n_recent. `len` counts tokens including the new
 * one, whose position is len-1.
 * ring_k, ring_v  [B, H, n_sink+n_recent, D] contiguous.
 * k_new, v_new    [B, H, D] contiguous.
 * slot_pos        [n_sink+n_recent] int32, shared by all heads: the position
 *                 now held by each slot is updated for the new token's slot.
 * kept_idx_out    optional [min(len, n_sink+n_recent)] int32: the held
 *                 positions, ascending (sinks 0 .. min(n_sink,len)-1, then
 *                 max(n_sink, len-n_recent) .. len-1).
 * Requires len >= 1, n_sink >= 0, n_recent >= 1. */
kvc_status kvc_sink_recent(void* ring_k, void* ring_v, int32_t* slot_pos,
                           const void* k_new, const void* v_new, int64_t len,
                           int n_sink, int n_recent, int B, int H, int D,
                           kvc_dtype dt, int32_t* kept_idx_out, hipStream_t stream);

/* Positions inside the cache (StreamingLLM page, cache structure and inference
 * flow; the page does not say which positions the model uses while streaming):
 * after `len` tokens, cache_pos_out[slot] is the rank of the token the slot
 * holds among the held tokens, sinks first (in arrival order), then the recent
 * window from oldest to newest, i.e. min(n_sink, len) + (p - max(n_sink,
 * len - n_recent)) for a recent token at position p and p for a sink; -1 for a
 * slot that holds no token yet. These stay below n_sink + n_recent however long
 * the stream runs, and the newest token takes the last one: the positions a
 * positional encoding would give the cached keys and the next query (which
 * takes min(len, n_sink + n_recent)). slot_pos: the [n_sink + n_recent] slot
 * map kept by kvc_sink_recent (read on the stream, after the calls before it);
 * cache_pos_out: [n_sink + n_recent] int32, device. Requires len >= 1,
 * n_sink >= 0, n_recent >= 1, and slot_pos as kvc_sink_recent leaves it after
 * `len` tokens. */
kvc_status kvc_sink_cache_positions(const int32_t* slot_pos, int64_t len, int n_sink, int n_recent,
                                    int32_t* cache_pos_out, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Decode attention over a compacted or windowed cache.                       */
/* ------------------------------------------------------------------------- */

/* Bytes of device workspace kvc_decode_attention needs (0 if the sizes are
 * invalid; a small non-zero size when no workspace is used). */
size_t kvc_decode_attention_workspace_bytes(int B, int H, int n, int D);

/* One query per head attends over the first n cached rows of that head:
 *   out[b,h,:] = sum_j softmax_j(q[b,h,:].k[b,h,j,:] / sqrt(D)) v[b,h,j,:],
 * j = 0 .. n-1. This is the generation step after compression: over the
 * compressed cache only (SnapKV page, processing flow step 4), or over the
 * sink and recent tokens only (StreamingLLM page, inference flow). The rows
 * may be in any order (no positional re-encoding inside the cache), so the
 * outputs of kvc_snapkv_compress (n = budget), a kvc_sink_recent ring
 * (n = min(len, n_sink + n_recent)) or an H2O cache (n = its n) are all
 * valid inputs.
 *
 * q       [B, H, D] with element strides qs.b, qs.h (qs.t unused).
 * k, v    [B, H, >= n, D], both with strides kvs (D contiguous).
 * out     [B, H, D] float32, contiguous; every element is written.
 * workspace  device buffer of kvc_decode_attention_workspace_bytes(...)
 *         bytes, used when the rows are split over several workgroups per
 *         head (n > 256, or n > 128 when B*H*ceil(n/256) < 512) and their
 *         partial results merged; may be NULL otherwise. Contents on entry
 *         do not matter.
 * Requires n >= 1, D in {64, 128}, 16-byte aligned pointers and strides.
 * Scores and the softmax are fp32 (2^x on the hardware unit); bf16 inputs are
 * widened exactly. */
kvc_status kvc_decode_attention(const void* q, kvc_strides qs, const void* k,
                                const void* v, kvc_strides kvs, int B, int H,
                                int n, int D, kvc_dtype dt, float* out,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* The same attention for callers that cannot allocate or bring device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument, and the call allocates nothing. Where the
 * rows are split over several workgroups per head, the partials go to a static
 * device array of the library (8 MiB on each GPU it runs on, held until the
 * process ends); sizes whose partials exceed it (kvc_decode_attention_workspace_bytes
 * > 8 MiB, e.g. B*H*ceil(n/256) > 16131 at D = 128) return KVC_ERR_WORKSPACE
 * and leave `out` untouched. Every call on one GPU shares that array: calls
 * that overlap on one GPU (on different streams, or from several threads)
 * race. The array needs no clearing: every partial is written before it is
 * read. Arguments, results and errors are otherwise those of
 * kvc_decode_attention (the same kernels compute the same values). */
kvc_status kvc_decode_attention_noalloc(const void* q, kvc_strides qs, const void* k,
                                        const void* v, kvc_strides kvs, int B, int H,
                                        int n, int D, kvc_dtype dt, float* out,
                                        hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Instrumentation (not part of the method).                                  */
/* ------------------------------------------------------------------------- */

/* A plain streaming read of `bytes` bytes at `buf` (device memory, 16-byte
 * aligned, a positive multiple of 16): blocks_per_cu (1..64) workgroups of 256
 * threads per compute unit, each thread reading four 16-byte pieces per step
 * of a grid-stride loop. Its time against `bytes` is what the device streams
 * with a read-only kernel, the reference for the library's HBM-bound kernels.
 * sink: device buffer of 256 words, written only in the unlikely case the
 * data's folded value hits a fixed pattern (it keeps the loads live). */
kvc_status kvc_measure_stream_read(const void* buf, size_t bytes, int blocks_per_cu, unsigned* sink,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
