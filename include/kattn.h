/*
 * kattn.h -- C ABI of libkattn.so: packed variable-length attention on the
 * AMD MI355X (gfx950), head width 64, FP32 in and out.
 *
 * Sources (docs.rs source pages):
 *   [kime-cpu plan.rs]   kime-cpu 0.0.17, src/kime_cpu/plan.rs -- CPU backend
 *   [kime-cuda plan.rs]  kime-cuda 0.0.3, src/plan.rs -- CUDA backend
 *   [argus text.rs]      ffai-argus 0.7.3, src/text.rs -- SmolLM2 text tower
 *
 * Conventions shared by every call
 * --------------------------------
 * - Status: KATTN_OK (0) or a negative KATTN_E* code.  On error,
 *   kattn_last_error() returns a message for the calling thread, valid until
 *   that thread's next kattn call.  Every argument check runs on the host and
 *   fails before anything is queued on the device (errors are values, as in
 *   the kime pages' lowering checks and the argus cache append's bail-outs).
 * - Pointers marked "device" are device memory owned by the caller (for
 *   example torch tensors); "host" pointers are host memory owned by the
 *   caller.  The library keeps no pointer after a call returns and allocates
 *   no memory on any call.
 * - Device calls queue work on `stream` (NULL: the null stream) and return
 *   without synchronising.  Errors raised by the device after the call
 *   returns show up at the caller's next synchronisation.
 * - Strides are in floats.  Every float pointer and every stride must be a
 *   multiple of 16 bytes (4 floats); the kernels load and store 16 bytes at a
 *   time.
 * - head_dim must be 64 (the pages lower heads of 64 only).
 * - Device index tables (cu, pos, used) are preconditions: kattn_build_index
 *   produces well-formed ones.  The kernels never read or write outside the
 *   buffers the sizes describe even when a table is malformed (offsets are
 *   clamped to [0, T], positions outside the table leave a row unrotated),
 *   but the results are then unspecified.  With KATTN_CHECK=1 in the
 *   environment each call copies its device tables to the host, validates
 *   them and returns KATTN_EBOUNDS on a bad one before queueing any work
 *   (synchronous; debugging only; read on every call).  KATTN_SPLIT=0 forces the shared-tile prefill kernel, 1 the
 *   key-split kernel that small launches get, 4 or 8 that kernel with 4 or 8
 *   waves per work-group, "band" the persistent sliding-window kernel that
 *   packed batches with a half-window of at most 64 and at most 1023
 *   sequences get by default; results agree to rounding either way (testing
 *   only, read on every call).
 *
 * Fixed shapes and graph capture
 * ------------------------------
 * The work of every device call is scheduled on the device from the device
 * tables (the query-tile list from cu, the decode key split from used), so a
 * launch's shape depends only on the host sizes.  A caller that captures a
 * fixed shape (a HIP graph, the pages' remark that padding matters to a
 * backend capturing one shape) sizes the call for a bucket and writes the
 * real counts into the device tables before each replay:
 *   - prefill (kattn_varlen_fwd*, kattn_prefill_cached): S and T are the
 *     bucket's; cu may end below T (cu[S] <= T) and trailing sequences may be
 *     empty.  Rows at and past cu[S] are neither read nor written.
 *     max_seqlen (max_chunk, max_ctx) is the bucket's bound.
 *   - decode: B is the bucket's; a slot with used[b] = 0 is skipped (its out
 *     row and caches untouched).  max_used is the bound (cap, say).
 * No call allocates, synchronises or queues a memset or a copy, so each can
 * be captured on the caller's stream (not with KATTN_CHECK=1).  A captured
 * call keeps the pointers and host sizes it was captured with.
 */
#ifndef KATTN_H
#define KATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KATTN_OK = 0,
    KATTN_EINVAL = -1,       /* null pointer, negative size, bad scalar */
    KATTN_EUNSUPPORTED = -2, /* head_dim != 64, H % G != 0, misaligned pointer or stride */
    KATTN_EBOUNDS = -3,      /* offsets, lengths, table or workspace too small */
    KATTN_EDEVICE = -4       /* a HIP call failed */
};

/* Message for the last failed call on this thread ("" after a success). */
const char* kattn_last_error(void);

/*
 * RoPE cos/sin tables for heads of 64 at one base `theta`, positions
 * 0..len-1, written to host arrays cos_host[len][32], sin_host[len][32].
 * Rounding follows [kime-cuda plan.rs] `rope_tables`, which that page states
 * matches the CPU backend: the exponent 2i/64 in f32, theta^e in f64 rounded
 * to f32, its f32 reciprocal, the f32 product with the f32 position, and
 * cos/sin of that angle in f64 rounded to f32.  The caller copies the tables
 * to the device once per base (the pages deduplicate tables by base).
 * Errors: EINVAL for theta <= 0 or not finite, len < 0, null outputs.
 */
int kattn_rope_tables(double theta, int32_t len, float* cos_host, float* sin_host);

/*
 * Host index build for a packed batch ([kime-cpu plan.rs] `CpuBackend::run`;
 * [kime-cuda plan.rs] `CudaBackend::run`): sequence s holds rows
 * cu[s] .. cu[s+1]-1 of every activation.
 *   cu_host:  host int32[S+1]; must satisfy cu[0] = 0, cu[s] <= cu[s+1], cu[S] = T.
 *   seq_host: host int32[T] or NULL; seq[r] = the sequence holding row r.
 *   pos_host: host int32[T] or NULL; pos[r] = r - cu[seq[r]], the position
 *             inside the sequence (RoPE restarts at 0 in every sequence).
 *   max_seqlen_out: host int32* or NULL; the longest sequence.
 * Errors: EINVAL for S < 0, T < 0 or cu_host NULL; EBOUNDS for malformed cu.
 */
int kattn_build_index(const int32_t* cu_host, int32_t S, int32_t T, int32_t* seq_host,
                      int32_t* pos_host, int32_t* max_seqlen_out);

/*
 * RoPE prologue, in place ([kime-cpu plan.rs] `Ctx::step` Rope arm;
 * [kime-cuda plan.rs] `launch_step` Rope arm; [argus text.rs] `rope`).
 * For every row r < T and every q head (H of them, row r of q at
 * q + r*q_stride, head h at columns 64h..64h+63) and every k head (G, in k),
 * with p = pos[r], c = cos[p][i], s = sin[p][i], i < 32:
 *   x[i]    <- x[i] c - x[i+32] s
 *   x[i+32] <- x[i+32] c + x[i] s
 * (half-split pairs, candle's non-interleaved rope).  v is never touched.
 *   q, k:       device float, rows of at least H*64 / G*64 floats.  For a
 *               packed qkv row pass k = q + H*64 and the same stride.
 *   pos:        device int32[T] (from kattn_build_index).
 *   cos, sin:   device float[table_len][32] (from kattn_rope_tables).
 * T == 0 queues nothing.  Rows whose pos is outside [0, table_len) are left
 * unrotated.
 * Errors: EINVAL (nulls, T < 0, H < 1, G < 0, table_len < 1), EUNSUPPORTED
 * (head_dim, alignment), EBOUNDS (stride narrower than the row), EDEVICE.
 */
int kattn_rope_prologue(float* q, int64_t q_stride, int32_t H, float* k, int64_t k_stride,
                        int32_t G, const int32_t* pos, int32_t T, const float* cos,
                        const float* sin, int32_t table_len, int32_t head_dim,
                        hipStream_t stream);

/*
 * Bytes of device workspace kattn_varlen_fwd (and its _rope and _f16 forms)
 * needs for a batch of S sequences and T rows.  The caller allocates it once
 * per bucket and passes it to every call, so no call allocates: the scratch
 * of the pages' CPU backend is likewise sized for the bucket when its plan is
 * built, and its run path never allocates ([kime-cpu plan.rs] module docs).
 * The size depends on S and T only (not on the lengths).  0 for S < 0 or T < 0.
 */
size_t kattn_varlen_fwd_workspace(int32_t S, int32_t T);

/*
 * Varlen attention forward over already-rotated q/k ([kime-cpu plan.rs]
 * `Ctx::step` Attention arm; [kime-cuda plan.rs] `launch_step` Attention arm;
 * [argus text.rs] `block`, `CausalSoftmax`).  For every sequence s, row i of
 * s (position i) and q head h, with g = h / (H/G) (the GQA grouping of
 * [argus text.rs] `block`: q heads 0..R-1 read kv head 0, and so on):
 *   out[i][64h..] = sum_j softmax_j(scale * <q_i,h , k_j,g> + M_ij) v_j,g
 * over keys j of the same sequence, where M_ij = 0 when j is visible and
 * -inf otherwise.  Visible: (window < 0 or |i - j| <= window / 2) and
 * (causal == 0 or j <= i).  Masked keys are skipped, which gives the same
 * result as the -inf mask ([argus text.rs] module docs).
 *   out:        device float (T, H*64), row stride out_stride.  Rows >= T
 *               and columns >= H*64 are never written.
 *   q, k, v:    device float (T, H*64), (T, G*64), (T, G*64) with their own
 *               strides (a packed qkv row: k = q + H*64, v = k + G*64).
 *   cu:         device int32[S+1], the offsets of kattn_build_index, or a
 *               bucket's padded offsets with cu[S] <= T (see above).
 *   max_seqlen: longest sequence (host scalar, from kattn_build_index).  It must not
 *               be smaller than the longest sequence: a window whose half-width reaches
 *               max_seqlen - 1 masks nothing and runs as global attention.
 *   window:     -1 for none (the CUDA page's encoding), else >= 0.
 *   causal:     0 or 1.
 *   scale:      finite, > 0; folded into q as it is loaded (exact for 1/8).
 *   workspace:  device, >= kattn_varlen_fwd_workspace(S, T) bytes, 256-byte
 *               aligned; holds the query-tile schedule built on the device
 *               (sliding-window launches and one-sequence batches schedule
 *               without it, but it is required all the same).
 * T == 0 or S == 0 queues nothing.
 * Errors: EINVAL, EUNSUPPORTED (head_dim, H % G, alignment), EBOUNDS
 * (stride narrower than the row, max_seqlen > T, workspace), EDEVICE.
 */
int kattn_varlen_fwd(float* out, int64_t out_stride, const float* q, int64_t q_stride,
                     const float* k, int64_t k_stride, const float* v, int64_t v_stride,
                     const int32_t* cu, int32_t S, int32_t T, int32_t max_seqlen, int32_t H,
                     int32_t G, int32_t head_dim, int32_t window, int32_t causal, float scale,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Varlen attention forward with the RoPE step fused into the tile loads
 * ([kime-cpu plan.rs] `Ctx::step` Rope then Attention arms; [argus text.rs]
 * `rope` then `block`).  The same result as kattn_rope_prologue at positions
 * pos[r] = r - cu[s] followed by kattn_varlen_fwd, up to rounding order, but
 * q and k are read-only: each q row is rotated as it is loaded and each k row
 * as it is staged, so the separate in-place pass over q and k disappears.
 *   q, k:       device float, UNROTATED (layout as in kattn_varlen_fwd).
 *   cos, sin:   device float[table_len][32] (from kattn_rope_tables), required;
 *               table_len >= max_seqlen.
 * Every other argument as in kattn_varlen_fwd (same workspace size).
 * Errors: as kattn_varlen_fwd, plus EINVAL for NULL tables and EBOUNDS for
 * table_len < max_seqlen.
 */
int kattn_varlen_fwd_rope(float* out, int64_t out_stride, const float* q, int64_t q_stride,
                          const float* k, int64_t k_stride, const float* v, int64_t v_stride,
                          const int32_t* cu, int32_t S, int32_t T, int32_t max_seqlen, int32_t H,
                          int32_t G, int32_t head_dim, int32_t window, int32_t causal, float scale,
                          const float* cos, const float* sin, int32_t table_len, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * Varlen attention forward with a binary16 output ([kime-cuda plan.rs] the
 * attention variants that store a half output for a half tower; q, k and v
 * stay FP32 and every step computes in FP32).  Each output element is the
 * FP32 result rounded to the nearest binary16 (ties to even).
 *   out:        device IEEE binary16 (T, H*64), row stride out_stride in
 *               halves, a multiple of 8 (16 bytes); 16-byte aligned.
 *   cos, sin:   both NULL when q and k are already rotated (as for
 *               kattn_varlen_fwd), or the tables for fused rotation (as for
 *               kattn_varlen_fwd_rope, table_len >= max_seqlen).
 * Every other argument as in kattn_varlen_fwd (same workspace size).
 */
int kattn_varlen_fwd_f16(void* out, int64_t out_stride, const float* q, int64_t q_stride,
                         const float* k, int64_t k_stride, const float* v, int64_t v_stride,
                         const int32_t* cu, int32_t S, int32_t T, int32_t max_seqlen, int32_t H,
                         int32_t G, int32_t head_dim, int32_t window, int32_t causal, float scale,
                         const float* cos, const float* sin, int32_t table_len, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace kattn_prefill_cached needs for B sequences and T chunk rows
 * (sized once per bucket, as kattn_varlen_fwd_workspace). */
size_t kattn_prefill_cached_workspace(int32_t B, int32_t T);

/*
 * Chunked prefill continuing from preallocated KV caches ([argus text.rs]
 * `KvAppend` at the cache's fill point, then `CausalSoftmax` with q_len > 1
 * and an offset, whose causal limit for query i is key offset + i; the GQA
 * fold of `block`).  Sequence b brings n_b = cu[b+1] - cu[b] new rows (packed
 * rows cu[b] .. cu[b+1]-1 of q, k_new, v_new) and already holds off_b =
 * offset[b] rows.  With p = off_b + i for chunk row i:
 *   1. k_new row i (rotated at p when cos != NULL) and v_new row i are
 *      written into cache row p of every kv head of b; no other cache row is
 *      written;
 *   2. q row i (rotated at p when cos != NULL, scaled by `scale`; q itself is
 *      not modified) attends, head h through kv head h / (H/G), to cache rows
 *      0 .. p: out[cu[b]+i][64h..] = sum_j softmax_j(scale <q, k_j>) v_j.
 * Decode is the case n_b = 1 (kattn_decode does it with a split over keys).
 *   out:        device float (T, H*64), row stride out_stride.
 *   q:          device float (T, H*64), row stride q_stride.
 *   k_new, v_new: device float (T, G*64) with their strides.
 *   cu:         device int32[B+1], chunk offsets (as kattn_build_index checks them).
 *   offset:     device int32[B], rows already in each sequence's caches.
 *   max_chunk:  host, the longest chunk (<= T); max_ctx: host, max of
 *               offset[b] + n_b, with max_chunk <= max_ctx <= cap.
 *   k_cache, v_cache: device float [B][G][cap][64] (the kattn_decode layout).
 *   cos, sin:   device float[table_len][32], table_len >= max_ctx, or both
 *               NULL when q and k_new are already rotated.
 *   workspace:  device, >= kattn_prefill_cached_workspace(B, T) bytes,
 *               256-byte aligned.
 * Preconditions on the device tables: 0 <= offset[b], offset[b] + n_b <=
 * max_ctx, n_b <= max_chunk.  The kernels stay inside every buffer when they
 * do not hold (rows past the cache are not appended; keys are clamped to the
 * cache), but the results are then unspecified; KATTN_CHECK=1 validates them.
 * T == 0 or B == 0 queues nothing.
 * Errors: EINVAL, EUNSUPPORTED (head_dim, H % G, alignment, B > 65535),
 * EBOUNDS (max_chunk, max_ctx, cap, table_len, strides, workspace), EDEVICE.
 */
int kattn_prefill_cached(float* out, int64_t out_stride, const float* q, int64_t q_stride,
                         const float* k_new, int64_t k_stride, const float* v_new, int64_t v_stride,
                         const int32_t* cu, const int32_t* offset, int32_t B, int32_t T,
                         int32_t max_chunk, int32_t max_ctx, float* k_cache, float* v_cache,
                         int32_t cap, int32_t H, int32_t G, int32_t head_dim, float scale,
                         const float* cos, const float* sin, int32_t table_len, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of device workspace kattn_decode needs for B sequences, H q heads and
 * G kv heads (0 for invalid sizes).  The size does not depend on the cache
 * lengths, so one workspace sized for a bucket serves every step of a decode
 * loop and no step allocates (the bucket-sized, allocate-nothing run path of
 * [kime-cpu plan.rs] module docs; the preallocated cache of [argus text.rs]
 * `KvAppend`).
 */
size_t kattn_decode_workspace(int32_t B, int32_t H, int32_t G);

/*
 * One decode step against preallocated caches ([argus text.rs] `KvAppend`,
 * the KV cache part of `block`, and `CausalSoftmax` with offset L-1, where a
 * decode row sees the whole cache).  For every sequence b with L = used[b]
 * (counting the new token) and p = L - 1:
 *   1. the new k (rotated at p when cos != NULL) and the new v are written
 *      into row p of every kv head of b's caches; no other cache row is
 *      written;
 *   2. the new q (rotated at p when cos != NULL, scaled by `scale`) attends,
 *      head h through kv head h / (H/G), to rows 0..p with no mask:
 *      out[b][64h..] = sum_j softmax_j(scale * <q_h, k_j>) v_j.
 *   out:        device float [B][H*64].
 *   q:          device float [B][H*64] (the new token's q heads).
 *   k_new, v_new: device float [B][G*64].
 *   k_cache, v_cache: device float [B][G][cap][64]; row j of kv head g of
 *               sequence b at ((b*G + g)*cap + j)*64 ([argus text.rs]
 *               `KvAppend` layout, stacked over the batch).
 *   used:       device int32[B], 1 <= used[b] <= max_used, or 0 for an idle
 *               slot of a fixed-shape call.
 *   max_used:   host scalar, 1 <= max_used <= cap; sizes the split over keys.
 *   cos, sin:   device float[table_len][32] with table_len >= max_used, or
 *               both NULL when q and k_new are already rotated.
 *   workspace:  device, >= kattn_decode_workspace(B, H, G) bytes, 256-byte
 *               aligned (the key-split schedule and per-piece partial max, sum
 *               and output).
 * B == 0 queues nothing.  Sequences whose used[b] is outside [1, max_used]
 * are skipped (their out row and caches are left untouched).
 * Errors: EINVAL, EUNSUPPORTED, EBOUNDS (max_used, cap, table_len,
 * workspace), EDEVICE.
 */
int kattn_decode(float* out, const float* q, const float* k_new, const float* v_new,
                 float* k_cache, float* v_cache, int32_t cap, const int32_t* used,
                 int32_t max_used, int32_t B, int32_t H, int32_t G, int32_t head_dim,
                 float scale, const float* cos, const float* sin, int32_t table_len,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kattn_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and the same result, with the key-split
 * partials in a static scratch of 16 MiB that the library holds on every GPU
 * it runs on until the process ends.  The caller still passes every input
 * and output.  Arguments and errors as kattn_decode, without `workspace` and
 * `workspace_bytes`; EBOUNDS when B, H and G need more scratch than 16 MiB
 * (about (1024 + min(B, 1024) * G) * (H / G) * 264 bytes on a 256-CU GPU:
 * B = 64, H = 9, G = 3 needs under 1 MiB), EDEVICE when the scratch has no
 * address on the current GPU.  The call allocates nothing, and nothing in
 * the scratch needs clearing between calls.  Every call on one GPU shares
 * that GPU's scratch: two calls that overlap on one GPU (queued on different
 * streams, or from different threads) race on it and give wrong results;
 * calls on one stream run one after the other and are safe.
 */
int kattn_decode_noalloc(float* out, const float* q, const float* k_new, const float* v_new,
                         float* k_cache, float* v_cache, int32_t cap, const int32_t* used,
                         int32_t max_used, int32_t B, int32_t H, int32_t G, int32_t head_dim,
                         float scale, const float* cos, const float* sin, int32_t table_len,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KATTN_H */
