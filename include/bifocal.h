/*
 * bifocal.h -- C ABI of the MI355X (gfx950) Dynamic Bifocal RoPE attention library.
 *
 * The method (Jet-Long, "Efficient Long-Context Extension with Dynamic Bifocal RoPE"):
 * causal grouped-query attention in which a query/key pair (i, j), j <= i, is
 *   - LOCAL  when 0 <= i - j < w0: scored with the ordinary RoPE positions i and j;
 *   - REMOTE when i - j >= w0:     scored as if the positions were f(i) and f(j),
 *     f(x) = floor(x / G), G = max(1, ceil(L / w_pretrained)) from the current length L.
 * Sources: review page "Paper Review -- Jet-Long" (romaanj.github.io), section Method;
 * gist.science technical summary "Technische Samenvatting: Jet-Long", Methodologie
 * sections 1 (G and f) and 2 (correction rotation, inclusion-exclusion merge).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (HIP), row-major, no padding.
 *   - Alignment: bf16 tensors and workspaces 16 bytes, float32 / int32 arrays 4 bytes (every
 *     hipMalloc or torch allocation is 256-byte aligned); a misaligned pointer returns
 *     BIFOCAL_EINVAL.
 *   - Element type is bfloat16 (raw 16-bit storage) for Q, K, V, O; LSE is float32.
 *   - q and k are POST-base-RoPE: each vector is already rotated at its absolute position
 *     (the cache convention of the method: cached keys stay at their base positions and
 *     are never rewritten). The library applies only the correction rotation by
 *     Delta_x = f(x) - x to remote vectors, in registers.
 *   - RoPE pairs are half-split, (d, d + D/2), with frequencies theta^(-2k/D).
 *   - Query head h reads KV head h / (n_q_heads / n_kv_heads).
 *   - Softmax scale is 1/sqrt(head_dim). LSE outputs are natural-log log-sum-exps.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream).
 *     The library allocates nothing, never synchronises the host, and keeps no state between
 *     calls apart from the static per-device scratch of bifocal_decode_noalloc (whose calls
 *     must therefore not overlap on one device); every other entry point is safe to call from
 *     several host threads at once. A call only launches kernels on `stream` (no memset, copy
 *     or allocation), so it can be captured into a HIP graph.
 *   - Every argument is validated on the host BEFORE any HIP call; a failed check
 *     returns a negative status and leaves device memory untouched. C++ exceptions never
 *     cross this boundary. A failed kernel launch returns BIFOCAL_EHIP.
 *   - Ownership: the caller owns every buffer; pointers are only used during the call's
 *     kernels. Input buffers are never written.
 */
#ifndef BIFOCAL_H_
#define BIFOCAL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BIFOCAL_OK = 0,
  BIFOCAL_EINVAL = -1,       /* null pointer, non-positive size, bad w0/theta, head mismatch */
  BIFOCAL_EUNSUPPORTED = -2, /* valid arguments the kernels do not implement (head_dim, group) */
  BIFOCAL_EWORKSPACE = -3,   /* workspace missing (decode) or smaller than required */
  BIFOCAL_EHIP = -4,         /* a HIP runtime call or kernel launch failed */
  BIFOCAL_ESCRATCH = -5      /* bifocal_decode_noalloc: the shapes need more than its static scratch */
} bifocal_status;

/* Dynamic group size G = max(1, ceil(L / w_pretrained)) (review page, Method; gist.science
 * summary, Methodologie section 1). Pure host arithmetic in int64.
 * Returns G >= 1, or BIFOCAL_EINVAL (< 0) when L < 1 or w_pretrained < 1. */
int64_t bifocal_group_size(int64_t L, int64_t w_pretrained);

/* Bytes of the optional bifocal_prefill workspace for these shapes: room for the corrected
 * keys K' = R(Delta) K~ (same size as k). Returns 0 for invalid arguments. */
size_t bifocal_prefill_workspace_bytes(int batch, int n_kv_heads, int head_dim, int64_t L);

/* Fused bifocal prefill: every pair routed by index, local/remote contributions merged by
 * log-sum-exp in registers, one attention kernel launch.
 *   q    [batch, L, n_q_heads,  head_dim] bf16, post-base-RoPE
 *   k    [batch, L, n_kv_heads, head_dim] bf16, post-base-RoPE
 *   v    [batch, L, n_kv_heads, head_dim] bf16
 *   o    [batch, L, n_q_heads,  head_dim] bf16, written
 *   lse  [batch, n_q_heads, L] float32, written when not NULL
 *   workspace / workspace_bytes: optional device buffer owned by the caller.
 *     NULL: the attention kernel applies the key correction rotation to each key tile as it
 *           stages it (single launch, no extra memory).
 *     non-NULL (>= bifocal_prefill_workspace_bytes): a first small kernel writes the
 *           corrected keys once into the workspace and the attention kernel reads them
 *           (two launches; the rotation is done once per key instead of once per key tile
 *           visit). Contents need no initialisation and are clobbered; calls sharing a
 *           workspace must be ordered (same stream).
 * Row i attends keys 0..i; G is computed once from the full L for every row.
 * w0 >= L makes every pair local (plain causal RoPE attention); w0 = 0 makes every pair
 * remote. head_dim must be 64 or 128; n_q_heads must be a multiple of n_kv_heads;
 * n_kv_heads * head_dim below 2^24 (BIFOCAL_EUNSUPPORTED otherwise, also for the chunked and
 * unfused prefill).
 * Limits: L <= 2^30, batch * L * heads * head_dim < 2^62.
 * Returns BIFOCAL_OK or a negative bifocal_status (BIFOCAL_EWORKSPACE when a non-NULL
 * workspace is smaller than required). */
int bifocal_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                    int batch, int n_q_heads, int n_kv_heads, int head_dim,
                    int64_t L, int64_t w0, int64_t w_pretrained, double rope_theta,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Chunked prefill (prefill against a cache prefix): q_len query rows at absolute positions
 * q_offset .. L - 1 attend keys 0 .. L - 1 of a base-position cache, L = q_offset + q_len, with
 * G = max(1, ceil(L / w_pretrained)) from this L (review page, Method: G follows the current
 * length, so a stream of chunks crosses length boundaries with no cache rewrite; gist.science
 * summary, Methodologie section 2: the cache keeps base positions and the correction is applied
 * in registers). Row r equals row q_offset + r of bifocal_prefill over the first L positions.
 *   q        [batch, q_len, n_q_heads, head_dim] bf16, post-base-RoPE at positions q_offset + r
 *   k_cache  [batch, cache_capacity, n_kv_heads, head_dim] bf16, positions 0 .. L-1 valid (the
 *            chunk's own keys already written at q_offset .. L-1); read only
 *   v_cache  same layout as k_cache
 *   o        [batch, q_len, n_q_heads, head_dim] bf16, written
 *   lse      [batch, n_q_heads, q_len] float32, written when not NULL
 *   workspace / workspace_bytes: as for bifocal_prefill, sized for L:
 *            >= bifocal_prefill_workspace_bytes(batch, n_kv_heads, head_dim, q_offset + q_len)
 *            (the corrected keys of positions 0 .. L-1, compact [batch, L, n_kv_heads, head_dim]).
 * q_offset = 0 with q_len = cache_capacity is bifocal_prefill. Requires q_len >= 1,
 * q_offset >= 0, q_offset + q_len <= cache_capacity <= 2^30; other limits as bifocal_prefill.
 * Returns BIFOCAL_OK or a negative bifocal_status. */
int bifocal_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                          int batch, int n_q_heads, int n_kv_heads, int head_dim,
                          int64_t q_len, int64_t q_offset, int64_t cache_capacity,
                          int64_t w0, int64_t w_pretrained, double rope_theta,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace bifocal_decode needs for any L <= max_L with these shapes.
 * Returns 0 for invalid arguments (which bifocal_decode would reject anyway). */
size_t bifocal_decode_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                      int64_t max_L);

/* One single-token decode step against a base-position KV cache (split-K + LSE reduce).
 *   q        [batch, n_q_heads, head_dim] bf16: the new token's query, post-base-RoPE at
 *            position p = L - 1
 *   k_cache  [batch, cache_capacity, n_kv_heads, head_dim] bf16, positions 0..L-1 valid
 *            (the new token's key/value already appended at L - 1); read only
 *   v_cache  same layout as k_cache
 *   o        [batch, n_q_heads, head_dim] bf16, written
 *   lse      [batch, n_q_heads] float32, written when not NULL
 *   workspace: device buffer of at least bifocal_decode_workspace_bytes(..., L) bytes,
 *            owned by the caller; its contents need no initialisation and are clobbered.
 * G is recomputed from this step's L (review page, Method: G follows the current length),
 * so a stream of calls crosses a change of G with no cache rewrite. Calls that share a
 * workspace must be ordered (same stream). head_dim must be 64 or 128, and
 * n_q_heads / n_kv_heads at most 16.
 * Returns BIFOCAL_OK or a negative bifocal_status. */
int bifocal_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                   int batch, int n_q_heads, int n_kv_heads, int head_dim,
                   int64_t L, int64_t cache_capacity, int64_t w0, int64_t w_pretrained,
                   double rope_theta, void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static device scratch of bifocal_decode_noalloc (bytes, per device). */
#define BIFOCAL_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* bifocal_decode without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid allocation. The split
 * partials go to a static device array of BIFOCAL_DECODE_NOALLOC_SCRATCH_BYTES that each device
 * the library runs on holds until the process ends; the call allocates nothing and calls no
 * allocating routine. Arguments, layouts, results and error checks are those of bifocal_decode;
 * calls whose bifocal_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, L) exceeds
 * the scratch return BIFOCAL_ESCRATCH before any HIP call (16 MiB holds, for example, 32 query
 * heads of head_dim 128 at any L for batch <= 256). The scratch used is the CURRENT device's:
 * the tensors and `stream` must belong to the current device. Every call on a device shares
 * that device's scratch, so calls that may overlap on one device (other streams, other host
 * threads) race and must be ordered by the caller; nothing in the scratch needs to start at
 * zero (every partial a call reads, it first writes). Returns BIFOCAL_OK or a negative
 * bifocal_status. */
int bifocal_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                           int batch, int n_q_heads, int n_kv_heads, int head_dim,
                           int64_t L, int64_t cache_capacity, int64_t w0, int64_t w_pretrained,
                           double rope_theta, void* stream);

/* One decode step that also takes in the new token (review page, Method: keys are cached at
 * their base positions and never rewritten; gist.science summary, Methodologie section 2). The
 * new token sits at p = L - 1; its query and key arrive raw (before any RoPE):
 *   q_raw    [batch, n_q_heads, head_dim] bf16, read only
 *   k_raw    [batch, n_kv_heads, head_dim] bf16, read only
 *   v_new    [batch, n_kv_heads, head_dim] bf16, read only
 *   k_cache, v_cache: as bifocal_decode, positions 0..L-2 valid; row L-1 is WRITTEN: the key
 *            rotated by base RoPE at p (angle p * omega_k, half-split pairs) and the value as is
 *   o, lse, workspace (>= bifocal_decode_workspace_bytes(..., L)), stream: as bifocal_decode.
 * The output equals bifocal_decode(rope(q_raw, p), caches with row p written, ..., L). The
 * rotation and the cache write happen inside the split kernel, so the step is the decode's two
 * launches; o is written only by the second, after every read of q_raw, k_raw and v_new, so it
 * may alias them. All arguments are checked before anything is written; on an error return
 * the caches are untouched. Returns BIFOCAL_OK or a negative bifocal_status. */
int bifocal_decode_step(const void* q_raw, const void* k_raw, const void* v_new, void* k_cache, void* v_cache,
                        void* o, float* lse, int batch, int n_q_heads, int n_kv_heads, int head_dim,
                        int64_t L, int64_t cache_capacity, int64_t w0, int64_t w_pretrained,
                        double rope_theta, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace bifocal_decode_varlen needs with these shapes, at any lengths:
 * (workgroups + batch) partial records of n_q_heads x (head_dim + 2) floats, workgroups = 256 per
 * group of 8 KV heads (rounded up), then two int32 per sequence. Linear in the batch.
 * Returns 0 for invalid arguments. */
size_t bifocal_decode_varlen_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                             int64_t max_len);

/* Batched decode with one length per sequence (a variable-length batch): sequence b's query, at
 * position L_b - 1, attends its cached keys 0 .. L_b - 1 with its own group size
 * G_b = max(1, ceil(L_b / w_pretrained)) (review page, Method: G follows the current length).
 *   seq_lens  [batch] int32 DEVICE array of the lengths L_b; values outside [1, max_len] are
 *             clamped into it
 *   max_len   host-side upper bound of every L_b; 1 <= max_len <= cache_capacity
 *   q, k_cache, v_cache, o, lse, w0, w_pretrained, rope_theta, stream: as bifocal_decode;
 *   workspace >= bifocal_decode_varlen_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim,
 *             max_len).
 * The device lays the 32-key blocks of all sequences end to end and gives each workgroup of one
 * grid (about one per CU) an equal run of them, whatever the mix of lengths; a run may hold the
 * end of one sequence and the start of the next. Sequence b's output is bifocal_decode of that
 * sequence alone at L = L_b, up to the rounding of a different split (the partials merge in
 * another order).
 * Returns BIFOCAL_OK or a negative bifocal_status (BIFOCAL_EINVAL when seq_lens is NULL). */
int bifocal_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                          int batch, int n_q_heads, int n_kv_heads, int head_dim,
                          const int32_t* seq_lens, int64_t max_len, int64_t cache_capacity,
                          int64_t w0, int64_t w_pretrained, double rope_theta,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---- Unfused three-pass forms (an ablation of the fusion, same results) ----
 * The pages write the prefill as three ordinary attention calls merged by inclusion-exclusion
 * (review page, Method; gist.science summary, Methodologie section 2): A = sliding window w0 on
 * the base-position vectors, B = full causal on the remote vectors R(Delta) q, R(Delta) k, C =
 * sliding window w0 on the remote vectors, then O = (W_A O_A + W_B O_B - W_C O_C) /
 * (W_A + W_B - W_C), W_X = exp(LSE_X - max(LSE_A, LSE_B)). These entry points run exactly that:
 * the remote vectors are rotated into the workspace, each pass is a separate plain-attention
 * launch writing O_X (fp32 in the prefill, bf16 in the decode, whose passes end in the decode's
 * own reduce) and fp32 LSE_X to the workspace, and a merge kernel writes o (and lse). They exist
 * to measure what the fusion saves; the results match the fused calls within the rounding of
 * the materialised remote vectors q' and k' (and, in the decode, of the bf16 pass outputs). */

/* Bytes of workspace for bifocal_prefill_unfused; 0 for invalid arguments. */
size_t bifocal_prefill_unfused_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                               int64_t L);

/* Arguments as bifocal_prefill (q, k, v post-base-RoPE); the workspace is required:
 * >= bifocal_prefill_unfused_workspace_bytes(...), caller-owned, clobbered. Six to eight
 * launches on `stream` (two rotations, three passes or one when w0 = 0, one merge).
 * Returns BIFOCAL_OK or a negative bifocal_status. */
int bifocal_prefill_unfused(const void* q, const void* k, const void* v, void* o, float* lse,
                            int batch, int n_q_heads, int n_kv_heads, int head_dim,
                            int64_t L, int64_t w0, int64_t w_pretrained, double rope_theta,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace for bifocal_decode_unfused at any L <= cache_capacity; 0 for invalid
 * arguments. It holds a rotated copy of the whole key cache ([batch, cache_capacity,
 * n_kv_heads, head_dim] bf16). */
size_t bifocal_decode_unfused_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim,
                                              int64_t cache_capacity);

/* Arguments as bifocal_decode; the workspace must hold
 * bifocal_decode_unfused_workspace_bytes(..., cache_capacity) bytes. Per call: all L cached
 * keys are rotated into the workspace copy, then three plain decode passes (each a split and
 * a reduce launch) and the merge. Returns BIFOCAL_OK or a negative bifocal_status. */
int bifocal_decode_unfused(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                           int batch, int n_q_heads, int n_kv_heads, int head_dim,
                           int64_t L, int64_t cache_capacity, int64_t w0, int64_t w_pretrained,
                           double rope_theta, void* workspace, size_t workspace_bytes, void* stream);

/* Parity hook for the position arithmetic: writes G (from L and w_pretrained) to
 * G_out[0] and f(x) = floor(x / G) to f_out[x] for x < L, using the same device code the
 * attention kernels use (gist.science summary, Methodologie section 1).
 *   f_out [L] int32 device buffer; G_out [1] int32 device buffer.  L <= 2^31 - 1. */
int bifocal_positions(int64_t L, int64_t w_pretrained, int32_t* f_out, int32_t* G_out,
                      void* stream);

/* Static, NUL-terminated, host-memory description of a status code (never NULL). */
const char* bifocal_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* BIFOCAL_H_ */
