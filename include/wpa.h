/*
 * wpa.h -- C ABI of libwpa: per-RoPE-wavelength windowed causal attention on MI355X.
 *
 * The operation (ATFlash, "Per-RoPE-Wavelength Attention Windows for Compute/Memory-
 * Efficient LLM Inference", abstract; WavePrune, "One period is often enough for RoPE",
 * original abstract):
 *   The RoPE attention score of query token r and key token c is an exact sum over the
 *   d/2 two-dimensional rotation ("frequency") pairs.  Pair i has wavelength
 *   lambda_i = 2*pi*base^(2i/d) and keeps its term only while the query-key distance
 *   |t_r - t_c| <= alpha*lambda_i; a pruned term contributes zero and the key stays in
 *   the softmax.  alpha = 1 is WavePrune's one-rotation-period window; alpha = +INFINITY is
 *   ordinary (full-window) causal RoPE attention in the same kernels.  Softmax and the
 *   P*V product are unchanged.
 *
 * Conventions shared by every entry point
 *   - Pair layout is half-split: pair i of a head vector is (x[i], x[i + d/2]); rotation
 *     x'[i] = x[i]cos(t th_i) - x[i+d/2] sin(t th_i), x'[i+d/2] = x[i+d/2]cos + x[i]sin,
 *     th_i = base^(-2i/d).
 *   - The window test uses alpha*lambda_i evaluated in IEEE double as
 *       alpha * ((2.0*M_PI) * pow(base, (2.0*i)/d))
 *     and keeps pair i at integer distance D iff D <= that value.
 *   - Logits are scale * (windowed sum); scale <= 0 selects 1/sqrt(d).
 *   - Causality is by token index (key c visible to query r iff c <= r).
 *   - GQA: q head h reads kv head h / (Hq/Hkv).
 *   - dtype (WPA_BF16 or WPA_FP32) is the element type of q, k and v; out_dtype that of
 *     out.  fp32 inputs are rounded to bf16 (round-to-nearest-even) on load.  Rotated
 *     queries (times scale*log2 e) and rotated keys are rounded to IEEE half precision
 *     for the q.k product; probabilities and values enter the P*V product as bf16; both
 *     products accumulate in fp32 and softmax statistics are fp32.  Rotated key components
 *     and scaled rotated query components must stay below 65504 in magnitude (larger ones
 *     overflow to infinity and the affected outputs are not finite).  A bf16 out is the
 *     fp32 result rounded to nearest even.
 *   - All pointers except those documented as host pointers are device pointers.  Device
 *     buffers must be 16-byte aligned.  The caller owns every buffer (including workspace
 *     and caches); the library allocates nothing and keeps no per-call state.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued and the call
 *     returns without waiting; faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Return value: WPA_OK, or a negative status.  Every argument is checked before any
 *     work is enqueued; a failing call enqueues nothing and wpa_last_error() describes it.
 *
 * Supported: d in {64, 128}; Hq % Hkv == 0; base > 1; alpha >= 0 (not NaN; +inf allowed);
 * B, N, heads >= 1; token counts and positions below 2^31.
 */
#ifndef WPA_H
#define WPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    WPA_OK = 0,
    WPA_ERR_INVALID = -1,      /* argument out of range, null or misaligned pointer */
    WPA_ERR_UNSUPPORTED = -2,  /* valid request this library does not implement (e.g. d) */
    WPA_ERR_WORKSPACE = -3,    /* workspace smaller than the matching *_bytes() query */
    WPA_ERR_HIP = -4           /* the HIP runtime reported an error while enqueueing */
};

enum { WPA_BF16 = 0, WPA_FP32 = 1 };

/*
 * Kept-term count, host only, exact (ATFlash abstract: how many terms the window drops
 * depends only on the shapes, d, base and alpha, not on the inputs, and the dropped share
 * grows like log N).  A term is one pair's
 * contribution to one (query, key) score.  Queries sit at positions q_pos0 ..
 * q_pos0+n_q-1, keys at 0 .. n_k-1, key c visible to query r iff c <= r.
 *   *kept  = #{(r, c, i) visible : r - c <= alpha*lambda_i}
 *   *total = (d/2) * #{(r, c) visible}
 * Prefill of N tokens: (n_q = n_k = N, q_pos0 = 0).  Decode at length L: (1, L-1, L).
 * Counts are per head.  Any even d >= 2 is accepted here.  O(d) time.
 */
int wpa_count_terms(int32_t d, double base, double alpha, int64_t n_q, int64_t q_pos0,
                    int64_t n_k, int64_t* kept, int64_t* total);

/*
 * Integer window table the kernels use: W[i] = floor(alpha*lambda_i), or INT32_MAX when
 * that is +inf or exceeds INT32_MAX-1 (every representable distance is then inside).
 * W is a host array of d/2 entries.  Any even d in [2, 128].
 */
int wpa_thresholds(int32_t d, double base, double alpha, int32_t* W);

/* Workspace bytes wpa_prefill needs: the rotated, pair-blocked K and V blocked by key
 * octets (the decode caches' layouts) of all B*Hkv heads, padded to 128 tokens
 * (2 * B*Hkv*roundup(N,128)*d*2 bytes). */
size_t wpa_prefill_workspace_bytes(int32_t B, int64_t N, int32_t Hkv, int32_t d);

/*
 * Causal windowed prefill.
 *   q         [B][N][Hq][d]  pre-RoPE queries (dtype)
 *   k, v      [B][N][Hkv][d] pre-RoPE keys, values (dtype)
 *   out       [B][N][Hq][d]  attention output (out_dtype)
 *   lse       [B][Hq][N] fp32 natural-log sum of exp(logits), or NULL
 *   positions [B][N] int32 token positions, non-decreasing within each sequence and in
 *             [0, 2^31); NULL means 0..N-1.  (Non-decreasing order is a precondition
 *             the kernels rely on; it is not checked.)
 *   term_count  NULL, or a device counter to which the number of kept (query, key, pair)
 *             terms summed over all heads is added (atomically).  It is not cleared.
 *   workspace at least wpa_prefill_workspace_bytes(B, N, Hkv, d) bytes, device.
 */
int wpa_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                const int32_t* positions, int32_t B, int64_t N, int32_t Hq, int32_t Hkv,
                int32_t d, double base, double alpha, float scale, int32_t dtype,
                int32_t out_dtype, unsigned long long* term_count, void* workspace,
                size_t ws_bytes, void* stream);

/*
 * The two halves of wpa_prefill, for callers that time them apart or reuse the prepared
 * keys and values for several query launches.  wpa_prefill(...) is exactly
 * wpa_prefill_prepare(...) followed by wpa_prefill_attend(...) on the same stream.
 *   prepare: rotate k at its positions into the workspace (pair-blocked half) and store v
 *            there by key octets (bf16, zero past token N); q is not read.
 *   attend:  the windowed attention of q against a workspace prepared for the same
 *            B, N, Hkv, d, base, positions (the workspace is only read).
 * Arguments have the meaning given for wpa_prefill.
 */
int wpa_prefill_prepare(const void* k, const void* v, const int32_t* positions, int32_t B,
                        int64_t N, int32_t Hkv, int32_t d, double base, int32_t dtype,
                        void* workspace, size_t ws_bytes, void* stream);
int wpa_prefill_attend(const void* q, void* out, float* lse, const int32_t* positions,
                       int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d, double base,
                       double alpha, float scale, int32_t dtype, int32_t out_dtype,
                       unsigned long long* term_count, const void* workspace, size_t ws_bytes,
                       void* stream);

/* Bytes of the decode caches for B sequences of up to Lmax tokens.  Both layouts belong to
 * the library (K: rotated keys, pair-blocked [B][Hkv][d/16][Lmax][16] half; V: blocked by
 * 8 consecutive tokens, [B][Hkv][ceil(Lmax/8)][d][8] bf16); callers only size, allocate
 * and pass them.  Sequence b's part of each cache is one block of
 * wpa_kcache_bytes(1, Lmax, Hkv, d) (wpa_vcache_bytes(...) for V) bytes at b times that
 * offset, so a call with B = 1 on those offsets touches that sequence alone (how a ragged
 * batch appends each sequence at its own start). */
size_t wpa_kcache_bytes(int32_t B, int64_t Lmax, int32_t Hkv, int32_t d);
size_t wpa_vcache_bytes(int32_t B, int64_t Lmax, int32_t Hkv, int32_t d);

/*
 * Append n tokens (token indices start .. start+n-1, which are also their positions) of
 * every sequence to the decode caches.  k, v are pre-RoPE [B][n][Hkv][d] (dtype).  Keys
 * are rotated once here and stored as IEEE half; values are stored as bf16.
 * Requires 0 <= start, n >= 1, start + n <= Lmax.
 */
int wpa_kv_write(const void* k, const void* v, int64_t start, int64_t n, void* k_cache,
                 void* v_cache, int32_t B, int64_t Lmax, int32_t Hkv, int32_t d, double base,
                 int32_t dtype, void* stream);

/* Workspace bytes wpa_decode needs for split-KV partial results (chunk_keys as passed to
 * wpa_decode; 0 = the library's choice for this shape). */
size_t wpa_decode_workspace_bytes(int32_t B, int64_t Lmax, int32_t Hq, int32_t Hkv,
                                  int32_t d, int32_t chunk_keys);

/*
 * One decode step per sequence (ATFlash abstract: the window ported into a decode
 * kernel; far keys read only the pairs still active).
 *   q        [B][Hq][d] pre-RoPE query (dtype)
 *   k_cache, v_cache  written by wpa_kv_write for the same B, Lmax, Hkv, d, base
 *   kv_len   [B] int32 device: the query sees keys 0 .. kv_len-1.  The kernels clamp each
 *            value into [0, Lmax] (no access leaves the caches, whatever the buffer holds); a
 *            sequence whose clamped kv_len is 0 has no keys: its out is 0 and its lse -inf
 *   q_pos    [B] int32 device query positions, or NULL for kv_len-1 (the query's own
 *            token is then the last cached key)
 *   out      [B][Hq][d] (out_dtype);  lse [B][Hq] fp32 or NULL
 *   chunk_keys  keys per split-KV work item: a multiple of 256 (item c then takes keys
 *            c*chunk_keys .. (c+1)*chunk_keys-1), or 0 for the library's choice: as many
 *            items as ceil(Lmax / C) for a chunk length C it picks, each taking the keys in a
 *            range of distances from the sequence's last key that streams the same cache
 *            bytes (near keys read more of K, so their ranges are shorter).  The result
 *            depends on the split only through rounding (probabilities enter the P*V product
 *            as bf16 relative to each split's running maximum); calls with the same split
 *            (the same d, window table, chunk_keys and ceil(Lmax / chunk)) give the same bits.
 *   workspace at least wpa_decode_workspace_bytes(B, Lmax, Hq, Hkv, d, chunk_keys).
 */
int wpa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_len,
               const int32_t* q_pos, void* out, float* lse, int32_t B, int64_t Lmax,
               int32_t Hq, int32_t Hkv, int32_t d, double base, double alpha, float scale,
               int32_t dtype, int32_t out_dtype, unsigned long long* term_count,
               int32_t chunk_keys, void* workspace, size_t ws_bytes, void* stream);

/*
 * RoPE variants.  The pages state the window for RoPE with frequencies base^(-2i/d) on
 * half-split pairs; models that scale their frequencies (Llama-3-style per-band scaling,
 * NTK or YaRN variants) or pair adjacent dims use the same window with their own per-pair
 * wavelength lambda_i = 2*pi/theta_i (ATFlash abstract: the window is proportional to each
 * pair's wavelength).
 *   pairs     WPA_PAIRS_HALF: pair i = dims (i, i + d/2); WPA_PAIRS_INTERLEAVED: (2i, 2i + 1).
 *   inv_freq  host array of the d/2 rotation frequencies theta_i (radians per position),
 *             finite, > 0 and non-increasing in i (so that the pairs active at a distance
 *             stay a suffix of the pair axis), or NULL for theta_i = base^(-2i/d).  With a
 *             table the window test is D <= alpha * ((2.0*M_PI) / theta_i) in IEEE double,
 *             and `base` is not used.  The table is read during the call only.
 *   head_inv_freq  NULL, or a DEVICE array [Hkv][d/2] of double: one frequency table per kv
 *             head (AdaRoPE abstract, on the ATFlash cards page: rotation frequencies chosen
 *             per head).  Kv head g rotates its keys, and the q heads that read it
 *             (h / (Hq/Hkv) = g) their queries, by row g, and pair i of those heads has the
 *             window D <= alpha * ((2.0*M_PI) / head_inv_freq[g][i]), evaluated on the device
 *             in IEEE double (the same decisions as the host's expression).  Each row must be
 *             finite, > 0 and non-increasing: a precondition (the values live on the device and
 *             are not checked).  inv_freq must then be NULL and `base` is not used.  Per-head
 *             tables are taken by wpa_prefill_ex / _prepare_ex / _attend_ex, wpa_kv_write_ex,
 *             wpa_kv_write_paged, wpa_decode_ex, wpa_decode_paged, wpa_decode_noalloc and the
 *             chunked prefills (wpa_prefill_cached, _varlen, wpa_prefill_paged, _varlen,
 *             wpa_prefill_cached_ex: the caches written with the same rows) and
 *             wpa_prefill_sparse; the other entry points return WPA_ERR_UNSUPPORTED for them, and the host-only count and threshold
 *             queries take one head's table (as inv_freq) at a time.
 * Every *_ex entry point below is its namesake with this description added; rope = NULL
 * means {WPA_PAIRS_HALF, NULL, NULL}.  A table that is not positive and non-increasing is
 * WPA_ERR_UNSUPPORTED; an unknown `pairs` value WPA_ERR_INVALID.  The decode caches hold
 * keys rotated by the description given to wpa_kv_write_ex; wpa_decode_ex must be given
 * the same one (q is rotated by it).
 */
enum { WPA_PAIRS_HALF = 0, WPA_PAIRS_INTERLEAVED = 1 };

typedef struct wpa_rope {
    int32_t pairs;
    const double* inv_freq;        /* host [d/2], or NULL */
    const double* head_inv_freq;   /* device [Hkv][d/2], or NULL */
} wpa_rope_t;

int wpa_count_terms_ex(int32_t d, double base, const wpa_rope_t* rope, double alpha, int64_t n_q,
                       int64_t q_pos0, int64_t n_k, int64_t* kept, int64_t* total);
int wpa_thresholds_ex(int32_t d, double base, const wpa_rope_t* rope, double alpha, int32_t* W);
int wpa_prefill_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                   const int32_t* positions, int32_t B, int64_t N, int32_t Hq, int32_t Hkv,
                   int32_t d, double base, const wpa_rope_t* rope, double alpha, float scale,
                   int32_t dtype, int32_t out_dtype, unsigned long long* term_count,
                   void* workspace, size_t ws_bytes, void* stream);
int wpa_prefill_prepare_ex(const void* k, const void* v, const int32_t* positions, int32_t B,
                           int64_t N, int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope,
                           int32_t dtype, void* workspace, size_t ws_bytes, void* stream);
int wpa_prefill_attend_ex(const void* q, void* out, float* lse, const int32_t* positions,
                          int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d, double base,
                          const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                          int32_t out_dtype, unsigned long long* term_count,
                          const void* workspace, size_t ws_bytes, void* stream);
int wpa_kv_write_ex(const void* k, const void* v, int64_t start, int64_t n, void* k_cache,
                    void* v_cache, int32_t B, int64_t Lmax, int32_t Hkv, int32_t d, double base,
                    const wpa_rope_t* rope, int32_t dtype, void* stream);
int wpa_decode_ex(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_len,
                  const int32_t* q_pos, void* out, float* lse, int32_t B, int64_t Lmax,
                  int32_t Hq, int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope,
                  double alpha, float scale, int32_t dtype, int32_t out_dtype,
                  unsigned long long* term_count, int32_t chunk_keys, void* workspace,
                  size_t ws_bytes, void* stream);

/*
 * Chunked prefill against the decode caches, with a ragged batch (a cached prefix per
 * sequence).  Sequence b holds kv_len[b] tokens in the caches, the last Nq of which are
 * the chunk's queries (tokens kv_len[b]-Nq .. kv_len[b]-1, positions = token indices).
 * Each query attends causally to keys 0 .. its own token under the same per-pair window
 * as wpa_prefill (WavePrune original, the pair-wise window; ATFlash abstract: one window
 * test per pair and distance), so a prompt prefilled in chunks gets the rows a one-shot
 * wpa_prefill would give it (up to rounding order).
 *   q        [B][Nq][Hq][d] pre-RoPE (dtype), device; row i is token kv_len[b]-Nq+i
 *   k_cache, v_cache  as for wpa_decode_ex, with the chunk's keys and values already
 *            appended (wpa_kv_write_ex) under the same rope description
 *   kv_len   [B] int32 device, each in [Nq, Lmax] (a precondition: the values live on the
 *            device; the kernel clamps them into that range so no access leaves the caches)
 *   out      [B][Nq][Hq][d] (out_dtype); lse [B][Hq][Nq] fp32 or NULL
 *   term_count  as for wpa_prefill: kept (pair, query, key) terms, added
 * No workspace: the kernel reads the caches in their own layouts.
 */
int wpa_prefill_cached(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* kv_len, void* out, float* lse, int32_t B, int32_t Nq,
                       int64_t Lmax, int32_t Hq, int32_t Hkv, int32_t d, double base,
                       const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                       int32_t out_dtype, unsigned long long* term_count, void* stream);

/*
 * Chunked prefill with a query count per sequence (varlen): sequence b's chunk is its last
 * q_b = cu_q[b+1] - cu_q[b] tokens (0 <= q_b <= max_q, q_b <= kv_len[b]; a sequence with
 * q_b = 0 is skipped), packed back to back.
 *   cu_q     [B+1] int32 device, non-decreasing from cu_q[0] >= 0: rows cu_q[b] ..
 *            cu_q[b+1]-1 of q and out.  Its values are trusted (the library does not read
 *            device memory on the host): offsets past the end of q/out are the caller's fault.
 *   q        [cu_q[B]][Hq][d] pre-RoPE;  out [cu_q[B]][Hq][d];  lse [cu_q[B]][Hq] or NULL
 *   max_q    an upper bound of every q_b (it sizes the launch; larger counts are clamped)
 * Each row is bit-identical to the same row of wpa_prefill_cached with Nq = q_b.
 */
int wpa_prefill_cached_varlen(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* cu_q, const int32_t* kv_len, void* out, float* lse,
                              int32_t B, int32_t max_q, int64_t Lmax, int32_t Hq, int32_t Hkv,
                              int32_t d, double base, const wpa_rope_t* rope, double alpha,
                              float scale, int32_t dtype, int32_t out_dtype,
                              unsigned long long* term_count, void* stream);

/*
 * Prefill composed with token-level block sparsity (ATFlash abstract: the window can be
 * applied on top of other sparse attention methods).  Tokens form blocks of 64; the query
 * rows of block R of q head h attend, besides block R itself (always), only the key blocks
 * listed for (b, h, R), with the per-pair window on every listed key; keys of unlisted blocks
 * leave the softmax altogether (unlike pruned terms, which keep the key at logit 0).
 *   blk_count  int32 device [B][Hq][ceil(N/64)]: list lengths (clamped to [0, blk_max])
 *   blk_idx    int32 device [B][Hq][ceil(N/64)][blk_max]: key blocks, in any order;
 *              duplicates count once, entries outside [0, R) are ignored (R is always visited).
 *   positions are token indices; other arguments as for wpa_prefill_ex (the workspace is
 *   prepared here).  term_count adds the kept terms of the visited keys.  The lists are held
 *   as bitmaps in LDS beside the kernel's tiles: N up to 2^21 at d = 64 and up to about
 *   9.1e5 tokens at d = 128; a longer N is WPA_ERR_UNSUPPORTED (checked before anything is
 *   enqueued).
 */
int wpa_prefill_sparse(const void* q, const void* k, const void* v, void* out, float* lse,
                       const int32_t* blk_count, const int32_t* blk_idx, int32_t blk_max,
                       int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d, double base,
                       const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                       int32_t out_dtype, unsigned long long* term_count, void* workspace,
                       size_t ws_bytes, void* stream);

/*
 * wpa_prefill_sparse with another block size (the token-level methods the window is composed
 * with index blocks of their own size; ATFlash abstract, as above).  Tokens form blocks of
 * `block` tokens, a power of two from 64 to 1024 (else WPA_ERR_INVALID); the rule, the lists and
 * every other argument are as above with 64 replaced by `block`:
 *   blk_count  int32 device [B][Hq][ceil(N/block)];  blk_idx [B][Hq][ceil(N/block)][blk_max]
 * The same LDS bound on N applies (the lists are held at 64-token granularity).
 * wpa_prefill_sparse is this call with block = 64.
 */
int wpa_prefill_sparse_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                          const int32_t* blk_count, const int32_t* blk_idx, int32_t blk_max,
                          int32_t block, int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d,
                          double base, const wpa_rope_t* rope, double alpha, float scale,
                          int32_t dtype, int32_t out_dtype, unsigned long long* term_count,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * wpa_prefill_sparse_ex at explicit positions (ATFlash abstract: the window is applied on top
 * of token-level block methods, and RoPE rotates each token by its position).  The blocks and
 * the causal rule stay those of token indices: row r attends key c <= r iff c // block is r's
 * own block or is listed for it.  The rotation of q and k and the window compare positions:
 *   positions  int32 device [B][N], non-negative and non-decreasing within each sequence
 *              (repeats allowed), below 2^31 - 1; not null (WPA_ERR_INVALID).
 * Every other argument, the LDS bound on N and the error behaviour are those of
 * wpa_prefill_sparse_ex, per-kv-head frequency tables (rope->head_inv_freq) included.
 */
int wpa_prefill_sparse_pos(const void* q, const void* k, const void* v, void* out, float* lse,
                           const int32_t* blk_count, const int32_t* blk_idx, int32_t blk_max,
                           int32_t block, const int32_t* positions, int32_t B, int64_t N,
                           int32_t Hq, int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope,
                           double alpha, float scale, int32_t dtype, int32_t out_dtype,
                           unsigned long long* term_count, void* workspace, size_t ws_bytes,
                           void* stream);

/*
 * Windowed decode cache (K-dim eviction).  In decode the query is the newest token, so the
 * distance to a given key only grows: once it exceeds the window of every pair of a 16-dim
 * pair block, that block of that key is never read again (WavePrune original abstract:
 * each pair keeps only its first rotation periods; ATFlash abstract: the window is
 * proportional to the wavelength, and a decode step reads only the dims still active).  A
 * windowed K cache keeps pair block j only for the newest W_j + 1 tokens, W_j being the
 * window of the block's last pair at `cache_alpha` (rounded up to 32 rows; a block whose
 * window reaches Lmax keeps all Lmax), in rows reused as a ring.  V is kept whole: a key
 * whose terms are all pruned still enters the softmax, with logit 0.
 *   cache_alpha  the window the cache is built for: finite, >= 0.  Decodes on it take any
 *            alpha <= cache_alpha (a larger alpha is WPA_ERR_INVALID).
 *   wpa_kcache_window_bytes  bytes of such a K cache (0 for invalid arguments); the V cache
 *            is wpa_vcache_bytes.  Sequence b's part is one block at b times the B = 1 size.
 *   wpa_kv_write_window  as wpa_kv_write_ex, into a windowed K cache (and the usual V cache).
 *            Rows are reused: only the newest rows of each block are kept.
 *   wpa_decode_window  as wpa_decode_ex with q_pos = NULL, on a windowed K cache.  Each
 *            kv_len[b] must be at least the end (start + n) of the last write to sequence b
 *            (append-only use: a shorter kv_len would need keys whose rows were reused).
 * Chunked prefill (wpa_prefill_cached) reads the dense cache only.
 */
size_t wpa_kcache_window_bytes(int32_t B, int64_t Lmax, int32_t Hkv, int32_t d, double base,
                               const wpa_rope_t* rope, double cache_alpha);
int wpa_kv_write_window(const void* k, const void* v, int64_t start, int64_t n, void* k_cache,
                        void* v_cache, int32_t B, int64_t Lmax, int32_t Hkv, int32_t d,
                        double base, const wpa_rope_t* rope, double cache_alpha, int32_t dtype,
                        void* stream);
int wpa_decode_window(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* kv_len, void* out, float* lse, int32_t B, int64_t Lmax,
                      int32_t Hq, int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope,
                      double cache_alpha, double alpha, float scale, int32_t dtype,
                      int32_t out_dtype, unsigned long long* term_count, int32_t chunk_keys,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * Paged decode caches (serving with a block table: the ragged-batch path around the decode
 * step; ATFlash abstract: the window ported into a serving decode kernel).  Keys and values
 * live in a pool of pages of page_size tokens each; the token range [i*page_size,
 * (i+1)*page_size) of sequence b is page block_table[b*max_pages + i] of the pool.  The
 * arithmetic is that of the contiguous caches (same rotation, same layouts inside a page):
 * a step on a paged cache gives bit-identical results to the same step on a contiguous cache
 * holding the same tokens with Lmax = max_pages * page_size.
 *   page_size    a power of two in [32, 65536] (a 32-token tile never straddles pages);
 *                max_pages * page_size < 2^31.
 *   k_pool, v_pool  num_pages pages of wpa_kv_page_bytes(Hkv, d, page_size) bytes each,
 *                16-byte aligned.  K page: [Hkv][d/16][page_size][16] IEEE half (rotated,
 *                pair-blocked); V page: [Hkv][page_size/8][d][8] bf16.  Caller-owned.
 *   block_table  int32 device [B][max_pages], entries in [0, num_pages) for every page a
 *                sequence's tokens reach (others are not read).  Entries outside that range
 *                break the contract; the kernels clamp them so that no access leaves the pool.
 *                Pages may be shared or reused by the caller as it sees fit: writes go where
 *                the table says.
 *   wpa_kv_page_bytes   bytes of one K page (one V page has the same size); 0 for invalid
 *                arguments (d not 64 or 128, page_size not a power of two in range).
 *   wpa_kv_write_paged  as wpa_kv_write_ex for tokens start .. start+n-1 of every sequence
 *                (start + n <= max_pages * page_size); a partly written V octet keeps its
 *                other tokens.  For one sequence, pass B = 1 and its block-table row.
 *   wpa_decode_paged    as wpa_decode_ex on the pools, kv_len clamped into
 *                [0, max_pages*page_size] (the table's reach).  Workspace:
 *                wpa_decode_workspace_bytes(B, max_pages*page_size, Hq, Hkv, d, chunk_keys).
 *   wpa_prefill_paged   as wpa_prefill_cached on the pools (Lmax = max_pages * page_size),
 *                bit-identical to it on contiguous caches holding the same tokens, for every
 *                page_size the pools accept (a 128-key tile spans up to 4 pages of 32).
 */
size_t wpa_kv_page_bytes(int32_t Hkv, int32_t d, int32_t page_size);
int wpa_kv_write_paged(const void* k, const void* v, int64_t start, int64_t n, void* k_pool,
                       void* v_pool, const int32_t* block_table, int32_t num_pages, int32_t B,
                       int32_t max_pages, int32_t page_size, int32_t Hkv, int32_t d, double base,
                       const wpa_rope_t* rope, int32_t dtype, void* stream);
int wpa_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, int32_t num_pages, const int32_t* kv_len,
                     const int32_t* q_pos, void* out, float* lse, int32_t B, int32_t max_pages,
                     int32_t page_size, int32_t Hq, int32_t Hkv, int32_t d, double base,
                     const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                     int32_t out_dtype, unsigned long long* term_count, int32_t chunk_keys,
                     void* workspace, size_t ws_bytes, void* stream);
int wpa_prefill_paged(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, int32_t num_pages, const int32_t* kv_len,
                      void* out, float* lse, int32_t B, int32_t Nq, int32_t max_pages,
                      int32_t page_size, int32_t Hq, int32_t Hkv, int32_t d, double base,
                      const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                      int32_t out_dtype, unsigned long long* term_count, void* stream);
/* Varlen chunked prefill on paged caches: wpa_prefill_cached_varlen's arguments with the
 * pools and block table of wpa_prefill_paged. */
int wpa_prefill_paged_varlen(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, int32_t num_pages, const int32_t* cu_q,
                             const int32_t* kv_len, void* out, float* lse, int32_t B,
                             int32_t max_q, int32_t max_pages, int32_t page_size, int32_t Hq,
                             int32_t Hkv, int32_t d, double base, const wpa_rope_t* rope,
                             double alpha, float scale, int32_t dtype, int32_t out_dtype,
                             unsigned long long* term_count, void* stream);

/*
 * Chunked prefill with key splits (the operation of wpa_prefill_cached: WavePrune original,
 * the pair-wise window; ATFlash abstract: one window test per pair and distance).  A short
 * chunk has too few row blocks to fill the GPU; here the key tiles each row block attends to
 * are divided among up to `splits` workgroups, each of which writes its rows' output over its
 * own share of the keys, normalised by its own softmax sum, and that sum's log; a second
 * kernel merges the shares with weights exp(share's lse - row lse).  Rows whose keys fit one
 * 128-key tile are written directly.  The result is the same attention up to fp32 rounding
 * order (the merge adds one fp32 rescale per share).
 *   One entry point for the four cached forms:
 *   block_table  NULL: dense caches (k_cache, v_cache, Lmax as for wpa_prefill_cached);
 *                else paged pools (num_pages, page_size as for wpa_prefill_paged, with
 *                Lmax = max_pages * page_size, a multiple of page_size).
 *   cu_q         NULL: Nq queries per sequence (out [B][Nq][Hq][d], lse [B][Hq][Nq]); else the
 *                varlen packing of wpa_prefill_cached_varlen with max_q = Nq.
 *   splits       0: the launch chooses (about two workgroups per compute unit on the current
 *                device, at most 16, within the workspace's room; with no room for two, or no
 *                workspace, it launches as wpa_prefill_cached does); 1: no key splits; 2..16:
 *                exactly that many (a workspace of at least
 *                wpa_prefill_cached_workspace_bytes(..., splits) bytes, else WPA_ERR_INVALID).
 *   workspace    device, 16-byte aligned, caller-owned, ws_bytes long (NULL with 0: none);
 *                overwritten.  Calls that overlap in time must not share it.
 *   Other arguments, their layouts and errors as for wpa_prefill_cached.
 * wpa_prefill_cached_workspace_bytes: bytes for `splits` splits (0: the count the launch
 * would choose on the current device) of B sequences of Nq queries: splits * B * Nq * Hq *
 * (d + 1) * 4, and 0 when no split is taken or for invalid arguments.
 */
size_t wpa_prefill_cached_workspace_bytes(int32_t B, int32_t Nq, int32_t Hq, int32_t Hkv,
                                          int32_t d, int32_t splits);
int wpa_prefill_cached_ex(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int32_t num_pages, int32_t page_size,
                          const int32_t* cu_q, const int32_t* kv_len, void* out, float* lse,
                          int32_t B, int32_t Nq, int64_t Lmax, int32_t Hq, int32_t Hkv, int32_t d,
                          double base, const wpa_rope_t* rope, double alpha, float scale,
                          int32_t dtype, int32_t out_dtype, unsigned long long* term_count,
                          int32_t splits, void* workspace, size_t ws_bytes, void* stream);

/*
 * Backward of the causal windowed prefill, for training with the window (WavePrune, "What the
 * paper found": models trained from scratch with each pair's term limited to its first
 * rotation period).  Given the forward's inputs q, k, v (pre-RoPE, bf16, [B][N][H][d]), its
 * output `out` [B][N][Hq][d] (out_dtype) and `lse` [B][Hq][N] (fp32, natural log, as
 * wpa_prefill writes them), and dout = dL/dout [B][N][Hq][d] (bf16), writes the gradients of
 * L with respect to the pre-RoPE q, k and v:
 *   dq [B][N][Hq][d], dk and dv [B][N][Hkv][d] (grad_dtype: WPA_BF16 or WPA_FP32)
 * with P recomputed under the same window, dl = P (dout.v - dout.out), dq' = scale sum_c dl k'
 * and dk' = scale sum_r dl q' restricted to the pairs kept at each distance, and dq, dk the
 * rotated gradients rotated back by minus their position's angle.  Positions are token indices
 * (the one-shot prefill's default).  Rotated q and k are rounded to IEEE half, dl to half and P
 * to bf16 for the MFMA products, which accumulate in fp32.  rope: pair layout and one shared
 * frequency table (per-head tables: WPA_ERR_UNSUPPORTED).  dtype must be WPA_BF16
 * (WPA_ERR_UNSUPPORTED otherwise).  workspace: 256-byte aligned, at least
 * wpa_prefill_backward_workspace_bytes(B, N, Hq, Hkv, d) bytes (it holds the rotated and
 * transposed operands and per-q-head dk/dv partials).
 */
size_t wpa_prefill_backward_workspace_bytes(int32_t B, int64_t N, int32_t Hq, int32_t Hkv,
                                            int32_t d);
int wpa_prefill_backward(const void* q, const void* k, const void* v, const void* out,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         int32_t B, int64_t N, int32_t Hq, int32_t Hkv, int32_t d, double base,
                         const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                         int32_t out_dtype, int32_t grad_dtype, void* workspace, size_t ws_bytes,
                         void* stream);

/*
 * wpa_decode_ex without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Arguments
 * are those of wpa_decode_ex minus workspace and ws_bytes; results are bit-identical to it
 * with the same chunk_keys.  The split-KV partials go to a scratch array the library holds
 * in device memory, 16 MiB per GPU, kept until the process ends: a call whose partials need
 * more (wpa_decode_workspace_bytes(B, Lmax, Hq, Hkv, d, chunk_keys) > 16 MiB) returns
 * WPA_ERR_UNSUPPORTED before enqueueing anything.  The call allocates nothing.  Every call on
 * one GPU uses that GPU's array: calls that may run concurrently on one GPU (different
 * streams without ordering between them) race on it.  The first call on a device looks up
 * the array's address on that device (it must be the current device).
 */
int wpa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* kv_len, const int32_t* q_pos, void* out, float* lse,
                       int32_t B, int64_t Lmax, int32_t Hq, int32_t Hkv, int32_t d, double base,
                       const wpa_rope_t* rope, double alpha, float scale, int32_t dtype,
                       int32_t out_dtype, unsigned long long* term_count, int32_t chunk_keys,
                       void* stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* wpa_last_error(void);

/*
 * Debug mode, for finding a caller's mistakes; off by default.  It starts on when the
 * environment variable WPA_DEBUG is set to anything but "0" when first consulted;
 * wpa_set_debug(1) / (0) switches it for the process, and wpa_set_debug(-1) only reports the
 * state.  Returns the previous state (0 or 1).
 * In debug mode every entry point that enqueues work also, before enqueueing anything:
 *   - checks that each device buffer it will read or write lies inside one allocation of
 *     the HIP runtime with at least the bytes the call needs from that pointer;
 *   - reads back, after the stream drains, the device-resident values the kernels otherwise
 *     trust, and checks them.  Those are positions (non-negative, non-decreasing per
 *     sequence), per-head frequency tables (finite, > 0, non-increasing), chunked prefill's
 *     kv_len (in [q_b, Lmax]) and cu_q (non-decreasing from >= 0, q_b <= max_q), and every
 *     block-table entry a call will use (in [0, num_pages));
 *   - returns WPA_ERR_INVALID with a message naming the buffer or value, enqueueing nothing.
 * After enqueueing, it waits for the stream and returns WPA_ERR_HIP if a kernel failed,
 * so that a fault is reported by the call that caused it.  Debug mode synchronises, and so
 * it is slow; results are bit-identical to normal mode.
 */
int wpa_set_debug(int32_t on);

#ifdef __cplusplus
}
#endif

#endif /* WPA_H */
