/*
 * lte.h -- C ABI of the Learnable Token Eviction (LTE) sparse-attention layer
 * for AMD MI355X (gfx950).
 *
 * Source of the method: "Alleviating Forgetfulness of Linear Attention by
 * Hybrid Sparse Attention and Contextualized Learnable Token Eviction"
 * (He & Garner, arXiv 2510.20787), summary page:
 *   - Figure 2 caption: attention sink of size s, sliding window of size w,
 *     a small convolutional network over each token's nearby past and future
 *     keys/values whose output r_{j,h} (one number per token and head) rates
 *     how well worth keeping the token is; eviction decided when a KV pair
 *     leaves the window, and the resulting per-head "A-plus-column" sparsity
 *     pattern.
 *   - Figure 3 caption: cache layout with a circular window segment and an
 *     out-of-window segment of capped capacity for retained KVs and the sink;
 *     scoring batched and deferred as late as possible.
 *   - Abstract / TL;DR: a limited set of KV pairs per head under a budget,
 *     constant time and space per step.
 * Readings this library takes where the page is silent:
 *   - window of query i = positions [i-w+1, i]; token j leaves at step j+w;
 *   - sink = positions [0, s), always visible, never scored or evicted;
 *   - scores and retention are per KV head (shared by the query heads of a
 *     GQA group, head h uses KV head h / (Hq/Hkv));
 *   - CNN per KV head: conv1d(2D -> hidden, kernel 3, zero pad 1) over
 *     concat(k, v) channels (keys first), GELU (erf evaluated by Abramowitz
 *     and Stegun's formula 7.1.26, absolute error at most 1.5e-7),
 *     conv1d(hidden -> 1, kernel 3, zero pad 1), sigmoid; tap t reads
 *     offset t-1;
 *   - keep rule: a token j >= s is a candidate iff r_j > 0.5 (fp32); at most
 *     C are retained; on overflow the C best by (score descending, index
 *     ascending) stay; decisions are causal (query i sees the set built from
 *     the tokens that left the window by step i);
 *   - attention: softmax(q.k / sqrt(D)) over sink U window U retained.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are caller-owned DEVICE memory, contiguous,
 *     row-major.  bf16 tensors are passed as uint16_t bit patterns.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     legacy default stream) and never synchronises.  The library keeps no
 *     pointer after a call returns and holds no mutable global state, except
 *     the static device array of lte_decode_step_static (and its per-device
 *     address).
 *   - Arguments are validated on the host before any launch; a failing call
 *     returns a status and leaves memory untouched.  A failed launch returns
 *     LTE_ERR_HIP.  No C++ exception crosses this interface.
 *   - Sequences of a batch have equal length, except in lte_prefill_varlen,
 *     after which each sequence decodes from its own position.
 *   - Supported: head_dim in {64, 128}; q_heads / kv_heads in {1, 2, 4, 8,
 *     16}; kv_heads <= 128; hidden == 32; 5 <= window <= 32768;
 *     0 <= sink <= 256; 0 <= capacity <= 4096; 1 <= T <= 32768 tokens per
 *     prefill.
 */
#ifndef LTE_H
#define LTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
typedef enum {
    LTE_OK = 0,
    LTE_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad shape      */
    LTE_ERR_UNSUPPORTED = 2,   /* valid but outside the supported range above */
    LTE_ERR_STATE = 3,         /* cache not in a state that allows the call   */
    LTE_ERR_HIP = 4,           /* a HIP launch or copy failed                 */
    LTE_ERR_WORKSPACE = 5,     /* workspace smaller than lte_workspace_bytes  */
    LTE_ERR_SCRATCH = 6        /* more scratch than lte_decode_step_static's
                                  static array holds                          */
} lte_status;

/* Layer shape. sink = s, window = w, capacity = C of the method. */
typedef struct {
    int32_t batch;      /* B                                   */
    int32_t q_heads;    /* Hq                                  */
    int32_t kv_heads;   /* Hkv; Hq % Hkv == 0                  */
    int32_t head_dim;   /* D                                   */
    int32_t sink;       /* s                                   */
    int32_t window;     /* w                                   */
    int32_t capacity;   /* C, retained out-of-window KVs/head  */
    int32_t hidden;     /* width of the scoring CNN (32)       */
} lte_config;

/* Scoring-CNN parameters, device fp32, one set per KV head (Figure 2's
 * "CNN stack").  w1 [Hkv][hidden][2D][3], b1 [Hkv][hidden],
 * w2 [Hkv][hidden][3], b2 [Hkv].  Input channel order: the D key channels,
 * then the D value channels of the same token. */
typedef struct {
    const float *w1, *b1, *w2, *b2;
} lte_cnn;

/* Byte offsets of the sections of a cache blob (Figure 3's layout).  Every
 * section starts on a 256-byte boundary.  S = sink + capacity + window slots
 * per (batch, KV head):
 *   k, v        bf16  [B][Hkv][S][D]: slots [0, s) sink, [s, s+C) retained
 *                     segment (compacted, first count[b][g] valid),
 *                     [s+C, s+C+w) ring (token j in slot s+C+(j mod w))
 *   ret_idx     int32 [B][Hkv][C]  token index of each retained slot
 *   ret_score   fp32  [B][Hkv][C]  its score
 *   ring_score  fp32  [B][Hkv][w]  score of the token in each ring slot,
 *                                  NaN while not yet scored
 *   count       int32 [B][Hkv]     valid retained slots
 *   pos         int64 [B][Hkv]     tokens ingested so far (equal over the
 *                                  heads of a sequence)
 *   next_unscored int64 [B][Hkv]   oldest token still lacking a score
 *   flags       int32 [B][Hkv]     bit 0: a token left the window unscored
 *   weak        int32 [B][Hkv]     slot of the weakest retained entry (lowest
 *                                  score, then highest index) while the
 *                                  segment is full, else -1
 *   nx_slot     int32 [B][Hkv]     decision for the token that leaves at the
 *                                  next ingest (token pos-w): the segment
 *                                  slot it takes, -1 if it is not kept, -2
 *                                  if it would leave unscored
 *   nx_score    fp32  [B][Hkv]     that token's score
 *   arrive      int32 [B][Hkv]     split arrivals of the decode call in
 *                                  progress; 0 between calls
 *   total       size of the blob in bytes                                */
typedef struct {
    size_t k, v, ret_idx, ret_score, ring_score, count, pos, next_unscored, flags, weak, nx_slot,
        nx_score, arrive, total;
} lte_cache_layout;

/* Byte offsets inside a prefill workspace for T tokens (intermediates that
 * the tests read back):
 *   scores  fp32  [B][Hkv][T]  retention score of every token
 *   rank    int32 [B][Hkv][T]  position of token j in the order (score desc,
 *                              index asc) among candidates; 0 for every
 *                              candidate when at most C exist; INT32_MAX for
 *                              a non-candidate
 *   thr     int32 [B][Hkv][T]  thr[m]: token j <= m with rank[j] <= thr[m]
 *                              is retained after the tokens 0..m have left
 *                              the window, i.e. R_{m+w} of the method
 *   ncand   int32 [B][Hkv]     number of candidates                        */
typedef struct {
    size_t scores, rank, thr, ncand, total;
} lte_workspace_layout;

/* Human-readable text of a status code (static storage). */
const char* lte_status_string(int status);

/* ABI version, currently 1. */
int lte_version(void);

/* Checks a configuration; LTE_OK if every entry point accepts it. */
int lte_check_config(const lte_config* cfg);

/* Cache blob size and section offsets for cfg (0 / error on a bad cfg). */
size_t lte_cache_bytes(const lte_config* cfg);
int lte_cache_get_layout(const lte_config* cfg, lte_cache_layout* out);

/* Workspace needed by a T-token prefill and by every decode call.  The
 * workspace is scratch: its contents are undefined between calls, except
 * that the views of lte_workspace_get_layout hold the last prefill's
 * intermediates until the next prefill into the same workspace.  Decode
 * calls use only the first lte_workspace_bytes(cfg, 0) bytes, which lie
 * before those views. */
size_t lte_workspace_bytes(const lte_config* cfg, int64_t T);
int lte_workspace_get_layout(const lte_config* cfg, int64_t T, lte_workspace_layout* out);

/* Resets a cache to the empty state: pos = 0, count = 0, every ring score
 * NaN, flags 0, weak -1, nx_slot -1, arrive 0.  K/V slots are left as they
 * are (never read while invalid). */
int lte_cache_init(const lte_config* cfg, void* cache, void* stream);

/* ---------------------------------------------------------------------------
 * Prefill of a T-token prompt: score, select, attend, build the cache.
 *   q   bf16 [B][T][Hq][D];  k, v bf16 [B][T][Hkv][D]
 *   cnn scoring-CNN parameters, or NULL when score_override is given
 *   score_override  fp32 [B][Hkv][T] explicit scores (the "artificial KV
 *       cache" of Figure 4(a)), or NULL to run the CNN
 *   cache  lte_cache_bytes(cfg) bytes, or NULL to skip building the cache
 *   workspace  lte_workspace_bytes(cfg, T) bytes
 *   out bf16 [B][T][Hq][D], o_i for every query row
 * The cache afterwards holds the sink, R_{T-1} in the retained segment, the
 * last w tokens in the ring, pos = T and next_unscored = max(T-2, s): the
 * scores of tokens T-2 and T-1 still lack their right neighbours.
 * ------------------------------------------------------------------------- */
int lte_prefill(const lte_config* cfg, int64_t T,
                const uint16_t* q, const uint16_t* k, const uint16_t* v,
                const lte_cnn* cnn, const float* score_override,
                void* cache, void* workspace, size_t workspace_bytes,
                uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * Prefill of a batch whose prompts differ in length.  Nothing in the method
 * couples the sequences of a batch (scores, selection and cache are per
 * sequence and head), so each is the prompt of its own length.  Arguments and
 * layouts are those of lte_prefill
 * with T the padded length, plus
 *   seq_lens  device int32 [B]: sequence b's prompt is rows [0, T_b) of its
 *       [T] rows, T_b = seq_lens[b] clamped to [1, T]
 * Rows >= T_b of q, k, v (and of score_override) are never read; rows >= T_b
 * of out are not written.  Sequence b's result is the one lte_prefill gives
 * for its first T_b rows alone: its cache holds pos = T_b and
 * next_unscored = max(T_b - 2, s), so later decode calls step every sequence
 * from its own position.  The workspace views then hold sequence b's
 * intermediates at indices < T_b only.
 * ------------------------------------------------------------------------- */
int lte_prefill_varlen(const lte_config* cfg, int64_t T, const int32_t* seq_lens,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const lte_cnn* cnn, const float* score_override,
                       void* cache, void* workspace, size_t workspace_bytes,
                       uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * Chunked prefill: n new tokens per sequence appended to a cache at any
 * position (after a prefill, decode steps or earlier chunks), their outputs
 * computed, the cache advanced to pos + n.  The result is that of one prefill
 * over the whole history (up to rounding), because the cache's segment is the
 * top-C of every candidate that left the window and top-C under the strict
 * order (score desc, index asc) continues over a union (Figure 2 caption of
 * the learnable-eviction paper: decisions from scores at window exit, at most
 * C kept).  Tokens still unscored in the ring get their scores now, those at
 * the chunk's end keep provisional ones (next_unscored = max(pos + n - 2, s)).
 *   q   bf16 [B][n][Hq][D];  k, v bf16 [B][n][Hkv][D]: the new tokens
 *   cnn scoring-CNN parameters (required)
 *   cache  lte_cache_bytes(cfg) bytes in any state reached by this library
 *   workspace  lte_chunk_workspace_bytes(cfg, n) bytes; its first
 *       lte_workspace_bytes(cfg, s + C + w + n) bytes hold the views of
 *       lte_workspace_get_layout for T = s + C + w + n over the call's
 *       extended sequence (sink, segment sorted by token, ring, chunk)
 *   out bf16 [B][n][Hq][D]
 * Sequences may stand at different positions.  s + C + w + n <= 32768.
 * ------------------------------------------------------------------------- */
size_t lte_chunk_workspace_bytes(const lte_config* cfg, int64_t n);
int lte_prefill_chunk(const lte_config* cfg, int64_t n,
                      const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const lte_cnn* cnn, void* cache, void* workspace,
                      size_t workspace_bytes, uint16_t* out, void* stream);

/* The four stages lte_prefill runs, in order, exposed for timing and tests.
 * Each reads and writes the workspace views described above.  Once
 * lte_prefill_select has completed, lte_prefill_attend and
 * lte_prefill_build_cache only read the workspace (scores, rank, thr), k and v,
 * and write disjoint outputs (out; cache), so a caller may run them
 * concurrently on two streams. */
int lte_prefill_score(const lte_config* cfg, int64_t T, const uint16_t* k, const uint16_t* v,
                      const lte_cnn* cnn, void* workspace, size_t workspace_bytes, void* stream);
int lte_prefill_select(const lte_config* cfg, int64_t T, const float* score_override,
                       void* workspace, size_t workspace_bytes, void* stream);
int lte_prefill_attend(const lte_config* cfg, int64_t T, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, void* workspace, size_t workspace_bytes,
                       uint16_t* out, void* stream);
int lte_prefill_build_cache(const lte_config* cfg, int64_t T, const uint16_t* k,
                            const uint16_t* v, void* workspace, size_t workspace_bytes,
                            void* cache, void* stream);
/* The same cache, bit for bit, with the row copy (about 2 x 67 MB at B=32,
 * C=w=512, D=128) spread over 32 workgroups that each walk many slot groups:
 * it draws little HBM bandwidth at a time, for callers that run it on a second
 * stream beside lte_prefill_attend, whose latency-bound phases a full-rate copy
 * slows.  On its own it takes several times longer than lte_prefill_build_cache.
 * Arguments, ownership and errors as lte_prefill_build_cache. */
int lte_prefill_build_cache_background(const lte_config* cfg, int64_t T, const uint16_t* k,
                                       const uint16_t* v, void* workspace,
                                       size_t workspace_bytes, void* cache, void* stream);

/* ---------------------------------------------------------------------------
 * Ingest one token per sequence (position t = pos).  Figure 2 caption of the
 * learnable-eviction paper: a token is kept or dropped when it leaves the
 * sliding window, by its retention score, with at most C kept per head;
 * Figure 3 caption: the window is a circular segment of the cache, retained
 * tokens sit in a capped out-of-window segment, and scoring is batched and
 * put off until the last step at which the CNN's inputs are still cached.
 *   1. the token t-w leaves ring slot t mod w; if t-w >= s and its score is
 *      > 0.5 it enters the retained segment, displacing the weakest entry
 *      (lowest score, then highest index) when the segment already holds C
 *      and the newcomer ranks above it;
 *   2. k_t, v_t (bf16 [B][Hkv][D]) are written into that ring slot (and into
 *      sink slot t when t < s);
 *   3. deferred batched scoring: when t = u + w - 3 for the oldest unscored
 *      token u, tokens u .. t-2 are scored from the ring, the last moment at
 *      which their left neighbour u-2 is still there;
 *   4. pos = t + 1.
 * cnn is required (it is read only on steps that score).
 * ------------------------------------------------------------------------- */
int lte_score_evict(const lte_config* cfg, const lte_cnn* cnn, const uint16_t* k_t,
                    const uint16_t* v_t, void* cache, void* stream);

/* Attention of the newest token's queries q_t (bf16 [B][Hq][D]) over the
 * cache: sink U retained segment U ring, out_t bf16 [B][Hq][D] (Figure 2
 * caption: each head attends to its sink, its window and the tokens it kept;
 * Abstract: so a decode step costs the same at any position).  Requires
 * pos >= 1 (LTE_ERR_STATE is not detectable on the host: a cache with
 * pos == 0 yields zeros).  The cache's arrive words are used during the
 * call and left at 0; nothing else in the cache changes. */
int lte_decode_attend(const lte_config* cfg, const uint16_t* q_t, void* cache,
                      void* workspace, size_t workspace_bytes, uint16_t* out_t, void* stream);

/* One decode step, with the result of lte_score_evict followed by
 * lte_decode_attend, in one launch (Figure 3 caption: the step reads and
 * updates the cache of Figure 3's layout in place, at constant cost per
 * token): the splits of the cache (64 slots each)
 * are read in their pre-step state with the new token and the segment slot
 * the leaving token takes substituted; the last split of a (batch, KV head)
 * to finish merges the partial softmax sums in split order and then updates
 * the cache.  Calls that use one cache must be ordered on one stream. */
int lte_decode_step(const lte_config* cfg, const uint16_t* q_t, const uint16_t* k_t,
                    const uint16_t* v_t, const lte_cnn* cnn, void* cache, void* workspace,
                    size_t workspace_bytes, uint16_t* out_t, void* stream);

/* lte_decode_step without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): identical results, bit for bit.  The split partials that
 * lte_decode_step keeps in the workspace live instead in a static device array
 * of 5 MiB (every supported shape needs at most about 4.3 MB; a larger need
 * returns LTE_ERR_SCRATCH), one per device, whose address is looked up on the
 * first call on each device.  The call allocates nothing.  Calls on one device
 * share that array: calls that overlap in time on one device race (serialise
 * them on one stream).  Nothing in the array needs clearing between calls:
 * every split writes its partial before the last one reads it. */
int lte_decode_step_static(const lte_config* cfg, const uint16_t* q_t, const uint16_t* k_t,
                           const uint16_t* v_t, const lte_cnn* cnn, void* cache,
                           uint16_t* out_t, void* stream);

/* Copies the cache's bookkeeping into caller device buffers (parity, resume):
 * the out-of-window segment of Figure 3's caption (which tokens it holds and
 * their retention scores), its fill and the position.
 * ret_idx int32 [B][Hkv][C], ret_score fp32 [B][Hkv][C], count int32
 * [B][Hkv], pos int64 [B][Hkv].  Slots x >= count hold unspecified values;
 * slots below count are in no particular order.  Plain device-to-device
 * copies on the stream.  Any pointer may be NULL to skip it. */
int lte_cache_export(const lte_config* cfg, const void* cache, int32_t* ret_idx,
                     float* ret_score, int32_t* count, int64_t* pos, void* stream);

/* ===========================================================================
 * Linear-attention layer of the hybrid ("Sparse Linear Attention: Viewing SWA
 * from the Perspective of Linear Attention", section "Background: Linear
 * attention"):  S_t = S_{t-1} A_t + v_t k_t^T,  o_t = S_t q_t, with
 * A_t = a_t I: one decay a_t = exp(log_a) in [0, 1] per head and step (1 is
 * naive linear attention; log_a below -80 acts as -80, a reset).  No scaling
 * or feature map of q and k.  S is D x D per (batch, head), fp32.
 * ========================================================================= */
typedef struct {
    int32_t batch;      /* B                               */
    int32_t heads;      /* H (q, k and v alike)            */
    int32_t head_dim;   /* D in {64, 128}                  */
} lte_linear_config;

int lte_linear_check_config(const lte_linear_config* cfg);
/* Bytes of the states of all (batch, head): B * H * D * D * 4. */
size_t lte_linear_state_bytes(const lte_linear_config* cfg);

/* The layer over T tokens (1 <= T <= 2^22).
 *   q, k, v  bf16 [B][T][H][D];  log_a fp32 [B][T][H]
 *   state_in  fp32 [B][H][D][D] (S[value dim][key dim]) the state before the
 *       first token, or NULL for zero; may be the same buffer as state_out
 *   state_out fp32 [B][H][D][D] the state after the last token
 *   out  bf16 [B][T][H][D] */
int lte_linear_prefill(const lte_linear_config* cfg, int64_t T,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const float* log_a, const float* state_in, float* state_out,
                       uint16_t* out, void* stream);

/* One token: q_t, k_t, v_t bf16 [B][H][D], log_a_t fp32 [B][H]; state fp32
 * [B][H][D][D] updated in place; out_t bf16 [B][H][D]. */
int lte_linear_decode_step(const lte_linear_config* cfg, const uint16_t* q_t,
                           const uint16_t* k_t, const uint16_t* v_t, const float* log_a_t,
                           float* state, uint16_t* out_t, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LTE_H */
