// Internal declarations shared by the HIP sources of liblte.so.
//
// Layout arithmetic (cache blob and workspace), vector types for the gfx950
// MFMA builtins, and the host-side launchers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lte.h"

namespace lte {

// ---------------------------------------------------------------------------
// vector types
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHidden = 32;         // scoring-CNN width
constexpr int kMaxSink = 256;
constexpr int kMaxCapacity = 4096;
constexpr int64_t kMaxT = 32768;     // the selection sort keeps <= 32 keys per thread
constexpr int64_t kMaxLinearT = int64_t(1) << 22;   // linear layer: tokens per call
constexpr int32_t kNotCand = 0x7fffffff;   // rank of a non-candidate
constexpr int32_t kAllPass = 0x7ffffffe;   // thr when every candidate is kept

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by 1, 2, 4
// and 8 within each row of 16 lanes, then each row's last lane is added into the rows
// after it (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3).  Lanes
// whose source is out of range add the 0 passed as the old value.
__device__ __forceinline__ int wave_incl_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
    return x;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Length of sequence b of a prefill: seq_lens[b] clamped to [1, T], or T for
// every sequence when there is no length array.
__device__ __forceinline__ int seq_len_of(const int32_t* seq_lens, int b, int T) {
    if (seq_lens == nullptr) return T;
    const int n = seq_lens[b];
    return n < 1 ? 1 : (n > T ? T : n);
}

// Plain copy of lte_config with derived sizes.
struct Shape {
    int B, Hq, Hkv, D, s, w, C, G, S;   // S = s + C + w cache slots per (b, g)
};

inline Shape make_shape(const lte_config& c) {
    Shape sh;
    sh.B = c.batch; sh.Hq = c.q_heads; sh.Hkv = c.kv_heads; sh.D = c.head_dim;
    sh.s = c.sink; sh.w = c.window; sh.C = c.capacity;
    sh.G = c.kv_heads > 0 ? c.q_heads / c.kv_heads : 0;
    sh.S = c.sink + c.capacity + c.window;
    return sh;
}

// ---------------------------------------------------------------------------
// cache blob layout
// ---------------------------------------------------------------------------
inline lte_cache_layout cache_layout(const Shape& sh) {
    lte_cache_layout L{};
    size_t bg = size_t(sh.B) * sh.Hkv;
    size_t off = 0;
    L.k = off; off = align256(off + bg * sh.S * sh.D * 2);
    L.v = off; off = align256(off + bg * sh.S * sh.D * 2);
    L.ret_idx = off; off = align256(off + bg * size_t(sh.C) * 4);
    L.ret_score = off; off = align256(off + bg * size_t(sh.C) * 4);
    L.ring_score = off; off = align256(off + bg * size_t(sh.w) * 4);
    L.count = off; off = align256(off + bg * 4);
    L.pos = off; off = align256(off + bg * 8);
    L.next_unscored = off; off = align256(off + bg * 8);
    L.flags = off; off = align256(off + bg * 4);
    L.weak = off; off = align256(off + bg * 4);
    L.nx_slot = off; off = align256(off + bg * 4);
    L.nx_score = off; off = align256(off + bg * 4);
    L.arrive = off; off = align256(off + bg * 4);
    L.total = off;
    return L;
}

// Device-side view of a cache blob.
struct CacheView {
    uint16_t* k;           // [B][Hkv][S][D]
    uint16_t* v;
    int32_t* ret_idx;      // [B][Hkv][C]
    float* ret_score;      // [B][Hkv][C]
    float* ring_score;     // [B][Hkv][w]
    int32_t* count;        // [B][Hkv]
    int64_t* pos;          // [B][Hkv]
    int64_t* next_unscored;
    int32_t* flags;
    int32_t* weak;         // [B][Hkv] weakest slot of a full segment, else -1
    int32_t* nx_slot;      // [B][Hkv] decision for the next leaving token
    float* nx_score;       // [B][Hkv] its score
    int32_t* arrive;       // [B][Hkv] decode split arrivals, 0 between calls
};

// Per-call data of a chunked prefill (device arrays in the workspace): the
// extended sequence of each batch entry and its row -> token map.
struct ChunkView {
    int32_t* ext_len;      // [B]  rows of the extended sequence
    int32_t* q_lo;         // [B]  first chunk row
    int32_t* tok_off;      // [B]  token = row + tok_off past the segment rows
    int32_t* warm;         // [B]  1: sink/segment/ring layout, 0: the whole history
    int32_t* score_lo;     // [B][Hkv] first row whose score is computed
    int32_t* seg_tok;      // [B][Hkv][C] tokens of the sorted segment rows
    int32_t* seg_slot;     // [B][Hkv][C] their cache slots - s, -1 past count
    int32_t* seg_row;      // [B][Hkv][C] rows of the new segment entries
};

inline CacheView cache_view(const Shape& sh, void* base) {
    lte_cache_layout L = cache_layout(sh);
    char* p = static_cast<char*>(base);
    CacheView c;
    c.k = reinterpret_cast<uint16_t*>(p + L.k);
    c.v = reinterpret_cast<uint16_t*>(p + L.v);
    c.ret_idx = reinterpret_cast<int32_t*>(p + L.ret_idx);
    c.ret_score = reinterpret_cast<float*>(p + L.ret_score);
    c.ring_score = reinterpret_cast<float*>(p + L.ring_score);
    c.count = reinterpret_cast<int32_t*>(p + L.count);
    c.pos = reinterpret_cast<int64_t*>(p + L.pos);
    c.next_unscored = reinterpret_cast<int64_t*>(p + L.next_unscored);
    c.flags = reinterpret_cast<int32_t*>(p + L.flags);
    c.weak = reinterpret_cast<int32_t*>(p + L.weak);
    c.nx_slot = reinterpret_cast<int32_t*>(p + L.nx_slot);
    c.nx_score = reinterpret_cast<float*>(p + L.nx_score);
    c.arrive = reinterpret_cast<int32_t*>(p + L.arrive);
    return c;
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
// Selection works on rank blocks of `rbs` ranks; one cumulative position
// bitmap ("snapshot") per rank block.
inline int select_rbs(int64_t T) {
    int64_t f = (T + 16383) / 16384;
    return int(64 * (f < 1 ? 1 : f));
}
inline int64_t select_nsnap_max(int64_t T) {
    int rbs = select_rbs(T);
    return (T + rbs - 1) / rbs;
}
inline int64_t select_words(int64_t T) { return (T + 31) / 32; }

// Per-(b, g) scratch of the selection kernel, in 4-byte words.
inline size_t select_scratch_words(int64_t T) {
    int64_t Tp = (T + 63) & ~int64_t(63);
    return size_t(4 * Tp) + align256(size_t(2 * select_nsnap_max(T) * select_words(T)) * 4) / 4;
}

// Decode split-K.  A workgroup (8 waves) attends over a contiguous range of one
// (b, g)'s visible rows; with at least 256 (b, g) pairs there is one workgroup
// per pair and the waves merge in LDS, otherwise each pair is split over up to
// 256 / (B * Hkv) workgroups of at least 128 slots (so that every compute unit
// reads), merged by the last to finish.
constexpr int kDecodeWaves = 8;
inline int decode_nsplit(const Shape& sh) {
    const long bg = long(sh.B) * sh.Hkv;
    if (bg >= 256) return 1;
    const long by_grid = (256 + bg - 1) / bg;
    const long by_rows = (sh.S + 127) / 128;
    const long n = by_grid < by_rows ? by_grid : by_rows;
    return int(n < 1 ? 1 : n);
}
// Floats per split partial: o [G][D], then (max, sum) per head, padded to 16 bytes.
__host__ __device__ constexpr int decode_part_floats(int G, int D) {
    return G * D + ((2 * G + 3) & ~3);
}

// Bytes of the decode split partials (the only workspace a decode call uses).
inline size_t decode_part_bytes(const Shape& sh) {
    return align256(size_t(sh.B) * sh.Hkv * size_t(decode_nsplit(sh)) *
                    decode_part_floats(sh.G, sh.D) * 4);
}
// Size of the static device array that holds them for lte_decode_step_static;
// every supported shape needs at most about 4.3 MB (fewer than 256 (b, g) pairs
// times at most 256 / (B Hkv) + 1 splits: at most 510 partials of 8320 bytes).
constexpr size_t kStaticScratchBytes = size_t(5) << 20;

struct WsLayout {
    size_t scores, rank, thr, ncand, select_scratch, dec_part, total;
};

inline WsLayout ws_layout(const Shape& sh, int64_t T) {
    // decode partials first: a decode call never overwrites a prefill's views
    WsLayout W{};
    size_t bg = size_t(sh.B) * sh.Hkv;
    size_t off = 0;
    W.dec_part = off;
    off = align256(off + bg * size_t(decode_nsplit(sh)) * decode_part_floats(sh.G, sh.D) * 4);
    W.scores = off; off = align256(off + bg * size_t(T) * 4);
    W.rank = off; off = align256(off + bg * size_t(T) * 4);
    W.thr = off; off = align256(off + bg * size_t(T) * 4);
    W.ncand = off; off = align256(off + bg * 4);
    W.select_scratch = off; off = align256(off + (T > 0 ? bg * select_scratch_words(T) * 4 : 0));
    W.total = off;
    return W;
}

// ---------------------------------------------------------------------------
// launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------
// Prefill launchers: T is the row count of every [B][T] tensor; seq_lens (device,
// [B], or null for T everywhere) gives each sequence's length.
// score_lo (device, [B][Hkv], or null): rows below it are left as they are.
hipError_t launch_score_prefill(const Shape& sh, int64_t T, const int32_t* seq_lens,
                                const int32_t* score_lo, const uint16_t* k, const uint16_t* v,
                                const lte_cnn& cnn, float* scores, hipStream_t st);
hipError_t launch_select(const Shape& sh, int64_t T, const int32_t* seq_lens, const float* scores,
                         int32_t* rank, int32_t* thr, int32_t* ncand, uint32_t* scratch,
                         hipStream_t st);
// q_lo (device, [B], or null): only rows >= q_lo[b] are queries; q and out are
// then [B][q_rows][Hq][D] with row i at i - q_lo[b].  ncand (device, [B][Hkv], or
// null): the selection's candidate counts; a (b, g) with none skips its rank scan.
hipError_t launch_attend_prefill(const Shape& sh, int64_t T, const int32_t* seq_lens,
                                 const int32_t* q_lo, int q_rows, const uint16_t* q,
                                 const uint16_t* k, const uint16_t* v, const int32_t* rank,
                                 const int32_t* thr, const int32_t* ncand, uint16_t* out,
                                 hipStream_t st);
// chunk (or null): the rows are a chunked prefill's extended sequence.  copy_wgs > 0
// caps the row copy's grid at that many workgroups (each then walks several slot
// groups); 0 gives every slot group its own workgroup.
hipError_t launch_build_cache(const Shape& sh, int64_t T, const int32_t* seq_lens,
                              const ChunkView* chunk, const uint16_t* k, const uint16_t* v,
                              const float* scores, const int32_t* rank, const int32_t* thr,
                              const CacheView& cache, hipStream_t st, int copy_wgs = 0);
// Workgroups of the row copy when the cache is built beside the prefill attention.
constexpr int kBackgroundCopyWgs = 32;
// Linear-attention layer: q, k, v [B][T][H][D] bf16, log_a [B][T][H] fp32,
// states [B][H][D][D] fp32 (S[dv][dk]); state_in may be null (zero state) and
// may equal state_out.
hipError_t launch_linear_prefill(int B, int H, int D, int64_t T, const uint16_t* q,
                                 const uint16_t* k, const uint16_t* v, const float* log_a,
                                 const float* state_in, float* state_out, uint16_t* out,
                                 hipStream_t st);
// One step: q, k, v [B][H][D], log_a [B][H], state in place, out [B][H][D].
hipError_t launch_linear_step(int B, int H, int D, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const float* log_a, float* state, uint16_t* out,
                              hipStream_t st);
// Extended sequence of a chunked prefill: layout data, known scores (into
// ext_scores [B][Hkv][Emax]) and K/V rows (ek, ev [B][Emax][Hkv][D]).
hipError_t launch_chunk_gather(const Shape& sh, int n, int Emax, const uint16_t* k,
                               const uint16_t* v, const CacheView& cache, const ChunkView& x,
                               float* ext_scores, uint16_t* ek, uint16_t* ev, hipStream_t st);
hipError_t launch_cache_init(const Shape& sh, const CacheView& cache, hipStream_t st);
// This device's address of the static split-partial array (kStaticScratchBytes),
// looked up once per device with that device current.
hipError_t static_scratch(float** out);
hipError_t launch_score_evict(const Shape& sh, const lte_cnn& cnn, const uint16_t* k_t,
                              const uint16_t* v_t, const CacheView& cache, hipStream_t st);
// ingest == false: attention over the cache as it is (lte_decode_attend);
// ingest == true: one fused decode step (lte_decode_step).
hipError_t launch_decode(const Shape& sh, bool ingest, const uint16_t* q_t, const uint16_t* k_t,
                         const uint16_t* v_t, const lte_cnn* cnn, const CacheView& cache,
                         float* part, uint16_t* out_t, hipStream_t st);

}  // namespace lte
