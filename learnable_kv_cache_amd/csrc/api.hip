// Host side of the C ABI declared in include/lte.h: argument validation,
// layout arithmetic and the launch order of the kernels.  Every check runs
// before the first launch; no C++ exception leaves this file.
#include <math.h>

#include "lte_internal.h"

using namespace lte;

namespace {

bool pow2_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

int check_cfg(const lte_config* cfg) {
    if (cfg == nullptr) return LTE_ERR_INVALID_ARG;
    const lte_config& c = *cfg;
    if (c.batch < 1 || c.q_heads < 1 || c.kv_heads < 1 || c.head_dim < 1) return LTE_ERR_INVALID_ARG;
    if (c.sink < 0 || c.capacity < 0 || c.window < 1 || c.hidden < 1) return LTE_ERR_INVALID_ARG;
    if (c.q_heads % c.kv_heads != 0) return LTE_ERR_INVALID_ARG;
    if (c.head_dim != 64 && c.head_dim != 128) return LTE_ERR_UNSUPPORTED;
    if (!pow2_group(c.q_heads / c.kv_heads)) return LTE_ERR_UNSUPPORTED;
    if (c.hidden != kHidden) return LTE_ERR_UNSUPPORTED;
    if (c.window < 5 || c.window > 32768) return LTE_ERR_UNSUPPORTED;
    if (c.sink > kMaxSink || c.capacity > kMaxCapacity) return LTE_ERR_UNSUPPORTED;
    // one sequence's K or V rows span T * kv_heads * head_dim * 2 bytes, addressed
    // with 32-bit offsets: kv_heads <= 128 keeps that below 2^31 at T = 32768
    if (c.kv_heads > 128) return LTE_ERR_UNSUPPORTED;
    if (long(c.batch) * c.kv_heads > (1L << 20)) return LTE_ERR_UNSUPPORTED;
    return LTE_OK;
}

int check_T(int64_t T) {
    if (T < 1) return LTE_ERR_INVALID_ARG;
    if (T > kMaxT) return LTE_ERR_UNSUPPORTED;
    return LTE_OK;
}

int check_cnn(const lte_cnn* cnn) {
    if (cnn == nullptr) return LTE_ERR_INVALID_ARG;
    if (!cnn->w1 || !cnn->b1 || !cnn->w2 || !cnn->b2) return LTE_ERR_INVALID_ARG;
    return LTE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LTE_OK : LTE_ERR_HIP; }

struct WsPtrs {
    float* scores;
    int32_t* rank;
    int32_t* thr;
    int32_t* ncand;
    uint32_t* select_scratch;
    float* dec_part;
};

WsPtrs ws_ptrs(const Shape& sh, int64_t T, void* ws) {
    WsLayout L = ws_layout(sh, T);
    char* p = static_cast<char*>(ws);
    WsPtrs w;
    w.scores = reinterpret_cast<float*>(p + L.scores);
    w.rank = reinterpret_cast<int32_t*>(p + L.rank);
    w.thr = reinterpret_cast<int32_t*>(p + L.thr);
    w.ncand = reinterpret_cast<int32_t*>(p + L.ncand);
    w.select_scratch = reinterpret_cast<uint32_t*>(p + L.select_scratch);
    w.dec_part = reinterpret_cast<float*>(p + L.dec_part);
    return w;
}

int check_ws(const Shape& sh, int64_t T, const void* ws, size_t bytes) {
    if (ws == nullptr) return LTE_ERR_INVALID_ARG;
    if (bytes < ws_layout(sh, T).total) return LTE_ERR_WORKSPACE;
    return LTE_OK;
}

// Decode partials sit at the start of any workspace, before the prefill views.
float* dec_part_ptr(const Shape& sh, void* ws) {
    return reinterpret_cast<float*>(static_cast<char*>(ws) + ws_layout(sh, 0).dec_part);
}

// Workspace of a chunk of n tokens: a prefill workspace for the extended
// sequence's Emax = s + C + w + n rows first (so its views read as usual), then
// the extended K/V and the chunk's per-sequence data.
struct ChunkLayout {
    int64_t Emax;
    size_t ek, ev, ext_len, q_lo, tok_off, warm, score_lo, seg_tok, seg_slot, seg_row, total;
};

ChunkLayout chunk_layout(const Shape& sh, int64_t n) {
    ChunkLayout L{};
    L.Emax = int64_t(sh.s) + sh.C + sh.w + n;
    const size_t B = size_t(sh.B), BG = B * sh.Hkv;
    size_t off = ws_layout(sh, L.Emax).total;
    const size_t kv = B * size_t(L.Emax) * sh.Hkv * sh.D * 2;
    L.ek = off; off = align256(off + kv);
    L.ev = off; off = align256(off + kv);
    L.ext_len = off; off = align256(off + B * 4);
    L.q_lo = off; off = align256(off + B * 4);
    L.tok_off = off; off = align256(off + B * 4);
    L.warm = off; off = align256(off + B * 4);
    L.score_lo = off; off = align256(off + BG * 4);
    L.seg_tok = off; off = align256(off + BG * size_t(sh.C) * 4);
    L.seg_slot = off; off = align256(off + BG * size_t(sh.C) * 4);
    L.seg_row = off; off = align256(off + BG * size_t(sh.C) * 4);
    L.total = off;
    return L;
}

#define LTE_TRY(expr)                 \
    do {                              \
        int _st = (expr);             \
        if (_st != LTE_OK) return _st; \
    } while (0)

}  // namespace

extern "C" {

const char* lte_status_string(int status) {
    switch (status) {
        case LTE_OK: return "ok";
        case LTE_ERR_INVALID_ARG: return "invalid argument";
        case LTE_ERR_UNSUPPORTED: return "unsupported configuration";
        case LTE_ERR_STATE: return "cache state does not allow this call";
        case LTE_ERR_HIP: return "HIP launch or copy failed";
        case LTE_ERR_WORKSPACE: return "workspace too small";
        case LTE_ERR_SCRATCH: return "needs more scratch than the static array holds";
        default: return "unknown status";
    }
}

int lte_version(void) { return 1; }

int lte_check_config(const lte_config* cfg) { return check_cfg(cfg); }

size_t lte_cache_bytes(const lte_config* cfg) {
    if (check_cfg(cfg) != LTE_OK) return 0;
    return cache_layout(make_shape(*cfg)).total;
}

int lte_cache_get_layout(const lte_config* cfg, lte_cache_layout* out) {
    LTE_TRY(check_cfg(cfg));
    if (out == nullptr) return LTE_ERR_INVALID_ARG;
    *out = cache_layout(make_shape(*cfg));
    return LTE_OK;
}

size_t lte_workspace_bytes(const lte_config* cfg, int64_t T) {
    if (check_cfg(cfg) != LTE_OK) return 0;
    if (T < 0 || T > kMaxT) return 0;
    return ws_layout(make_shape(*cfg), T).total;
}

int lte_workspace_get_layout(const lte_config* cfg, int64_t T, lte_workspace_layout* out) {
    LTE_TRY(check_cfg(cfg));
    LTE_TRY(check_T(T));
    if (out == nullptr) return LTE_ERR_INVALID_ARG;
    WsLayout L = ws_layout(make_shape(*cfg), T);
    out->scores = L.scores;
    out->rank = L.rank;
    out->thr = L.thr;
    out->ncand = L.ncand;
    out->total = L.total;
    return LTE_OK;
}

int lte_cache_init(const lte_config* cfg, void* cache, void* stream) {
    LTE_TRY(check_cfg(cfg));
    if (cache == nullptr) return LTE_ERR_INVALID_ARG;
    Shape sh = make_shape(*cfg);
    return hip_status(launch_cache_init(sh, cache_view(sh, cache), hipStream_t(stream)));
}

int lte_prefill_score(const lte_config* cfg, int64_t T, const uint16_t* k, const uint16_t* v,
                      const lte_cnn* cnn, void* workspace, size_t workspace_bytes, void* stream) {
    LTE_TRY(check_cfg(cfg));
    LTE_TRY(check_T(T));
    LTE_TRY(check_cnn(cnn));
    if (!k || !v) return LTE_ERR_INVALID_ARG;
    Shape sh = make_shape(*cfg);
    LTE_TRY(check_ws(sh, T, workspace, workspace_bytes));
    WsPtrs w = ws_ptrs(sh, T, workspace);
    hipStream_t st = hipStream_t(stream);
    return hip_status(
        launch_score_prefill(sh, T, nullptr, nullptr, k, v, *cnn, w.scores, st));
}

int lte_prefill_select(const lte_config* cfg, int64_t T, const float* score_override,
                       void* workspace, size_t workspace_bytes, void* stream) {
    LTE_TRY(check_cfg(cfg));
    LTE_TRY(check_T(T));
    Shape sh = make_shape(*cfg);
    LTE_TRY(check_ws(sh, T, workspace, workspace_bytes));
    WsPtrs w = ws_ptrs(sh, T, workspace);
    hipStream_t st = hipStream_t(stream);
    const float* sc = w.scores;
    if (score_override != nullptr) {
        // the override becomes the workspace's score view, so later stages and
        // the tests read one place
        hipError_t e = hipMemcpyAsync(w.scores, score_override,
                                      size_t(sh.B) * sh.Hkv * T * sizeof(float),
                                      hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return LTE_ERR_HIP;
    }
    return hip_status(
        launch_select(sh, T, nullptr, sc, w.rank, w.thr, w.ncand, w.select_scratch, st));
}

int lte_prefill_attend(const lte_config* cfg, int64_t T, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, void* workspace, size_t workspace_bytes,
                       uint16_t* out, void* stream) {
    LTE_TRY(check_cfg(cfg));
    LTE_TRY(check_T(T));
    if (!q || !k || !v || !out) return LTE_ERR_INVALID_ARG;
    Shape sh = make_shape(*cfg);
    LTE_TRY(check_ws(sh, T, workspace, workspace_bytes));
    WsPtrs w = ws_ptrs(sh, T, workspace);
    return hip_status(
        launch_attend_prefill(sh, T, nullptr, nullptr, 0, q, k, v, w.rank, w.thr, w.ncand, out,
                              hipStream_t(stream)));
}

int lte_prefill_build_cache(const lte_config* cfg, int64_t T, const uint16_t* k,
                            const uint16_t* v, void* workspace, size_t workspace_bytes,
                            void* cache, void* stream) {
    LTE_TRY(check_cfg(cfg));
    LTE_TRY(check_T(T));
    if (!k || !v || !cache) return LTE_ERR_INVALID_ARG;
    Shape sh = make_shape(*cfg);
    LTE_TRY(check_ws(sh, T, workspace, workspace_bytes));
    WsPtrs w = ws_ptrs(sh, T, workspace);
    return hip_status(launch_build_cache(sh, T, nullptr, nullptr, k, v, w.scores, w.rank, w.thr,
                                         cache_view(sh, cache), hipStream_t(stream)));
}

int lte_prefill_build_cache_background(const lte_config* cfg, int64_t T, const uint16_t* k,
                                       const uint16_t* v, void* workspace,
                                       size_t workspace_bytes, void* cache, void* stream) {
    LTE_TRY(check_cfg(cfg));
    LTE_TRY(check_T(T));
    if (!k || !v || !cache) return LTE_ERR_INVALID_ARG;
    Shape sh = make_shape(*cfg);
    LTE_TRY(check_ws(sh, T, workspace, workspace_bytes));
    WsPtrs w = ws_ptrs(sh, T, workspace);
    return hip_status(launch_build_cache(sh, T, nullptr, nullptr, k, v, w.scores, w.rank, w.thr,
                                         cache_view(sh, cache), hipStream_t(stream),
                                         kBackgroundCopyWgs));
}

int lte_prefill(const lte_config* cfg, int64_t T, const uint16_t* q, const uint16_t* k,
                const uint16_t* v, const lte_cnn* cnn, const float* score_override, void* cache,
                void* workspace, size_t workspace_bytes, uint16_t* out, void* stream) {
    LTE_TRY(check_cfg(cfg));
    LTE_TRY(check_T(T));
    if (!q || !k || !v || !out) return LTE_ERR_INVALID_ARG;
    if (score_override == nullptr) LTE_TRY(check_cnn(cnn));
    Shape sh = make_shape(*cfg);
    LTE_TRY(check_ws(sh, T, workspace, workspace_bytes));
    if (score_override == nullptr)
        LTE_TRY(lte_prefill_score(cfg, T, k, v, cnn, workspace, workspace_bytes, stream));
    LTE_TRY(lte_prefill_select(cfg, T, score_override, workspace, workspace_bytes, stream));
    LTE_TRY(lte_prefill_attend(cfg, T, q, k, v, workspace, workspace_bytes, out, stream));
    if (cache != nullptr)
        LTE_TRY(lte_prefill_build_cache(cfg, T, k, v, workspace, workspace_bytes, cache, stream));
    return LTE_OK;
}

int lte_prefill_varlen(const lte_config* cfg, int64_t T, const int32_t* seq_lens,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const lte_cnn* cnn, const float* score_override, void* cache,
                       void* workspace, size_t workspace_bytes, uint16_t* out, void* stream) {
    LTE_TRY(check_cfg(cfg));
    LTE_TRY(check_T(T));
    if (!seq_lens || !q || !k || !v || !out) return LTE_ERR_INVALID_ARG;
    if (score_override == nullptr) LTE_TRY(check_cnn(cnn));
    Shape sh = make_shape(*cfg);
    LTE_TRY(check_ws(sh, T, workspace, workspace_bytes));
    WsPtrs w = ws_ptrs(sh, T, workspace);
    hipStream_t st = hipStream_t(stream);
    const float* sc = w.scores;
    if (score_override == nullptr) {
        LTE_TRY(hip_status(
            launch_score_prefill(sh, T, seq_lens, nullptr, k, v, *cnn, w.scores, st)));
    } else {
        hipError_t e = hipMemcpyAsync(w.scores, score_override,
                                      size_t(sh.B) * sh.Hkv * T * sizeof(float),
                                      hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return LTE_ERR_HIP;
    }
    LTE_TRY(hip_status(
        launch_select(sh, T, seq_lens, sc, w.rank, w.thr, w.ncand, w.select_scratch, st)));
    LTE_TRY(hip_status(
        launch_attend_prefill(sh, T, seq_lens, nullptr, 0, q, k, v, w.rank, w.thr, w.ncand, out,
                              st)));
    if (cache != nullptr)
        LTE_TRY(hip_status(launch_build_cache(sh, T, seq_lens, nullptr, k, v, w.scores, w.rank, w.thr,
                                             cache_view(sh, cache), st)));
    return LTE_OK;
}

size_t lte_chunk_workspace_bytes(const lte_config* cfg, int64_t n) {
    if (check_cfg(cfg) != LTE_OK) return 0;
    const Shape sh = make_shape(*cfg);
    if (n < 1 || int64_t(sh.s) + sh.C + sh.w + n > kMaxT) return 0;
    return chunk_layout(sh, n).total;
}

int lte_prefill_chunk(const lte_config* cfg, int64_t n, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const lte_cnn* cnn, void* cache, void* workspace,
                      size_t workspace_bytes, uint16_t* out, void* stream) {
    LTE_TRY(check_cfg(cfg));
    if (n < 1) return LTE_ERR_INVALID_ARG;
    if (!q || !k || !v || !cache || !out || !workspace) return LTE_ERR_INVALID_ARG;
    LTE_TRY(check_cnn(cnn));
    const Shape sh = make_shape(*cfg);
    if (int64_t(sh.s) + sh.C + sh.w + n > kMaxT) return LTE_ERR_UNSUPPORTED;
    const ChunkLayout L = chunk_layout(sh, n);
    if (workspace_bytes < L.total) return LTE_ERR_WORKSPACE;
    const int64_t E = L.Emax;
    char* p = static_cast<char*>(workspace);
    WsPtrs w = ws_ptrs(sh, E, workspace);
    ChunkView x;
    x.ext_len = reinterpret_cast<int32_t*>(p + L.ext_len);
    x.q_lo = reinterpret_cast<int32_t*>(p + L.q_lo);
    x.tok_off = reinterpret_cast<int32_t*>(p + L.tok_off);
    x.warm = reinterpret_cast<int32_t*>(p + L.warm);
    x.score_lo = reinterpret_cast<int32_t*>(p + L.score_lo);
    x.seg_tok = reinterpret_cast<int32_t*>(p + L.seg_tok);
    x.seg_slot = reinterpret_cast<int32_t*>(p + L.seg_slot);
    x.seg_row = reinterpret_cast<int32_t*>(p + L.seg_row);
    uint16_t* ek = reinterpret_cast<uint16_t*>(p + L.ek);
    uint16_t* ev = reinterpret_cast<uint16_t*>(p + L.ev);
    const CacheView c = cache_view(sh, cache);
    hipStream_t st = hipStream_t(stream);
    LTE_TRY(hip_status(launch_chunk_gather(sh, int(n), int(E), k, v, c, x, w.scores, ek, ev, st)));
    LTE_TRY(hip_status(
        launch_score_prefill(sh, E, x.ext_len, x.score_lo, ek, ev, *cnn, w.scores, st)));
    LTE_TRY(hip_status(
        launch_select(sh, E, x.ext_len, w.scores, w.rank, w.thr, w.ncand, w.select_scratch, st)));
    LTE_TRY(hip_status(launch_attend_prefill(sh, E, x.ext_len, x.q_lo, int(n), q, ek, ev, w.rank,
                                             w.thr, w.ncand, out, st)));
    return hip_status(
        launch_build_cache(sh, E, x.ext_len, &x, ek, ev, w.scores, w.rank, w.thr, c, st));
}

int lte_linear_check_config(const lte_linear_config* cfg) {
    if (cfg == nullptr) return LTE_ERR_INVALID_ARG;
    if (cfg->batch < 1 || cfg->heads < 1 || cfg->head_dim < 1) return LTE_ERR_INVALID_ARG;
    if (cfg->head_dim != 64 && cfg->head_dim != 128) return LTE_ERR_UNSUPPORTED;
    if (int64_t(cfg->batch) * cfg->heads > (int64_t(1) << 24)) return LTE_ERR_UNSUPPORTED;
    return LTE_OK;
}

size_t lte_linear_state_bytes(const lte_linear_config* cfg) {
    if (lte_linear_check_config(cfg) != LTE_OK) return 0;
    return size_t(cfg->batch) * cfg->heads * cfg->head_dim * cfg->head_dim * sizeof(float);
}

int lte_linear_prefill(const lte_linear_config* cfg, int64_t T, const uint16_t* q,
                       const uint16_t* k, const uint16_t* v, const float* log_a,
                       const float* state_in, float* state_out, uint16_t* out, void* stream) {
    LTE_TRY(lte_linear_check_config(cfg));
    if (T < 1) return LTE_ERR_INVALID_ARG;
    if (T > kMaxLinearT) return LTE_ERR_UNSUPPORTED;
    if (!q || !k || !v || !log_a || !state_out || !out) return LTE_ERR_INVALID_ARG;
    return hip_status(launch_linear_prefill(cfg->batch, cfg->heads, cfg->head_dim, T, q, k, v,
                                            log_a, state_in, state_out, out,
                                            hipStream_t(stream)));
}

int lte_linear_decode_step(const lte_linear_config* cfg, const uint16_t* q_t, const uint16_t* k_t,
                           const uint16_t* v_t, const float* log_a_t, float* state,
                           uint16_t* out_t, void* stream) {
    LTE_TRY(lte_linear_check_config(cfg));
    if (!q_t || !k_t || !v_t || !log_a_t || !state || !out_t) return LTE_ERR_INVALID_ARG;
    return hip_status(launch_linear_step(cfg->batch, cfg->heads, cfg->head_dim, q_t, k_t, v_t,
                                         log_a_t, state, out_t, hipStream_t(stream)));
}

int lte_score_evict(const lte_config* cfg, const lte_cnn* cnn, const uint16_t* k_t,
                    const uint16_t* v_t, void* cache, void* stream) {
    LTE_TRY(check_cfg(cfg));
    LTE_TRY(check_cnn(cnn));
    if (!k_t || !v_t || !cache) return LTE_ERR_INVALID_ARG;
    Shape sh = make_shape(*cfg);
    return hip_status(
        launch_score_evict(sh, *cnn, k_t, v_t, cache_view(sh, cache), hipStream_t(stream)));
}

int lte_decode_attend(const lte_config* cfg, const uint16_t* q_t, void* cache,
                      void* workspace, size_t workspace_bytes, uint16_t* out_t, void* stream) {
    LTE_TRY(check_cfg(cfg));
    if (!q_t || !cache || !out_t) return LTE_ERR_INVALID_ARG;
    Shape sh = make_shape(*cfg);
    if (workspace == nullptr) return LTE_ERR_INVALID_ARG;
    if (workspace_bytes < ws_layout(sh, 0).total) return LTE_ERR_WORKSPACE;
    return hip_status(launch_decode(sh, false, q_t, nullptr, nullptr, nullptr,
                                    cache_view(sh, cache), dec_part_ptr(sh, workspace), out_t,
                                    hipStream_t(stream)));
}

int lte_decode_step(const lte_config* cfg, const uint16_t* q_t, const uint16_t* k_t,
                    const uint16_t* v_t, const lte_cnn* cnn, void* cache, void* workspace,
                    size_t workspace_bytes, uint16_t* out_t, void* stream) {
    LTE_TRY(check_cfg(cfg));
    LTE_TRY(check_cnn(cnn));
    if (!q_t || !k_t || !v_t || !cache || !out_t || !workspace) return LTE_ERR_INVALID_ARG;
    Shape sh = make_shape(*cfg);
    if (workspace_bytes < ws_layout(sh, 0).total) return LTE_ERR_WORKSPACE;
    return hip_status(launch_decode(sh, true, q_t, k_t, v_t, cnn, cache_view(sh, cache),
                                    dec_part_ptr(sh, workspace), out_t, hipStream_t(stream)));
}

int lte_decode_step_static(const lte_config* cfg, const uint16_t* q_t, const uint16_t* k_t,
                           const uint16_t* v_t, const lte_cnn* cnn, void* cache,
                           uint16_t* out_t, void* stream) {
    LTE_TRY(check_cfg(cfg));
    LTE_TRY(check_cnn(cnn));
    if (!q_t || !k_t || !v_t || !cache || !out_t) return LTE_ERR_INVALID_ARG;
    Shape sh = make_shape(*cfg);
    if (decode_part_bytes(sh) > kStaticScratchBytes) return LTE_ERR_SCRATCH;
    float* part = nullptr;
    if (static_scratch(&part) != hipSuccess) return LTE_ERR_HIP;
    return hip_status(launch_decode(sh, true, q_t, k_t, v_t, cnn, cache_view(sh, cache), part,
                                    out_t, hipStream_t(stream)));
}

int lte_cache_export(const lte_config* cfg, const void* cache, int32_t* ret_idx,
                     float* ret_score, int32_t* count, int64_t* pos, void* stream) {
    LTE_TRY(check_cfg(cfg));
    if (cache == nullptr) return LTE_ERR_INVALID_ARG;
    Shape sh = make_shape(*cfg);
    lte_cache_layout L = cache_layout(sh);
    const char* p = static_cast<const char*>(cache);
    hipStream_t st = hipStream_t(stream);
    const size_t bg = size_t(sh.B) * sh.Hkv;
    struct Item { void* dst; size_t off; size_t bytes; } items[4] = {
        {ret_idx, L.ret_idx, bg * sh.C * 4},
        {ret_score, L.ret_score, bg * sh.C * 4},
        {count, L.count, bg * 4},
        {pos, L.pos, bg * 8},
    };
    for (const Item& it : items) {
        if (it.dst == nullptr || it.bytes == 0) continue;
        if (hipMemcpyAsync(it.dst, p + it.off, it.bytes, hipMemcpyDeviceToDevice, st) != hipSuccess)
            return LTE_ERR_HIP;
    }
    return LTE_OK;
}

}  // extern "C"
