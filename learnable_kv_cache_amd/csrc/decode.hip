// Decode path of the LTE layer on gfx950: one token per sequence per step.
//
// LTE paper (arXiv 2510.20787) summary page:
//   Figure 2 caption - a KV pair's eviction is decided when it moves out of
//     the window; its score needs the short-range future neighbours, so it is
//     computable once the CNN's receptive field is covered by the window.
//   Figure 3 caption - circular window segment + capped out-of-window segment
//     (retained KVs and the sink); scoring batched and deferred as late as
//     possible.
// "Sparse Linear Attention: Viewing SWA from the Perspective of Linear
// Attention", section "Viewing SWA from the linear-state perspective": each
// token overwrites one window slot, first in first out.
//
// Ingesting token t (position pos):
//   1. token t-w leaves ring slot t mod w; if t-w >= s and its score is > 0.5
//      it enters the capped segment: appended while count < C, otherwise it
//      replaces the weakest entry (lowest score, then highest index) when its
//      score is strictly higher (being the newest, it loses score ties);
//   2. k_t, v_t go into that ring slot (and into sink slot t when t < s);
//   3. when t = u + w - 3 for the oldest unscored token u, tokens u .. t-2 are
//      scored from the ring -- the last step at which their left neighbour
//      u-2 is still there;
//   4. pos = t + 1.
// The decision of step 1 depends only on the state the previous step left,
// so whoever finishes an ingest (or builds the cache) also records the next
// one (nx_slot, nx_score): the attention of a step never waits for it.
//
// A decode step is one launch.  Each (batch, KV head) is served by one
// workgroup of 8 waves, or, when there are fewer than 256 such pairs, by a few
// workgroups that split its visible rows:
//   * the visible rows (sink, post-step segment, window) are read in chunks of
//     32 by direct global->LDS loads of whole 256-byte rows, so only occupied
//     slots cost bandwidth.  A wave refills its K tile with its next chunk as
//     soon as the q.k operands are in registers and its V tile as soon as the
//     p.v operands are, so its loads are in flight while it computes.  Rows
//     that differ in the post-ingest state are read from where they are before
//     the step: the new token from the k_t/v_t inputs, the leaving token
//     (taking segment slot X) from its ring slot;
//   * q.k and p.v run on v_mfma_f32_16x16x32_bf16 with the G <= 16 query heads
//     of the KV head as the 16 columns; V is read back transposed
//     (ds_read_b64_tr_b16);
//   * the waves' (max, sum, unnormalised o) merge in LDS, in wave order.  With
//     several workgroups per pair, each writes its partial with device-scope
//     coherent stores and counts itself in on the pair's arrival word; the last
//     to arrive merges the partials in split order (deterministic);
//   * the finishing workgroup writes o_t, moves the leaving token's row into its
//     segment slot, writes k_t/v_t into the ring, records the next decision and
//     the weakest segment entry (computed by every workgroup while its first
//     chunks load);
//   * on a scoring step the waves share the deferred batch, 28 tokens per wave
//     call.
// The partials bypass the non-coherent L2 copies instead of a cache-wide
// write-back and invalidate, which a device-scope fence would cost on gfx950.
#include <mutex>

#include "score_core.h"

namespace lte {

// Split partials of lte_decode_step_static: a fixed device array instead of a
// caller workspace, for callers that cannot allocate.  Every device the library
// runs on holds its own copy until the process ends; host code never passes the
// array's name to a kernel (on the host it only stands for the symbol), only the
// per-device address that hipGetSymbolAddress returns.
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

hipError_t static_scratch(float** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float* ptrs[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {              // first call on this device, which is current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptrs[dev] = static_cast<float*>(p);
    }
    *out = ptrs[dev];
    return hipSuccess;
}

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16]
// and D[4(l/16)+r][l%16].
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS chunk swizzle of V tile row r: 16-byte chunk c of row r sits at chunk
// position c ^ swz(r).  A transposing read of the p.v operand fetches chunks
// 2dt, 2dt+1 of 4 consecutive rows per 16 lanes (8 rows per 32 lanes); with
// swz = 2 (r mod 8) (D = 128) or 2 (r mod 4) (D = 64) those land on distinct
// bank groups.
template <int D>
__device__ __forceinline__ int vswz(int r) { return D == 128 ? 2 * (r & 7) : 2 * (r & 3); }

// Device-scope coherent traffic for the split partials: buffer loads and
// stores with the sc1 cache-policy bit, the bit relaxed agent-scope atomic
// loads and stores carry, in 16-byte pieces.  Offsets in bytes.
constexpr int kSc1 = 16;                       // cache-policy operand: sc1
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(float* p) {
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, 0x7fffffff, 0x00020000);
}

// Max and sum of a value over the four lanes l, l ^ 16, l ^ 32, l ^ 48, by the two
// row-swapping permutes (each lane takes the larger, or the sum, of the pair it
// holds afterwards: its own value and its partner's), with no LDS round trip.
__device__ __forceinline__ float max_swap(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float add_swap(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Decision for the token leaving at the ingest of position t, from the state
// after the previous step: -2 unscored, -1 not kept, else its segment slot.
__device__ __forceinline__ int decide_slot(int64_t t, float rl, int cnt, int weak,
                                           float weak_score, int s, int w, int C) {
    if (t - w < s) return -1;
    if (rl != rl) return -2;
    if (!(rl > 0.5f) || C == 0) return -1;
    if (cnt < C) return cnt;
    if (weak >= 0 && rl > weak_score) return weak;
    return -1;
}

// Scores chunk ch (tokens u + 28 ch .. u + 28 ch + 27, clipped to t-2) of the
// deferred batch of (b, g) at step t, reading tokens < t from their ring slots
// and token t from the inputs.  One wave.
template <int D>
__device__ void score_deferred_chunk(const CacheView& c, int bg, int g, int s, int w, int C,
                                     int S, int t, int u, int ch,
                                     const uint16_t* __restrict__ k_t,
                                     const uint16_t* __restrict__ v_t, const lte_cnn& cnn,
                                     float* Ya, float* Yb) {
    const uint16_t* kring = c.k + (long(bg) * S + s + C) * D;
    const uint16_t* vring = c.v + (long(bg) * S + s + C) * D;
    float* rs = c.ring_score + long(bg) * w;
    score_wave<D>(
        Ya, Yb, cnn.w1 + long(g) * kHidden * 2 * D * 3, cnn.b1 + g * kHidden,
        cnn.w2 + g * kHidden * 3, cnn.b2[g], u + kWaveScoreTile * ch, u, t - 2,
        [&](int x, const uint16_t*& kp, const uint16_t*& vp) {
            if (x < 0 || x > t) return false;
            if (x == t) {
                kp = k_t + long(bg) * D;
                vp = v_t + long(bg) * D;
            } else {
                kp = kring + long(x % w) * D;
                vp = vring + long(x % w) * D;
            }
            return true;
        },
        [&](int x) { return x < 0; },
        [&](int tok, float r) { rs[tok % w] = r; });
}

// Order of segment entries for eviction: a is weaker than b when its score is
// lower, or equal with the higher token index.
__device__ __forceinline__ bool weaker(float sa, int ta, float sb, int tb) {
    return sa < sb || (sa == sb && ta > tb);
}

// Weakest of (score, token, slot) over the wave; lanes without an entry hold
// (+inf, -1, -1).
__device__ __forceinline__ void wave_weakest(float& sc, int& tk, int& sl) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float os = __shfl_xor(sc, o, 64);
        const int ot = __shfl_xor(tk, o, 64);
        const int ol = __shfl_xor(sl, o, 64);
        if (weaker(os, ot, sc, tk)) { sc = os; tk = ot; sl = ol; }
    }
}

// Writes of the ingest of token t into the cache of one (b, g), from the
// state before the step (cnt, X = nx_slot, rl = nx_score, u) and what the
// step computed: (wk, ws) the weakest slot and score of the post-step
// segment when it holds C entries (else wk = -1), r1 the score of token
// t+1-w, which leaves at the next ingest (scored at least three steps before
// it leaves, never by this step's batch), and the new token's 16-byte chunk
// `lane` of k and v for lanes < D/8.  One wave.
template <int D>
__device__ void ingest_commit(const CacheView& c, int bg, int s, int w, int C, int S, int t,
                              int cnt, int X, float rl, int u, int wk, float ws, float r1,
                              const u32x4& nk, const u32x4& nv) {
    const int lane = threadIdx.x & 63;
    const int tslot = t % w;
    const int new_cnt = (X >= 0 && X == cnt) ? cnt + 1 : cnt;
    if (lane < D / 8) {
        const long ring_row = (long(bg) * S + s + C + tslot) * D + lane * 8;
        *reinterpret_cast<u32x4*>(c.k + ring_row) = nk;
        *reinterpret_cast<u32x4*>(c.v + ring_row) = nv;
        if (t < s) {
            const long srow = (long(bg) * S + t) * D + lane * 8;
            *reinterpret_cast<u32x4*>(c.k + srow) = nk;
            *reinterpret_cast<u32x4*>(c.v + srow) = nv;
        }
    }
    if (lane == 0) {
        if (X >= 0) {
            c.ret_idx[long(bg) * C + X] = t - w;
            c.ret_score[long(bg) * C + X] = rl;
            c.count[bg] = new_cnt;
        }
        if (X == -2) c.flags[bg] |= 1;
        c.ring_score[long(bg) * w + tslot] = __builtin_nanf("");
        c.weak[bg] = wk;
        c.nx_slot[bg] = decide_slot(t + 1, r1, new_cnt, wk, ws, s, w, C);
        c.nx_score[bg] = r1;
        c.next_unscored[bg] = (t == u + w - 3) ? t - 1 : u;
        c.pos[bg] = t + 1;
    }
}

// lte_score_evict: the ingest alone, one wave per (batch, KV head).
template <int D>
__global__ __launch_bounds__(64) void score_evict_kernel(int s, int w, int C, int S, int Hkv,
                                                         const uint16_t* __restrict__ k_t,
                                                         const uint16_t* __restrict__ v_t,
                                                         lte_cnn cnn, CacheView c) {
    __shared__ __align__(16) float Ya[kWaveScoreBytesA / 4];
    __shared__ __align__(16) float Yb[kWaveScoreBytesB / 4];
    const int lane = threadIdx.x;
    const int bg = blockIdx.x;
    const int t = int(c.pos[bg]);
    const int cnt = c.count[bg];
    const int X = c.nx_slot[bg];
    const float rl = c.nx_score[bg];
    const int u = int(c.next_unscored[bg]);
    const int tslot = t % w;
    const int new_cnt = (X >= 0 && X == cnt) ? cnt + 1 : cnt;
    const float r1 = (t + 1 - w >= s) ? c.ring_score[long(bg) * w + (t + 1) % w] : 0.0f;
    u32x4 nk = u32x4{}, nv = u32x4{};
    if (lane < D / 8) {
        nk = *reinterpret_cast<const u32x4*>(k_t + long(bg) * D + lane * 8);
        nv = *reinterpret_cast<const u32x4*>(v_t + long(bg) * D + lane * 8);
        if (X >= 0) {                         // the leaving token's row into its slot
            const long rr = (long(bg) * S + s + C + tslot) * D + lane * 8;
            const long dst = (long(bg) * S + s + X) * D + lane * 8;
            *reinterpret_cast<u32x4*>(c.k + dst) = *reinterpret_cast<const u32x4*>(c.k + rr);
            *reinterpret_cast<u32x4*>(c.v + dst) = *reinterpret_cast<const u32x4*>(c.v + rr);
        }
    }
    // weakest entry of the post-step segment when full, slot X holding the newcomer
    float wsc = INFINITY;
    int wtk = -1, wsl = -1;
    if (C > 0 && new_cnt == C) {
        for (int x = lane; x < C; x += 64) {
            const float sc = (x == X) ? rl : c.ret_score[long(bg) * C + x];
            const int tk = (x == X) ? t - w : c.ret_idx[long(bg) * C + x];
            if (weaker(sc, tk, wsc, wtk)) { wsc = sc; wtk = tk; wsl = x; }
        }
        wave_weakest(wsc, wtk, wsl);
    }
    if (t == u + w - 3) {                     // deferred batch: ring rows of tokens < t
        const int nch = (t - 1 - u + kWaveScoreTile - 1) / kWaveScoreTile;
        for (int ch = 0; ch < nch; ++ch)
            score_deferred_chunk<D>(c, bg, bg % Hkv, s, w, C, S, t, u, ch, k_t, v_t, cnn, Ya, Yb);
    }
    __builtin_amdgcn_s_waitcnt(0);            // ring row copied before it is overwritten
    ingest_commit<D>(c, bg, s, w, C, S, t, cnt, X, rl, u, wsl, wsc, r1, nk, nv);
}

// Per-wave LDS of the decode step: one chunk of 32 visible rows of K (in Ks) and
// of V (in Vs), each a [32][D/8] array of 16-byte pieces; afterwards the wave's
// scorer rows (taps 0-1 in Ks, tap 2 in Vs) and its partial output.  K and V
// tiles are separate LDS objects so that the compiler can tell a tile being
// read from one being filled by direct loads, and does not wait for the latter.
template <int D>
struct DecTile {
    static constexpr int CPR = D / 8;                      // 16-byte pieces per row
    static constexpr int kRows = 32;                       // rows per chunk
    static constexpr int kTile = kRows * CPR;              // pieces per tensor tile
    static constexpr int kLoads = kTile / 64;              // direct loads per tensor tile
    static constexpr int kKW = (kTile * 16 > kWaveScoreBytesA ? kTile * 16 : kWaveScoreBytesA) / 16;
    static constexpr int kVW = (kTile * 16 > kWaveScoreBytesB ? kTile * 16 : kWaveScoreBytesB) / 16;
};

// LDS piece swizzle of K tile row r: logical piece c of row r sits at c ^ kswz(r).
// The q.k operand read takes one piece of 16 consecutive rows per 16 lanes; the
// swizzle spreads them over 256 bytes of banks.
template <int D>
__device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }

// One decode step (INGEST) or an attention over the cache as it is.
//
// The slots of (b, g) are read in chunks of 32 rows in a fixed list: the ring
// chunks first (slots s+C .. s+C+w-1, which need no state to address), then the
// chunks of [0, s+C) that hold a sink token or a segment entry -- an empty
// segment costs nothing.  With one workgroup per (b, g) the list is dealt
// round-robin to the 8 waves; with nsplit > 1 each workgroup takes a contiguous
// run of it.  Rows past a chunk's valid ones re-read a valid row.  The list, the
// order and the split depend only on the visible set, so the fused step and
// score_evict + attend produce identical bits.
//
// A chunk's K and V rows arrive by direct global->LDS loads of whole 256-byte
// rows, issued as soon as the wave's tiles are free.  Loads whose results are only
// needed by the ingest (segment scores, the leaving token's row, the next leaving
// token's score) are issued before the chunks are computed, so the ingest at the
// end only stores.
template <int D, int G, bool INGEST>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_step_kernel(
    int Hq, int Hkv, int s, int w, int C, int S, int nsplit,
    const uint16_t* __restrict__ q_t, const uint16_t* __restrict__ k_t,
    const uint16_t* __restrict__ v_t, lte_cnn cnn, CacheView c, float* __restrict__ part,
    uint16_t* __restrict__ out_t) {
    using TL = DecTile<D>;
    constexpr int NW = kDecodeWaves;
    constexpr int RW = TL::kRows;
    constexpr int NL = TL::kLoads;
    constexpr int KS = D / 32;                 // q.k k-steps
    constexpr int DT = D / 16;                 // p.v output tiles
    constexpr int CPR = TL::CPR;
    constexpr int PW = decode_part_floats(G, D);
    constexpr int kScan = (kMaxCapacity + 64 * NW - 1) / (64 * NW);   // segment entries per thread
    static_assert(G * D * 4 <= TL::kKW * 16 && 2 * G * 4 <= TL::kVW * 16, "wave partials fit");
    __shared__ __align__(16) u32x4 Ks[NW][TL::kKW];
    __shared__ __align__(16) u32x4 Vs[NW][TL::kVW];
    __shared__ __align__(16) u32x4 Kx[TL::kTile];     // wave 0's prefetched last chunk
    __shared__ __align__(16) u32x4 Vx[TL::kTile];
    __shared__ float wk_sc[NW];
    __shared__ int wk_tk[NW], wk_sl[NW];
    __shared__ int last_flag;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int q16 = lane >> 4;
    const int sp = __builtin_amdgcn_readfirstlane(blockIdx.x % nsplit);
    const int bg = __builtin_amdgcn_readfirstlane(blockIdx.x / nsplit);
    const int b = bg / Hkv;
    const int g = bg % Hkv;
    // the state first (scalar loads; positions fit in 32 bits)
    const int p = int(c.pos[bg]);
    const int cnt = c.count[bg];
    const int X = INGEST ? c.nx_slot[bg] : -1;
    const int u = INGEST ? int(c.next_unscored[bg]) : 0;
    const float rl = INGEST ? c.nx_score[bg] : 0.0f;
    u32x4* Kt = Ks[wave];
    u32x4* Vt = Vs[wave];
    const long base = long(bg) * S * D;
    const char* kb = reinterpret_cast<const char*>(c.k + base);
    const char* vb = reinterpret_cast<const char*>(c.v + base);

    // list entries [e_lo, e_lo + per) of this workgroup: nr ring chunks, then head chunks
    const int nr = (w + RW - 1) / RW;
    const int nh = (s + C + RW - 1) / RW;
    const int per = nsplit > 1 ? (nr + nh + nsplit - 1) / nsplit : nr + nh;
    const int e_lo = sp * per;
    const int ent0 = e_lo + wave;

    // A tile piece x*64 + lane is row (x*64+lane)/CPR at position (x*64+lane)%CPR and
    // holds that row's logical piece position ^ swizzle(row); rows are byte offsets
    // from this (b, g)'s K and V slots.
    auto kaddr = [&](const uint32_t (&roff)[NL], int x) {
        const int pidx = 64 * x + lane;
        return kb + roff[x] + 16 * ((pidx % CPR) ^ kswz<D>(pidx / CPR));
    };
    auto vaddr = [&](const uint32_t (&roff)[NL], int x) {
        const int pidx = 64 * x + lane;
        return vb + roff[x] + 16 * ((pidx % CPR) ^ vswz<D>(pidx / CPR));
    };
    auto load_k = [&](const uint32_t (&roff)[NL], u32x4* Kd) {
#pragma unroll
        for (int x = 0; x < NL; ++x)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)kaddr(roff, x),
                (__attribute__((address_space(3))) void*)(&Kd[64 * x]), 16, 0, 0);
    };
    auto load_v = [&](const uint32_t (&roff)[NL], u32x4* Vd) {
#pragma unroll
        for (int x = 0; x < NL; ++x)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)vaddr(roff, x),
                (__attribute__((address_space(3))) void*)(&Vd[64 * x]), 16, 0, 0);
    };
    auto load_lds = [&](const uint32_t (&roff)[NL], u32x4* Kd, u32x4* Vd) {
        load_k(roff, Kd);
        load_v(roff, Vd);
    };
    // ring chunk i: slots s+C+32i .. (rows past the ring re-read its last slot)
    auto ring_rows = [&](int i, uint32_t (&roff)[NL]) {
        const int r0 = RW * i + lane / CPR;
#pragma unroll
        for (int x = 0; x < NL; ++x)
            roff[x] = uint32_t(s + C + min(r0 + x * (64 / CPR), w - 1)) * (D * 2);
    };

    // ring chunks can be requested before the state is known
    const bool early0 = ent0 < nr && ent0 < e_lo + per;
    if (early0) {
        uint32_t roff[NL];
        ring_rows(ent0, roff);
        load_lds(roff, Kt, Vt);
    }
    // the segment's scores and tokens, for the weakest entry after the ingest
    float sc_e[kScan];
    int tk_e[kScan];
    if (INGEST) {
#pragma unroll
        for (int i = 0; i < kScan; ++i) {
            const int e = tid + i * 64 * NW;
            sc_e[i] = INFINITY;
            tk_e[i] = -1;
            if (e < C) {
                sc_e[i] = c.ret_score[long(bg) * C + e];
                tk_e[i] = c.ret_idx[long(bg) * C + e];
            }
        }
    }
    // q: B operand of q.k, head l16 (zero past G), dims 32kk + 8q16 .. +7
    bf16x8 qf[KS];
    {
        const bool hv = l16 < G;
        const uint16_t* qrow = q_t + (long(b) * Hq + g * G + (hv ? l16 : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            qf[kk] = hv ? *reinterpret_cast<const bf16x8*>(qrow + 32 * kk + 8 * q16) : bf16x8{};
    }
    // the new token's row pieces (lanes < D/8): the LDS patches and the ingest
    u32x4 nk = u32x4{}, nvv = u32x4{};
    if (INGEST && lane < CPR) {
        nk = *reinterpret_cast<const u32x4*>(k_t + long(bg) * D + lane * 8);
        nvv = *reinterpret_cast<const u32x4*>(v_t + long(bg) * D + lane * 8);
    }

    // ---- the visible rows ------------------------------------------------------------------
    const int t = INGEST ? p : p - 1;
    const int tslot = t >= 0 ? t % w : 0;
    const int new_cnt = (X >= 0 && X == cnt) ? cnt + 1 : cnt;
    const int ns = t >= 0 ? min(s, t + 1) : 0;                  // sink rows
    const bool ring_full = t - s + 1 >= w;                      // every ring slot visible
    // ring slot r holds token t - d, d = (tslot - r) mod w: visible when >= s
    auto ring_ok = [&](int r) {
        const int d = tslot - r + (tslot < r ? w : 0);
        return (r < w) & (d <= t - s);
    };
    auto head_ok = [&](int slot) {
        return (slot < ns) | (unsigned(slot - s) < unsigned(new_cnt));
    };
    // head chunks holding a visible row: [0, ha) U [hb, he)
    const int ha = (ns + RW - 1) / RW;
    const int hb = s / RW;
    const int he = new_cnt > 0 ? (s + new_cnt + RW - 1) / RW : hb;
    const bool merged = hb <= ha;
    const int nvh = merged ? max(ha, he) : ha + (he - hb);
    const int e_hi = min(e_lo + per, nr + nvh);
    auto head_chunk = [&](int hi) { return (merged || hi < ha) ? hi : hb + hi - ha; };
    // head chunk k: invalid rows re-read the chunk's first visible one; in the
    // post-ingest state the segment slot the leaving token takes reads it from its
    // ring slot (the new token's sink row is patched in LDS once it has landed)
    const int xslot = (INGEST && X >= 0) ? s + X : -1;
    auto chunk_rows = [&](int ent, uint32_t (&roff)[NL]) {
        if (ent < nr) {
            ring_rows(ent, roff);
        } else {
            const int k = head_chunk(ent - nr);
            const int fv = (RW * k < ns) ? RW * k : max(RW * k, s);
#pragma unroll
            for (int x = 0; x < NL; ++x) {
                int slot = RW * k + (64 * x + lane) / CPR;
                slot = head_ok(slot) ? slot : fv;
                slot = (slot == xslot) ? s + C + tslot : slot;
                roff[x] = uint32_t(slot) * (D * 2);
            }
        }
    };
    if (!early0 && ent0 < e_hi) {
        uint32_t roff[NL];
        chunk_rows(ent0, roff);
        load_lds(roff, Kt, Vt);
    }
    // When the last round of the list would hold one chunk (wave 0's), that chunk loads
    // now into a tile pair of its own and is consumed right after wave 0's first, so no
    // round waits on a single chunk.
    const int n_ent = e_hi - e_lo;
    const bool xtra = n_ent > NW && n_ent % NW == 1;
    const int e_rr = xtra ? e_hi - 1 : e_hi;                    // entries dealt round-robin
    if (xtra && wave == 0) {
        uint32_t roff[NL];
        chunk_rows(e_hi - 1, roff);
        load_lds(roff, Kx, Vx);
    }
    // ingest operands consumed at the end: the score of the token leaving at the next
    // step and the leaving token's row (lanes < D/8 of wave 0)
    float r1 = 0.0f;
    u32x4 lk = u32x4{}, lv = u32x4{};
    if (INGEST) {
        if (t + 1 - w >= s) r1 = c.ring_score[long(bg) * w + (t + 1) % w];
        if (X >= 0 && wave == 0 && lane < CPR) {
            const long rr = long(s + C + tslot) * D + lane * 8;
            lk = *reinterpret_cast<const u32x4*>(c.k + base + rr);
            lv = *reinterpret_cast<const u32x4*>(c.v + base + rr);
        }
    }

    // the weakest entry of the post-step segment when it holds C entries (slot X
    // holding the newcomer), this wave's share
    if (INGEST) {
        float wsc = INFINITY;
        int wtk = -1, wsl = -1;
        if (C > 0 && new_cnt == C) {
#pragma unroll
            for (int i = 0; i < kScan; ++i) {
                const int e = tid + i * 64 * NW;
                const float sc = (e == X) ? rl : sc_e[i];
                const int tk = (e == X) ? t - w : tk_e[i];
                if (e < C && weaker(sc, tk, wsc, wtk)) { wsc = sc; wtk = tk; wsl = e; }
            }
            wave_weakest(wsc, wtk, wsl);
        }
        if (lane == 0) {
            wk_sc[wave] = wsc;
            wk_tk[wave] = wtk;
            wk_sl[wave] = wsl;
        }
    }

    // ---- this wave's chunks: online softmax.  The reference maximum of a head moves
    //      only when exceeded by more than 2^8 in the exponent, so p <= 256 and o is
    //      rarely rescaled; the final division by the sum cancels the choice exactly ----
    const float csc = kLog2e * rsqrtf(float(D));
    float m_ref = -INFINITY;       // reference max of head l16 (raw logits)
    float l_run = 0.0f;            // this lane's share of the running sum
    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{};
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    // nxt >= 0: the entry whose rows replace this chunk's in the same tiles, K as soon as
    // the q.k operands are read, V as soon as the p.v operands are
    auto consume = [&](int ent, u32x4* Kc, u32x4* Vc, int nxt) {
        uint32_t nroff[NL];
        if (nxt >= 0) chunk_rows(nxt, nroff);
        const bool is_ring = ent < nr;
        const int k0 = is_ring ? RW * ent : RW * head_chunk(ent - nr);   // first row / slot
        // visible rows of the chunk as a bit mask (lane j < 32 tests row k0 + j)
        const bool okj = is_ring ? ring_ok(k0 + (lane & 31)) : head_ok(k0 + (lane & 31));
        const uint32_t vmask = uint32_t(__ballot(okj));
        // rows holding the new token: ring slot t mod w, or sink slot t while t < s
        int pr = -1;
        if (is_ring) {
            // until the ring is full some of its slots were never written: zero their V
            // rows so that p = 0 meets finite values
            if (!ring_full) {
#pragma unroll
                for (int x = 0; x < NL; ++x) {
                    const int pidx = 64 * x + lane;
                    if (!((vmask >> (pidx / CPR)) & 1u)) Vc[pidx] = u32x4{};
                }
            }
            if (INGEST && t >= s) pr = tslot - k0;
        } else if (INGEST && t < s) {
            pr = t - k0;
        }
        if (INGEST && pr >= 0 && pr < RW && lane < CPR) {
            Kc[pr * CPR + (lane ^ kswz<D>(pr))] = nk;
            Vc[pr * CPR + (lane ^ vswz<D>(pr))] = nvv;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // s^T = K q^T: rows = keys 16mt + 4q16 + r of the chunk, column = head l16
        bf16x8 ka[2][KS];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int row = 16 * mt + l16;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                ka[mt][kk] = __builtin_bit_cast(
                    bf16x8, Kc[row * CPR + ((4 * kk + q16) ^ kswz<D>(row))]);
        }
        if (nxt >= 0) {
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the K tile is read
            __builtin_amdgcn_sched_barrier(0);
            load_k(nroff, Kc);
            __builtin_amdgcn_sched_barrier(0);
        }
        f32x4 sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = f32x4{};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) sacc[mt] = mfma16(ka[mt][kk], qf[kk], sacc[mt]);
        }
        if (vmask != 0xffffffffu) {
            const uint32_t lm = vmask >> (4 * q16);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (!((lm >> (16 * mt + r)) & 1u)) sacc[mt][r] = -INFINITY;
        }
        float mc = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                         fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
        mc = max_swap(mc);
        // NaN (both -inf: nothing visible yet) compares false: no move
        const bool move = (mc - m_ref) * csc > 8.0f;
        if (__ballot(move) != 0ull) {
            const float m_new = move ? mc : m_ref;
            const float alpha = move ? __builtin_amdgcn_exp2f((m_ref - m_new) * csc) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
            m_ref = m_new;
        }
        const float moff = (m_ref == -INFINITY) ? 0.0f : -m_ref * csc;
        // B operand element e: key 16(e/4) + 4q16 + e%4
        bf16x8 pf;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[mt][r], csc, moff));
                l_run += pe;
                pf[mt * 4 + r] = (__bf16)pe;
            }
        }
        // o^T += V^T p^T: rows = dims 16dt + 4q16 + r, column = head l16.  A operand
        // element e of lane (q16, i): V[16(e/4) + 4q16 + e%4][16dt + i], two transposing
        // reads of 4 keys; lane j of 16 reads key .. + j/4, dims 16dt + 4(j%4) .. +3
        bf16x8 va[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int key = 16 * r2 + 4 * q16 + (l16 >> 2);
                const int d0 = 16 * dt + 4 * (l16 & 3);
                const __bf16* src = reinterpret_cast<const __bf16*>(
                                        &Vc[key * CPR + ((d0 >> 3) ^ vswz<D>(key))]) + (d0 & 7);
                const v4i16 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16*)(src));
                const bf16x4 b4 = __builtin_bit_cast(bf16x4, t4);
#pragma unroll
                for (int e = 0; e < 4; ++e) va[dt][4 * r2 + e] = b4[e];
            }
        }
        if (nxt >= 0) {
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the V tile is read
            __builtin_amdgcn_sched_barrier(0);
            load_v(nroff, Vc);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] = mfma16(va[dt], pf, oacc[dt]);
    };
    bool xpend = xtra && wave == 0;
    for (int ent = ent0; ent < e_rr; ent += NW) {
        __builtin_amdgcn_s_waitcnt(0);        // this chunk's direct loads have landed
        consume(ent, Kt, Vt, ent + NW < e_rr ? ent + NW : -1);
        if (xpend) {                          // landed with the first chunk
            xpend = false;
            consume(e_hi - 1, Kx, Vx, -1);
        }
    }
    l_run = add_swap(l_run);
    // ---- this step's share of the deferred batch (wave-private LDS) ----------------------
    if (INGEST && t == u + w - 3) {
        __builtin_amdgcn_s_waitcnt(0);
        const int nchs = (t - 1 - u + kWaveScoreTile - 1) / kWaveScoreTile;
        for (int ch = sp * NW + wave; ch < nchs; ch += nsplit * NW)
            score_deferred_chunk<D>(c, bg, g, s, w, C, S, t, u, ch, k_t, v_t, cnn,
                                    reinterpret_cast<float*>(Kt), reinterpret_cast<float*>(Vt));
    }

    // ---- the waves' partials combine in LDS: wave wv's o [G][D] in its K region,
    //      (max, sum) of head h (log2 units) at 2h of its V region (the wave's own tiles,
    //      free once its last chunk and scorer rows are consumed) -------------------------
    if (l16 < G) {
        float* po = reinterpret_cast<float*>(Kt);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<f32x4*>(&po[l16 * D + 16 * dt + 4 * q16]) = oacc[dt];
        if (q16 == 0)
            *reinterpret_cast<f32x2*>(reinterpret_cast<float*>(Vt) + 2 * l16) =
                f32x2{m_ref == -INFINITY ? -INFINITY : m_ref * csc, l_run};
    }
    __syncthreads();
    // thread -> head hh, dims [d0, d0 + DPL); waves merged in order (deterministic)
    constexpr int NT = 64 * NW;
    constexpr int TPH0 = NT / G >= D ? D : NT / G;
    constexpr int TPH = TPH0 >= 64 ? (TPH0 >= 128 ? 128 : 64) : (TPH0 >= 32 ? 32 : 16);  // threads per head
    constexpr int DPL = D / TPH;                                 // 1, 2 or 4
    static_assert(TPH * G <= NT && DPL * TPH == D, "merge split");
    const bool active = tid < TPH * G;
    const int hh = active ? tid / TPH : 0;
    const int d0 = active ? (tid % TPH) * DPL : 0;
    float M = -INFINITY, L = 0.0f;
    float o[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = 0.0f;
    auto merge_in = [&](float ms, float ls, const float* ov) {
        const float Mn = fmaxf(M, ms);
        const float Ms = (Mn == -INFINITY) ? 0.0f : Mn;
        const float a = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Ms);
        const float f = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - Ms);
        L = L * a + f * ls;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = o[e] * a + f * ov[e];
        M = Mn;
    };
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
        const float* po = reinterpret_cast<const float*>(Ks[wv]);
        const float* pm = reinterpret_cast<const float*>(Vs[wv]);
        float ov[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) ov[e] = po[hh * D + d0 + e];
        merge_in(pm[2 * hh], pm[2 * hh + 1], ov);
    }
    // the weakest entry of the post-step segment over the waves' candidates (tokens are
    // distinct, so the order is total and any reduction order gives the same entry);
    // only wave 0 commits
    float wsc = INFINITY;
    int wtk = -1, wsl = -1;
    if (INGEST && wave == 0) {
        if (lane < NW) {
            wsc = wk_sc[lane];
            wtk = wk_tk[lane];
            wsl = wk_sl[lane];
        }
        wave_weakest(wsc, wtk, wsl);
    }

    if (nsplit > 1) {
        // ---- split partial out, coherent; the last workgroup of (b, g) merges the
        //      splits in split order and finishes the step --------------------------------
        __amdgpu_buffer_rsrc_t prs = part_rsrc(part + long(bg) * nsplit * PW);
        if (active) {
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[e]), prs,
                                                      (sp * PW + hh * D + d0 + e) * 4, 0, kSc1);
            if (d0 == 0)
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f32x2{M, L}), prs,
                                                      (sp * PW + G * D + 2 * hh) * 4, 0, kSc1);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);        // partials and scores complete
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();
        if (tid == 0) {
            const int old = __hip_atomic_fetch_add(c.arrive + bg, 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            last_flag = (old == nsplit - 1) ? 1 : 0;
        }
        __syncthreads();
        if (last_flag == 0) return;
        M = -INFINITY;
        L = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = 0.0f;
        constexpr int CH = 8;                     // splits loaded per round
        for (int c0 = 0; c0 < nsplit; c0 += CH) {
            f32x2 ml[CH];
            float ov[CH][DPL];
#pragma unroll
            for (int qq = 0; qq < CH; ++qq) {
                const int pb = min(c0 + qq, nsplit - 1) * PW;
                ml[qq] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                       prs, (pb + G * D + 2 * hh) * 4, 0, kSc1));
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    ov[qq][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        prs, (pb + hh * D + d0 + e) * 4, 0, kSc1));
            }
#pragma unroll
            for (int qq = 0; qq < CH; ++qq)   // splits past the last weigh in as nothing
                merge_in((c0 + qq < nsplit) ? ml[qq][0] : -INFINITY, ml[qq][1], ov[qq]);
        }
    }

    // ---- the ingest (its stores wait on nothing outstanding), then o_t -------------------
    if (INGEST && wave == 0) {
        // the leaving token's row into its segment slot; no workgroup reads that slot's
        // old contents in this step, and every read of the ring slot is complete
        if (X >= 0 && lane < CPR) {
            const long dst = base + long(s + X) * D + lane * 8;
            *reinterpret_cast<u32x4*>(c.k + dst) = lk;
            *reinterpret_cast<u32x4*>(c.v + dst) = lv;
        }
        ingest_commit<D>(c, bg, s, w, C, S, t, cnt, X, rl, u, wsl, wsc, r1, nk, nvv);
    }
    if (active) {
        const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
        __bf16* orow = reinterpret_cast<__bf16*>(out_t) + (long(b) * Hq + g * G + hh) * D + d0;
#pragma unroll
        for (int e = 0; e < DPL; ++e) orow[e] = (__bf16)(o[e] * inv);
    }
    if (nsplit > 1 && tid == 0)
        __hip_atomic_store(c.arrive + bg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_score_evict(const Shape& sh, const lte_cnn& cnn, const uint16_t* k_t,
                              const uint16_t* v_t, const CacheView& cache, hipStream_t st) {
    dim3 grid(unsigned(sh.B * sh.Hkv));
    if (sh.D == 128) {
        hipLaunchKernelGGL(score_evict_kernel<128>, grid, dim3(64), 0, st, sh.s, sh.w, sh.C,
                           sh.S, sh.Hkv, k_t, v_t, cnn, cache);
    } else {
        hipLaunchKernelGGL(score_evict_kernel<64>, grid, dim3(64), 0, st, sh.s, sh.w, sh.C,
                           sh.S, sh.Hkv, k_t, v_t, cnn, cache);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const Shape& sh, bool ingest, const uint16_t* q_t, const uint16_t* k_t,
                         const uint16_t* v_t, const lte_cnn* cnn, const CacheView& cache,
                         float* part, uint16_t* out_t, hipStream_t st) {
    const int nsplit = decode_nsplit(sh);
    dim3 grid(unsigned(sh.B * sh.Hkv * nsplit));
    lte_cnn cn{};
    if (cnn != nullptr) cn = *cnn;
#define LTE_DECODE_G(DD, GG, ING)                                                               \
    case GG:                                                                                    \
        hipLaunchKernelGGL((decode_step_kernel<DD, GG, ING>), grid, dim3(64 * kDecodeWaves), 0, st,       \
                           sh.Hq, sh.Hkv, sh.s, sh.w, sh.C, sh.S, nsplit, q_t, k_t, v_t, cn,     \
                           cache, part, out_t);                                                 \
        break;
#define LTE_DECODE(DD, ING)                                                                     \
    switch (sh.G) {                                                                             \
        LTE_DECODE_G(DD, 1, ING)                                                                \
        LTE_DECODE_G(DD, 2, ING)                                                                \
        LTE_DECODE_G(DD, 4, ING)                                                                \
        LTE_DECODE_G(DD, 8, ING)                                                                \
        LTE_DECODE_G(DD, 16, ING)                                                               \
        default: return hipErrorInvalidValue;                                                   \
    }
    if (sh.D == 128) {
        if (ingest) { LTE_DECODE(128, true) } else { LTE_DECODE(128, false) }
    } else {
        if (ingest) { LTE_DECODE(64, true) } else { LTE_DECODE(64, false) }
    }
#undef LTE_DECODE_G
#undef LTE_DECODE
    return hipGetLastError();
}

}  // namespace lte
