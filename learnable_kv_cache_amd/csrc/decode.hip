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
// A decode step is one launch of one-wave workgroups, one per 64 cache
// slots of a (batch, KV head):
//   * each reads its slots in the PRE-step state with the post-ingest
//     contents substituted: ring slot t mod w (and sink slot t) come from the
//     k_t/v_t inputs, and the segment slot the leaving token takes reads that
//     token from its ring slot (that wave also copies the row into the slot:
//     no other wave reads it).  K rows go straight into MFMA operand
//     registers; V rows are loaded into LDS by direct global->LDS loads and
//     read back transposed (ds_read_b64_tr_b16).  q.k and p.v run on
//     v_mfma_f32_16x16x32_bf16 with the G <= 16 query heads of the KV head
//     as the 16 columns;
//   * on a scoring step the waves of a (batch, KV head) share the deferred
//     batch, 28 tokens per wave call;
//   * each wave writes (max, sum, unnormalised o) per head with device-scope
//     coherent stores and counts itself in on the (batch, KV head)'s arrival
//     word; the last to arrive merges the partials in split order
//     (deterministic), writes o_t, applies the rest of the ingest, records
//     the next decision and clears the arrival word.  The partials bypass
//     the non-coherent L2 copies instead of a cache-wide write-back and
//     invalidate, which a device-scope fence would cost on gfx950.
#include "score_core.h"

namespace lte {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int KPB = 64;                        // cache slots per wave
constexpr int NWV = kDecodeSplitKeys / KPB;    // waves per workgroup (2)

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
                                     float* Y) {
    const uint16_t* kring = c.k + (long(bg) * S + s + C) * D;
    const uint16_t* vring = c.v + (long(bg) * S + s + C) * D;
    float* rs = c.ring_score + long(bg) * w;
    score_wave<D>(
        Y, cnn.w1 + long(g) * kHidden * 2 * D * 3, cnn.b1 + g * kHidden,
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
    __shared__ __align__(16) float Y[kWaveScoreBytes / 4];
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
            score_deferred_chunk<D>(c, bg, bg % Hkv, s, w, C, S, t, u, ch, k_t, v_t, cnn, Y);
    }
    __builtin_amdgcn_s_waitcnt(0);            // ring row copied before it is overwritten
    ingest_commit<D>(c, bg, s, w, C, S, t, cnt, X, rl, u, wsl, wsc, r1, nk, nv);
}

// One decode step (INGEST) or an attention over the cache as it is.
template <int D, int G, bool INGEST>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(3)))
void decode_step_kernel(
    int Hq, int Hkv, int s, int w, int C, int S, int nsplit,
    const uint16_t* __restrict__ q_t, const uint16_t* __restrict__ k_t,
    const uint16_t* __restrict__ v_t, lte_cnn cnn, CacheView c, float* __restrict__ part,
    uint16_t* __restrict__ out_t) {
    constexpr int KS = D / 32;                 // q.k k-steps
    constexpr int DT = D / 16;                 // p.v output tiles
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int kVBytes = KPB * CPR * 16;
    constexpr int kBuf = kVBytes > kWaveScoreBytes ? kVBytes : kWaveScoreBytes;
    // per wave: its V tile; later its scorer rows (and wave 1's partial for wave 0,
    // then the last-arrival flag).  32 KB: five workgroups fit a CU.
    __shared__ __align__(16) u32x4 Vs[NWV][kBuf / 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int q16 = lane >> 4;
    const int sp = blockIdx.x % nsplit;
    const int bg = blockIdx.x / nsplit;
    const int b = bg / Hkv;
    const int g = bg % Hkv;
    const int slot0 = (sp * NWV + wave) * KPB;
    u32x4* Vw = Vs[wave];
    const long base = long(bg) * S * D;

    // ---- bulk loads first: the V tile (direct to LDS), q (B operand) and the K
    //      rows (A operands of q.k), in the pre-step state -------------------------------
#pragma unroll
    for (int x = 0; x < CPR; ++x) {
        const int cidx = 64 * x + lane;
        const int row = cidx / CPR;
        const int gch = (cidx % CPR) ^ vswz<D>(row);
        const uint16_t* src = c.v + base + long(min(slot0 + row, S - 1)) * D + gch * 8;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(&Vw[64 * x]),
                                         16, 0, 0);
    }
    bf16x8 qf[KS];
    {
        const bool hv = l16 < G;
        const uint16_t* qrow = q_t + (long(b) * Hq + g * G + (hv ? l16 : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            qf[kk] = hv ? *reinterpret_cast<const bf16x8*>(qrow + 32 * kk + 8 * q16) : bf16x8{};
    }
    bf16x8 ka[4][KS];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const uint16_t* r = c.k + base + long(min(slot0 + 16 * mt + l16, S - 1)) * D;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            ka[mt][kk] = *reinterpret_cast<const bf16x8*>(r + 32 * kk + 8 * q16);
    }

    // ---- the state, loaded alongside (positions fit in 32 bits) ----------------------
    const int p = int(c.pos[bg]);
    const int cnt = c.count[bg];
    const int X = INGEST ? c.nx_slot[bg] : -1;
    const int u = INGEST ? int(c.next_unscored[bg]) : 0;
    const float rl = INGEST ? c.nx_score[bg] : 0.0f;
    const int t = INGEST ? p : p - 1;
    const int tslot = t >= 0 ? t % w : 0;
    const int new_cnt = (X >= 0 && X == cnt) ? cnt + 1 : cnt;
    // ingest operands every wave fetches (the last to arrive commits them): the new
    // token's row chunk, the score of the token leaving next, and the weakest of this
    // split's segment entries in the post-step state (slot X holding the newcomer)
    u32x4 nk = u32x4{}, nv = u32x4{};
    float r1 = 0.0f;
    float wsc = INFINITY;
    int wtk = -1, wsl = -1;
    if (INGEST) {
        if (lane < CPR) {
            nk = *reinterpret_cast<const u32x4*>(k_t + long(bg) * D + lane * 8);
            nv = *reinterpret_cast<const u32x4*>(v_t + long(bg) * D + lane * 8);
        }
        if (t + 1 - w >= s) r1 = c.ring_score[long(bg) * w + (t + 1) % w];
        const int e = slot0 + lane - s;
        if (C > 0 && new_cnt == C && e >= 0 && e < C) {
            wsc = (e == X) ? rl : c.ret_score[long(bg) * C + e];
            wtk = (e == X) ? t - w : c.ret_idx[long(bg) * C + e];
            wsl = e;
        }
    }

    // rows that differ in the post-ingest state: the new token (ring slot t mod w and,
    // while t < s, sink slot t) comes from the inputs; segment slot X holds the leaving
    // token, still in ring slot t mod w.  At most three slots, each checked once.
    int fs[3] = {-1, -1, -1};
    if (INGEST) {
        fs[0] = t < s ? t : -1;
        fs[1] = X >= 0 ? s + X : -1;
        fs[2] = s + C + tslot;
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            const int kk = fs[f] - slot0;                     // wave-uniform
            if (fs[f] < 0 || kk < 0 || kk >= KPB || fs[f] >= S) continue;
            const uint16_t* rk = (f == 1) ? c.k + base + long(s + C + tslot) * D : k_t + long(bg) * D;
            if (l16 == (kk & 15)) {                           // q.k A operand rows
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    if (mt == (kk >> 4)) {
#pragma unroll
                        for (int kq = 0; kq < KS; ++kq)
                            ka[mt][kq] = *reinterpret_cast<const bf16x8*>(rk + 32 * kq + 8 * q16);
                    }
                }
            }
        }
    }
    // validity of the 64 slots as a wave-wide bit mask (lane k tests slot slot0 + k)
    uint64_t vmask;
    {
        const int cs = slot0 + lane;
        bool ok = false;
        if (cs < S && t >= 0) {
            if (cs < s) {
                ok = cs <= t;
            } else if (cs < s + C) {
                ok = (cs - s) < new_cnt;
            } else {
                // ring slot r holds token t - d, d = (tslot - r) mod w: valid when >= s
                const int r = cs - s - C;
                const int d = (r <= tslot) ? tslot - r : tslot - r + w;
                ok = d <= t - s;
            }
        }
        vmask = __ballot(ok);
    }

    // the wave owning the slot the leaving token takes also moves its row there
    if (INGEST && X >= 0) {
        const int lr = s + X - slot0;
        if (lr >= 0 && lr < KPB && lane < D / 8) {
            const long rr = base + long(s + C + tslot) * D + lane * 8;
            const long dst = base + long(s + X) * D + lane * 8;
            *reinterpret_cast<uint4*>(c.k + dst) = *reinterpret_cast<const uint4*>(c.k + rr);
            *reinterpret_cast<uint4*>(c.v + dst) = *reinterpret_cast<const uint4*>(c.v + rr);
        }
    }

    // ---- s^T = K q^T: rows = keys 16mt + 4q16 + r, column = head l16 -----------------
    f32x4 sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        sacc[mt] = f32x4{};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) sacc[mt] = mfma16(ka[mt][kk], qf[kk], sacc[mt]);
    }
    const float csc = kLog2e * rsqrtf(float(D));
    float x[4][4];
    float m = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool ok = (vmask >> (16 * mt + 4 * q16 + r)) & 1ull;
            x[mt][r] = ok ? sacc[mt][r] * csc : -INFINITY;
            m = fmaxf(m, x[mt][r]);
        }
    }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    const float msafe = (m == -INFINITY) ? 0.0f : m;
    // p = p_hi + p_lo, both bf16: the P.V product keeps ~16 mantissa bits of p.
    // B operand of chunk cc, element e: key 32cc + 16(e/4) + 4q16 + e%4
    float l = 0.0f;
    bf16x8 pf[2], pl[2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pr = __builtin_amdgcn_exp2f(x[mt][r] - msafe);
            l += pr;
            const __bf16 hi = (__bf16)pr;
            pf[mt >> 1][(mt & 1) * 4 + r] = hi;
            pl[mt >> 1][(mt & 1) * 4 + r] = (__bf16)(pr - float(hi));
        }
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);

    // ---- V tile landed; substituted rows overwrite theirs --------------------------------
    __builtin_amdgcn_s_waitcnt(0);
    if (INGEST) {
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            const int kk = fs[f] - slot0;
            if (fs[f] < 0 || kk < 0 || kk >= KPB || fs[f] >= S) continue;
            const uint16_t* rv = (f == 1) ? c.v + base + long(s + C + tslot) * D : v_t + long(bg) * D;
            if (lane < CPR)
                Vw[kk * CPR + lane] = *reinterpret_cast<const u32x4*>(rv + 8 * (lane ^ vswz<D>(kk)));
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- o^T = V^T p^T: rows = dims 16dt + 4q16 + r, column = head l16.  A operand
    //      element e of lane (q16, i): V[32cc + 16(e/4) + 4q16 + e%4][16dt + i], two
    //      transposing reads of 4 keys; lane j of the 16 reads key .. + j/4, dims
    //      16dt + 4(j%4) .. +3 --------------------------------------------------------------
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        oacc[dt] = f32x4{};
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            bf16x8 a;
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int key = 32 * cc + 16 * r2 + 4 * q16 + (l16 >> 2);
                const int d0 = 16 * dt + 4 * (l16 & 3);
                const __bf16* src = reinterpret_cast<const __bf16*>(
                                        &Vw[key * CPR + ((d0 >> 3) ^ vswz<D>(key))]) + (d0 & 7);
                const v4i16 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16*)(src));
                const bf16x4 b4 = __builtin_bit_cast(bf16x4, t4);
#pragma unroll
                for (int e = 0; e < 4; ++e) a[4 * r2 + e] = b4[e];
            }
            oacc[dt] = mfma16(a, pf[cc], oacc[dt]);
            oacc[dt] = mfma16(a, pl[cc], oacc[dt]);
        }
    }
    // ---- the waves' partials combine into one per workgroup: o [G][D] at 0, (max, sum)
    //      of head h at G*D + 2h, the weakest segment entry at G*D + 2G -----------------
    constexpr int kPart = decode_part_floats(G, D);             // floats per split
    __amdgpu_buffer_rsrc_t prs = part_rsrc(part + long(bg) * nsplit * kPart);
    if (INGEST) wave_weakest(wsc, wtk, wsl);
    float* xw = reinterpret_cast<float*>(Vs[1]);               // wave 1's, read by now
    if (wave == 1) {
        if (l16 < G) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *reinterpret_cast<f32x4*>(&xw[l16 * D + 16 * dt + 4 * q16]) = oacc[dt];
            if (q16 == 0) *reinterpret_cast<f32x2*>(&xw[G * D + 2 * l16]) = f32x2{m, l};
        }
        if (INGEST && lane == 0)
            *reinterpret_cast<u32x4*>(&xw[G * D + 2 * G]) =
                u32x4{__float_as_uint(wsc), uint32_t(wtk), uint32_t(wsl), 0u};
    }
    __syncthreads();
    if (wave == 0) {
        const int pbase = sp * kPart * 4;                          // bytes
        if (l16 < G) {
            const f32x2 ml1 = *reinterpret_cast<const f32x2*>(&xw[G * D + 2 * l16]);
            const float Mn = fmaxf(m, ml1[0]);
            const float Ms = (Mn == -INFINITY) ? 0.0f : Mn;
            const float a0 = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - Ms);
            const float a1 = (ml1[0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ml1[0] - Ms);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const f32x4 o1 = *reinterpret_cast<const f32x4*>(&xw[l16 * D + 16 * dt + 4 * q16]);
                const f32x4 o4 = oacc[dt] * a0 + o1 * a1;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o4), prs,
                                                       pbase + (l16 * D + 16 * dt + 4 * q16) * 4,
                                                       0, kSc1);
            }
            if (q16 == 0) {
                const f32x2 ml = {Mn, l * a0 + ml1[1] * a1};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ml), prs,
                                                      pbase + (G * D + 2 * l16) * 4, 0, kSc1);
            }
        }
        if (INGEST && lane == 0) {
            const u32x4 w1 = *reinterpret_cast<const u32x4*>(&xw[G * D + 2 * G]);
            if (weaker(__uint_as_float(w1[0]), int(w1[1]), wsc, wtk)) {
                wsc = __uint_as_float(w1[0]);
                wtk = int(w1[1]);
                wsl = int(w1[2]);
            }
            const u32x4 wt = {__float_as_uint(wsc), uint32_t(wtk), uint32_t(wsl), 0u};
            __builtin_amdgcn_raw_buffer_store_b128(wt, prs, pbase + (G * D + 2 * G) * 4, 0, kSc1);
        }
    }

    // ---- this step's share of the deferred batch ---------------------------------------
    if (INGEST && t == u + w - 3) {
        __syncthreads();                          // wave 1's partial read: its rows are free
        float* Y = reinterpret_cast<float*>(Vw);
        const int nch = (t - 1 - u + kWaveScoreTile - 1) / kWaveScoreTile;
        for (int ch = sp * NWV + wave; ch < nch; ch += nsplit * NWV)
            score_deferred_chunk<D>(c, bg, g, s, w, C, S, t, u, ch, k_t, v_t, cnn, Y);
    }

    // ---- arrival: the last workgroup of (b, g) merges and finishes the step ---------------
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);            // partials, row copies, scores complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    int* last_arrival = reinterpret_cast<int*>(Vs[1]);        // every LDS use is over
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(c.arrive + bg, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        *last_arrival = (old == nsplit - 1) ? 1 : 0;
    }
    __syncthreads();
    if (*last_arrival == 0) return;

    // the splits' weakest segment entries, loaded alongside the first merge round
    u32x4 wt0 = u32x4{__float_as_uint(INFINITY), ~0u, ~0u, 0u};
    if (INGEST && wave == 0 && lane < nsplit)
        wt0 = __builtin_amdgcn_raw_buffer_load_b128(prs, lane * kPart * 4 + (G * D + 2 * G) * 4,
                                                    0, kSc1);
    // merge: thread handles head hh = tid / TPH, dims [d0, d0 + DPL), online over the
    // splits in split order; coherent loads CH splits at a time
    {
        constexpr int NT = 64 * NWV;
        constexpr int TPH = (G * D >= NT ? NT : G * D) / G;      // threads per head
        constexpr int DPL = D / TPH;              // dims per thread: 1, 2 or a multiple of 4
        constexpr int NQ = DPL >= 4 ? DPL / 4 : 1;        // loads of o per split
        constexpr int CH = 96 / (DPL + 2) > 0 ? 96 / (DPL + 2) : 1;   // splits per round
        const bool active = tid < TPH * G;
        const int hh = active ? tid / TPH : 0;
        const int d0 = active ? (tid % TPH) * DPL : 0;
        float M = -INFINITY, L = 0.0f;
        float o[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = 0.0f;
        for (int c0 = 0; c0 < nsplit; c0 += CH) {
            f32x2 ml[CH];
            f32x4 ov[CH][NQ];
#pragma unroll
            for (int q = 0; q < CH; ++q) {
                const int pb = min(c0 + q, nsplit - 1) * kPart * 4;
                ml[q] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                      prs, pb + (G * D + 2 * hh) * 4, 0, kSc1));
#pragma unroll
                for (int e = 0; e < NQ; ++e) {
                    const int off = pb + (hh * D + d0 + 4 * e) * 4;
                    if (DPL >= 4) {
                        ov[q][e] = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, kSc1));
                    } else if (DPL == 2) {
                        const f32x2 t2 = __builtin_bit_cast(
                            f32x2, __builtin_amdgcn_raw_buffer_load_b64(prs, off, 0, kSc1));
                        ov[q][e] = f32x4{t2[0], t2[1], 0.0f, 0.0f};
                    } else {
                        const float t1 = __builtin_bit_cast(
                            float, __builtin_amdgcn_raw_buffer_load_b32(prs, off, 0, kSc1));
                        ov[q][e] = f32x4{t1, 0.0f, 0.0f, 0.0f};
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < CH; ++q) {
                // splits past the last one re-read it and weigh in as nothing
                const float ms = (c0 + q < nsplit) ? ml[q][0] : -INFINITY;
                const float ls = ml[q][1];
                const float Mn = fmaxf(M, ms);
                const float Ms = (Mn == -INFINITY) ? 0.0f : Mn;
                const float a = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Ms);
                const float f = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - Ms);
                L = L * a + f * ls;
#pragma unroll
                for (int e = 0; e < DPL; ++e) o[e] = o[e] * a + f * ov[q][e / 4][e % 4];
                M = Mn;
            }
        }
        const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
        __bf16* orow = reinterpret_cast<__bf16*>(out_t) + (long(b) * Hq + g * G + hh) * D + d0;
        if (active) {
#pragma unroll
            for (int e = 0; e < DPL; ++e) orow[e] = (__bf16)(o[e] * inv);
        }
    }
    if (INGEST && wave == 0) {
        // weakest of the post-step segment: over the splits' weakest entries
        float bs = __uint_as_float(wt0[0]);
        int bt = int(wt0[1]), bl = int(wt0[2]);
        for (int q = lane + 64; q < nsplit; q += 64) {
            const u32x4 wt = __builtin_amdgcn_raw_buffer_load_b128(
                prs, q * kPart * 4 + (G * D + 2 * G) * 4, 0, kSc1);
            const float sc = __uint_as_float(wt[0]);
            if (weaker(sc, int(wt[1]), bs, bt)) { bs = sc; bt = int(wt[1]); bl = int(wt[2]); }
        }
        wave_weakest(bs, bt, bl);
        ingest_commit<D>(c, bg, s, w, C, S, t, cnt, X, rl, u, bl, bs, r1, nk, nv);
    }
    if (tid == 0) __hip_atomic_store(c.arrive + bg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        hipLaunchKernelGGL((decode_step_kernel<DD, GG, ING>), grid, dim3(64 * NWV), 0, st,       \
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
