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
// A decode step is two launches and no device-scope fence:
//   decode_split_kernel   one wave per 64 cache slots, reading them in the
//       PRE-step state with the post-ingest contents substituted: ring slot
//       t mod w (and sink slot t) come from the k_t/v_t inputs, and the
//       segment slot the leaving token takes reads that token from its ring
//       slot (that wave also copies the row into the slot: no other wave
//       reads it).  q.k and p.v run on v_mfma_f32_16x16x32_bf16 with the
//       G <= 16 query heads of the KV head as the 16 columns; the wave writes
//       (max, sum, unnormalised o) per head.
//   decode_finish_kernel  one workgroup per (batch, KV head): merges the
//       partials in split order (deterministic), writes o_t, then applies the
//       rest of the ingest and records the next decision.
// (Merging inside one launch would need an agent-scope fence per workgroup,
// which on gfx950 writes back and invalidates the XCD's L2.)
#include "score_core.h"

namespace lte {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxG = 16;
constexpr int KPB = kDecodeSplitKeys;          // cache slots per split (64)

// v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16]
// and D[4(l/16)+r][l%16].
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Position of key k (0..63 within a split) in the V^T rows: keys are permuted
// inside each 32-key chunk so that lane group q of the P.V MFMA reads its 8
// keys {4q..4q+3, 16+4q..16+4q+3} -- the rows of the q.k output it holds --
// as one 16-byte run.
__device__ __forceinline__ int vt_pos(int k) {
    const int cc = k >> 5;
    const int kc = k & 31;
    const int hi = kc >> 4;            // second 16-key tile of the chunk
    const int q = (kc & 15) >> 2;
    const int e = (kc & 3) + 4 * hi;
    return 32 * cc + 8 * q + e;
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

// Finishes an ingest of token t in the cache of one (b, g), given the state
// the caller read before any write (cnt, X = nx_slot, rl = nx_score, u, wk,
// wscore = ret_score[wk]).  Run by one whole workgroup of 256 threads.
// copy_row: also move the leaving token's row into segment slot X (the
// split kernel did it already on the decode-step path).
template <int D>
__device__ void ingest_finish(const CacheView& c, int bg, int g, int s, int w, int C, int S,
                              int64_t t, int cnt, int X, float rl, int64_t u, int wk, float wscore,
                              bool copy_row, const uint16_t* __restrict__ k_t,
                              const uint16_t* __restrict__ v_t, const lte_cnn& cnn,
                              unsigned char* smem, float* w2s, float* red_s, int* red_t,
                              int* red_x) {
    constexpr int KK = ScoreSmem<D>::KK;
    constexpr int NW = ScoreSmem<D>::NW;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tslot = int(t % w);
    const int ring0 = s + C;
    const long ring_row = (long(bg) * S + ring0 + tslot) * D;
    const int64_t jl = t - w;
    const int new_cnt = (X >= 0 && X == cnt) ? cnt + 1 : cnt;
    // score of token t+1-w, which leaves at the next ingest: scored at least three
    // steps before it leaves, never by this step's batch
    const int64_t t1 = t + 1;
    const float r1 = (t1 - w >= s) ? c.ring_score[long(bg) * w + int(t1 % w)] : 0.0f;

    if (tid < D / 8) {       // same thread reads the ring chunk before overwriting it
        const int ch = tid;
        const uint4 kv = *reinterpret_cast<const uint4*>(k_t + long(bg) * D + ch * 8);
        const uint4 vv = *reinterpret_cast<const uint4*>(v_t + long(bg) * D + ch * 8);
        if (copy_row && X >= 0) {
            const uint4 lk = *reinterpret_cast<const uint4*>(c.k + ring_row + ch * 8);
            const uint4 lv = *reinterpret_cast<const uint4*>(c.v + ring_row + ch * 8);
            const long dst = (long(bg) * S + s + X) * D + ch * 8;
            *reinterpret_cast<uint4*>(c.k + dst) = lk;
            *reinterpret_cast<uint4*>(c.v + dst) = lv;
        }
        *reinterpret_cast<uint4*>(c.k + ring_row + ch * 8) = kv;
        *reinterpret_cast<uint4*>(c.v + ring_row + ch * 8) = vv;
        if (t < s) {
            const long srow = (long(bg) * S + t) * D + ch * 8;
            *reinterpret_cast<uint4*>(c.k + srow) = kv;
            *reinterpret_cast<uint4*>(c.v + srow) = vv;
        }
    }
    if (tid == 0) {
        if (X >= 0) {
            c.ret_idx[long(bg) * C + X] = int(jl);
            c.ret_score[long(bg) * C + X] = rl;
            c.count[bg] = new_cnt;
        }
        if (X == -2) c.flags[bg] |= 1;
        c.ring_score[long(bg) * w + tslot] = __builtin_nanf("");
    }

    // weakest entry of a full segment, with slot X already holding the newcomer
    int wk2 = wk;
    float ws2 = wscore;
    if (X >= 0 && new_cnt == C) {
        float bs = INFINITY;
        int bt = -1, bx = -1;
        for (int x = tid; x < C; x += 256) {
            float sc;
            int tk;
            if (x == X) {
                sc = rl;
                tk = int(jl);
            } else {
                sc = c.ret_score[long(bg) * C + x];
                tk = c.ret_idx[long(bg) * C + x];
            }
            if (sc < bs || (sc == bs && tk > bt)) { bs = sc; bt = tk; bx = x; }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float os = __shfl_xor(bs, o, 64);
            const int ot = __shfl_xor(bt, o, 64);
            const int ox = __shfl_xor(bx, o, 64);
            if (os < bs || (os == bs && ot > bt)) { bs = os; bt = ot; bx = ox; }
        }
        if (lane == 0) { red_s[wave] = bs; red_t[wave] = bt; red_x[wave] = bx; }
        __syncthreads();
        bs = red_s[0]; bt = red_t[0]; bx = red_x[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            if (red_s[q] < bs || (red_s[q] == bs && red_t[q] > bt)) {
                bs = red_s[q]; bt = red_t[q]; bx = red_x[q];
            }
        }
        wk2 = bx;
        ws2 = bs;
        if (tid == 0) c.weak[bg] = bx;
    }

    int64_t u2 = u;
    if (t == u + w - 3) {                             // deferred batched scoring
        __threadfence_block();
        __syncthreads();                              // ring row of token t written
        for (int x = tid; x < kHidden * 3; x += 256) w2s[x] = cnn.w2[g * kHidden * 3 + x];
        const uint16_t* kring = c.k + (long(bg) * S + ring0) * D;
        const uint16_t* vring = c.v + (long(bg) * S + ring0) * D;
        float* rs = c.ring_score + long(bg) * w;
        const int tt = int(t);
        for (int t0 = int(u); t0 <= tt - 2; t0 += kScoreTile) {
            bf16x8* wl = reinterpret_cast<bf16x8*>(smem);     // W1 as packed bf16 operands
            for (int x = tid; x < NW; x += 256) {
                int tap, kk, ln;
                w1p_coords(x, KK, tap, kk, ln);
                const float* src = cnn.w1 +
                    ((long(g) * kHidden + ln % 32) * (2 * D) + kk * 16 + (ln / 32) * 8) * 3 + tap;
                bf16x8 e8;
#pragma unroll
                for (int e = 0; e < 8; ++e) e8[e] = (__bf16)src[e * 3];
                wl[x] = e8;
            }
            score_chunk<D>(
                smem, w2s, cnn.b1 + g * kHidden, cnn.b2[g], t0, int(u), tt - 2,
                [&](int x, const uint16_t*& kp, const uint16_t*& vp) {
                    if (x < 0 || x > tt) return false;
                    kp = kring + long(x % w) * D;
                    vp = vring + long(x % w) * D;
                    return true;
                },
                [&](int x) { return x < 0; },
                [&](int tok, float r) { rs[tok % w] = r; });
        }
        u2 = t - 1;
    }
    // the next ingest's decision
    if (tid == 0) {
        c.nx_slot[bg] = decide_slot(t1, r1, new_cnt, wk2, ws2, s, w, C);
        c.nx_score[bg] = r1;
        c.next_unscored[bg] = u2;
        c.pos[bg] = t1;
    }
}

template <int D>
__global__ __launch_bounds__(256) void score_evict_kernel(int s, int w, int C, int S, int Hkv,
                                                          const uint16_t* __restrict__ k_t,
                                                          const uint16_t* __restrict__ v_t,
                                                          lte_cnn cnn, CacheView c) {
    __shared__ __align__(16) unsigned char smem[ScoreSmem<D>::kBytes];
    __shared__ float w2s[kHidden * 3];
    __shared__ float red_s[4];
    __shared__ int red_t[4], red_x[4];
    const int bg = blockIdx.x;
    const int64_t t = c.pos[bg];
    const int cnt = c.count[bg];
    const int X = c.nx_slot[bg];
    const float rl = c.nx_score[bg];
    const int64_t u = c.next_unscored[bg];
    const int wk = c.weak[bg];
    const float ws = (wk >= 0) ? c.ret_score[long(bg) * C + wk] : 0.0f;
    __syncthreads();                       // every thread has read the pre-step state
    ingest_finish<D>(c, bg, bg % Hkv, s, w, C, S, t, cnt, X, rl, u, wk, ws, true, k_t, v_t, cnn,
                     smem, w2s, red_s, red_t, red_x);
}

// Attention partials of one split of 64 cache slots; one wave.
template <int D, bool INGEST>
__global__ __launch_bounds__(64) void decode_split_kernel(
    int Hq, int Hkv, int G, int s, int w, int C, int S, int nsplit,
    const uint16_t* __restrict__ q_t, const uint16_t* __restrict__ k_t,
    const uint16_t* __restrict__ v_t, CacheView c, float* __restrict__ part) {
    constexpr int KS = D / 32;                 // q.k k-steps
    constexpr int DT = D / 16;                 // p.v output tiles
    constexpr int NU = D / 32;                 // V transpose units per lane
    constexpr int VST = KPB + 8;               // V^T row stride (bf16), padded
    __shared__ __align__(16) __bf16 Vt[D * VST];

    const int lane = threadIdx.x;
    const int l16 = lane & 15;
    const int q16 = lane >> 4;
    const int sp = blockIdx.x % nsplit;
    const int bg = blockIdx.x / nsplit;
    const int b = bg / Hkv;
    const int g = bg % Hkv;
    const int slot0 = sp * KPB;

    const long base = long(bg) * S * D;

    // ---- bulk loads first: q (B operand), and every slot's row of the cache as it
    //      is (A operands of q.k; V transpose units) -- none waits for the state ----
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
    uint4 vr[NU][4];
#pragma unroll
    for (int uu = 0; uu < NU; ++uu) {
        const int U = lane + 64 * uu;
        const int kg = U / (D / 8);            // 4 keys 4kg .. 4kg+3
        const int dg = U % (D / 8);            // 8 dims 8dg .. 8dg+7
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
            vr[uu][k4] = *reinterpret_cast<const uint4*>(
                c.v + base + long(min(slot0 + 4 * kg + k4, S - 1)) * D + 8 * dg);
    }

    // ---- the state, loaded alongside (positions fit in 32 bits) ----------------------
    const int p = int(c.pos[bg]);
    const int cnt = c.count[bg];
    const int X = INGEST ? c.nx_slot[bg] : -1;
    const int t = INGEST ? p : p - 1;
    const int tslot = t >= 0 ? t % w : 0;
    const int new_cnt = (X >= 0 && X == cnt) ? cnt + 1 : cnt;

    // rows that differ in the post-ingest state: the new token (ring slot t mod w and,
    // while t < s, sink slot t) comes from the inputs; segment slot X holds the leaving
    // token, still in ring slot t mod w.  At most three slots, each checked once.
    if (INGEST) {
        const int fs[3] = {t < s ? t : -1, X >= 0 ? s + X : -1, s + C + tslot};
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            const int kk = fs[f] - slot0;                     // wave-uniform
            if (fs[f] < 0 || kk < 0 || kk >= KPB || fs[f] >= S) continue;
            const uint16_t* rk = (f == 1) ? c.k + base + long(s + C + tslot) * D : k_t + long(bg) * D;
            const uint16_t* rv = (f == 1) ? c.v + base + long(s + C + tslot) * D : v_t + long(bg) * D;
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
#pragma unroll
            for (int uu = 0; uu < NU; ++uu) {                 // V transpose units
                const int U = lane + 64 * uu;
                if (U / (D / 8) == (kk >> 2)) {
                    const uint4 nv = *reinterpret_cast<const uint4*>(rv + 8 * (U % (D / 8)));
                    switch (kk & 3) {
                        case 0: vr[uu][0] = nv; break;
                        case 1: vr[uu][1] = nv; break;
                        case 2: vr[uu][2] = nv; break;
                        default: vr[uu][3] = nv; break;
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
    auto valid = [&](int k) -> bool { return (vmask >> k) & 1ull; };

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

    // ---- V^T into LDS ----------------------------------------------------------------
#pragma unroll
    for (int uu = 0; uu < NU; ++uu) {
        const int U = lane + 64 * uu;
        const int kg = U / (D / 8);
        const int dg = U % (D / 8);
        const int pos = vt_pos(4 * kg);
        const uint16_t* r0 = reinterpret_cast<const uint16_t*>(&vr[uu][0]);
        const uint16_t* r1 = reinterpret_cast<const uint16_t*>(&vr[uu][1]);
        const uint16_t* r2 = reinterpret_cast<const uint16_t*>(&vr[uu][2]);
        const uint16_t* r3 = reinterpret_cast<const uint16_t*>(&vr[uu][3]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint2 pk;
            pk.x = uint32_t(r0[e]) | (uint32_t(r1[e]) << 16);
            pk.y = uint32_t(r2[e]) | (uint32_t(r3[e]) << 16);
            *reinterpret_cast<uint2*>(&Vt[(8 * dg + e) * VST + pos]) = pk;
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
            const bool ok = valid(16 * mt + 4 * q16 + r);
            x[mt][r] = ok ? sacc[mt][r] * csc : -INFINITY;
            m = fmaxf(m, x[mt][r]);
        }
    }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    const float msafe = (m == -INFINITY) ? 0.0f : m;
    // p = p_hi + p_lo, both bf16: the P.V product keeps ~16 mantissa bits of p
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
    __syncthreads();                                  // V^T complete

    // ---- o^T = V^T p^T: rows = dims 16dt + 4q16 + r, column = head l16 ----------------
    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        oacc[dt] = f32x4{};
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const bf16x8 a =
                *reinterpret_cast<const bf16x8*>(&Vt[(16 * dt + l16) * VST + 32 * cc + 8 * q16]);
            oacc[dt] = mfma16(a, pf[cc], oacc[dt]);
            oacc[dt] = mfma16(a, pl[cc], oacc[dt]);
        }
    }
    if (l16 < G) {
        float* pb = part + ((long(bg) * nsplit + sp) * G + l16) * (D + 2);
        if (q16 == 0) {
            pb[0] = m;
            pb[1] = l;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) pb[2 + 16 * dt + 4 * q16 + r] = oacc[dt][r];
    }
}

// Merge of the split partials (fixed split order) and, for a decode step, the
// rest of the ingest.  One workgroup per (batch, KV head).  Every load that
// does not depend on another is issued first: the state words, k_t/v_t, the
// segment entries (for a possible weakest-entry search), every split's
// (max, sum) and the first CH splits' o values.
template <int D, int G, bool INGEST>
__global__ __launch_bounds__(256) void decode_finish_kernel(
    int Hq, int Hkv, int s, int w, int C, int S, int nsplit, const uint16_t* __restrict__ k_t,
    const uint16_t* __restrict__ v_t, lte_cnn cnn, CacheView c, const float* __restrict__ part,
    uint16_t* __restrict__ out_t) {
    constexpr int NO = (G * D + 255) / 256;                  // outputs per thread
    constexpr int CH = (64 / NO < 2) ? 2 : (64 / NO > 32 ? 32 : 64 / NO);   // splits per round
    constexpr int kSplitMax = (kMaxSink + kMaxCapacity + 32768 + KPB - 1) / KPB;
    constexpr int kFw = kSplitMax * G * 4;
    constexpr int kBuf = (INGEST && ScoreSmem<D>::kBytes > kFw) ? ScoreSmem<D>::kBytes : kFw;
    __shared__ __align__(16) unsigned char smem[kBuf];       // split weights; later the scorer
    __shared__ float invL[G];
    __shared__ float w2s[INGEST ? kHidden * 3 : 1];
    __shared__ float red_s[4];
    __shared__ int red_t[4], red_x[4];
    float* fw = reinterpret_cast<float*>(smem);              // [nsplit][G]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int bg = blockIdx.x;
    const int b = bg / Hkv;
    const int g = bg % Hkv;
    const long stride = long(G) * (D + 2);                   // floats per split
    const float* p0 = part + long(bg) * nsplit * stride;

    // ---- round 1 -----------------------------------------------------------------------
    int64_t t = 0, u = 0;
    int cnt = 0, X = -1, wk = -1;
    float rl = 0.0f;
    if (INGEST) {
        t = c.pos[bg];
        cnt = c.count[bg];
        X = c.nx_slot[bg];
        rl = c.nx_score[bg];
        u = c.next_unscored[bg];
        wk = c.weak[bg];
    }
    float ov[NO][CH];
#pragma unroll
    for (int j = 0; j < NO; ++j) {
        const int x = tid + 256 * j;
        const int hh = x / D;
        const int dd = x % D;
#pragma unroll
        for (int q = 0; q < CH; ++q)
            ov[j][q] = (x < G * D && q < nsplit) ? p0[q * stride + hh * (D + 2) + 2 + dd] : 0.0f;
    }
    constexpr int kMl = (kSplitMax + 63) / 64;
    float mv[(G + 3) / 4][kMl], lv[(G + 3) / 4][kMl];
#pragma unroll
    for (int j = 0; j < (G + 3) / 4; ++j) {
        const int hh = wave + 4 * j;
#pragma unroll
        for (int q = 0; q < kMl; ++q) {
            const int sp = lane + 64 * q;
            const bool ok = hh < G && sp < nsplit;
            mv[j][q] = ok ? p0[sp * stride + hh * (D + 2)] : -INFINITY;
            lv[j][q] = ok ? p0[sp * stride + hh * (D + 2) + 1] : 0.0f;
        }
    }

    // ---- per head: M = max of the split maxima, weights 2^(m_sp - M), 1/L ---------------
#pragma unroll
    for (int j = 0; j < (G + 3) / 4; ++j) {
        const int hh = wave + 4 * j;
        if (hh < G) {
            float M = -INFINITY;
#pragma unroll
            for (int q = 0; q < kMl; ++q) M = fmaxf(M, mv[j][q]);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
            float L = 0.0f;
#pragma unroll
            for (int q = 0; q < kMl; ++q) {
                const int sp = lane + 64 * q;
                const float f = (mv[j][q] == -INFINITY) ? 0.0f
                                                         : __builtin_amdgcn_exp2f(mv[j][q] - M);
                if (sp < nsplit) fw[sp * G + hh] = f;
                L += f * lv[j][q];
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
            if (lane == 0) invL[hh] = (L > 0.0f) ? 1.0f / L : 0.0f;
        }
    }
    __syncthreads();

    // ---- o = sum_sp w_sp o_sp / L in split order ------------------------------------------
#pragma unroll
    for (int j = 0; j < NO; ++j) {
        const int x = tid + 256 * j;
        if (x >= G * D) break;
        const int hh = x / D;
        const int dd = x % D;
        float o = 0.0f;
#pragma unroll
        for (int q = 0; q < CH; ++q)
            if (q < nsplit) o += fw[q * G + hh] * ov[j][q];
        for (int c0 = CH; c0 < nsplit; c0 += CH) {
            float nv[CH];
#pragma unroll
            for (int q = 0; q < CH; ++q)
                nv[q] = (c0 + q < nsplit) ? p0[(c0 + q) * stride + hh * (D + 2) + 2 + dd] : 0.0f;
#pragma unroll
            for (int q = 0; q < CH; ++q)
                if (c0 + q < nsplit) o += fw[(c0 + q) * G + hh] * nv[q];
        }
        reinterpret_cast<__bf16*>(out_t)[(long(b) * Hq + g * G + hh) * D + dd] =
            (__bf16)(o * invL[hh]);
    }
    if (INGEST) {
        const float ws = (wk >= 0) ? c.ret_score[long(bg) * C + wk] : 0.0f;
        __syncthreads();                              // split weights no longer read
        ingest_finish<D>(c, bg, g, s, w, C, S, t, cnt, X, rl, u, wk, ws, false, k_t, v_t, cnn,
                         smem, w2s, red_s, red_t, red_x);
    }
}

}  // namespace

hipError_t launch_score_evict(const Shape& sh, const lte_cnn& cnn, const uint16_t* k_t,
                              const uint16_t* v_t, const CacheView& cache, hipStream_t st) {
    dim3 grid(unsigned(sh.B * sh.Hkv));
    if (sh.D == 128) {
        hipLaunchKernelGGL(score_evict_kernel<128>, grid, dim3(256), 0, st, sh.s, sh.w, sh.C,
                           sh.S, sh.Hkv, k_t, v_t, cnn, cache);
    } else {
        hipLaunchKernelGGL(score_evict_kernel<64>, grid, dim3(256), 0, st, sh.s, sh.w, sh.C,
                           sh.S, sh.Hkv, k_t, v_t, cnn, cache);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const Shape& sh, bool ingest, const uint16_t* q_t, const uint16_t* k_t,
                         const uint16_t* v_t, const lte_cnn* cnn, const CacheView& cache,
                         float* part, uint16_t* out_t, hipStream_t st) {
    const int nsplit = decode_nsplit(sh);
    dim3 grid(unsigned(sh.B * sh.Hkv * nsplit));
    dim3 fgrid(unsigned(sh.B * sh.Hkv));
    lte_cnn cn{};
    if (cnn != nullptr) cn = *cnn;
#define LTE_FINISH(DD, GG, ING)                                                                  \
    case GG:                                                                                     \
        hipLaunchKernelGGL((decode_finish_kernel<DD, GG, ING>), fgrid, dim3(256), 0, st, sh.Hq, \
                           sh.Hkv, sh.s, sh.w, sh.C, sh.S, nsplit, k_t, v_t, cn, cache, part,    \
                           out_t);                                                               \
        break;
#define LTE_DECODE(DD, ING)                                                                      \
    do {                                                                                         \
        hipLaunchKernelGGL((decode_split_kernel<DD, ING>), grid, dim3(64), 0, st, sh.Hq, sh.Hkv, \
                           sh.G, sh.s, sh.w, sh.C, sh.S, nsplit, q_t, k_t, v_t, cache, part);    \
        hipError_t e_ = hipGetLastError();                                                       \
        if (e_ != hipSuccess) return e_;                                                         \
        switch (sh.G) {                                                                          \
            LTE_FINISH(DD, 1, ING)                                                               \
            LTE_FINISH(DD, 2, ING)                                                               \
            LTE_FINISH(DD, 4, ING)                                                               \
            LTE_FINISH(DD, 8, ING)                                                               \
            LTE_FINISH(DD, 16, ING)                                                              \
            default: return hipErrorInvalidValue;                                                \
        }                                                                                        \
    } while (0)
    if (sh.D == 128) {
        if (ingest) LTE_DECODE(128, true); else LTE_DECODE(128, false);
    } else {
        if (ingest) LTE_DECODE(64, true); else LTE_DECODE(64, false);
    }
#undef LTE_FINISH
#undef LTE_DECODE
    return hipGetLastError();
}

}  // namespace lte
