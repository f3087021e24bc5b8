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
// Kernels per step:
//   score_evict  one workgroup per (batch, KV head): the token t-w leaving
//                ring slot t mod w joins the capped segment if its score is
//                > 0.5, displacing the weakest entry (lowest score, then
//                highest index) when the segment is full and the newcomer
//                ranks above it; k_t/v_t are written into the slot; when
//                t = u + w - 3 for the oldest unscored token u, tokens
//                u .. t-2 are scored from the ring (their left neighbour u-2
//                is about to leave).
//   decode_attend split-K over the S = s + C + w cache slots, 128 slots per
//                workgroup; all G query heads of a KV head share each K/V
//                read; per-split (max, sum, unnormalised o) partials.
//   combine      fixed-order merge of the partials (deterministic).
#include "score_core.h"

namespace lte {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxG = 16;

template <int D>
__global__ __launch_bounds__(256) void score_evict_kernel(
    int Hkv, int s, int w, int C, int S, const uint16_t* __restrict__ k_t,
    const uint16_t* __restrict__ v_t, const float* __restrict__ w1, const float* __restrict__ b1,
    const float* __restrict__ w2, const float* __restrict__ b2, CacheView c) {
    __shared__ __align__(16) unsigned char buf[ScoreSmem<D>::kBytes];
    __shared__ float w2s[kHidden * 3];
    __shared__ float red_s[4];
    __shared__ int red_tok[4];
    __shared__ int red_slot[4];
    constexpr int KK = ScoreSmem<D>::KK;
    constexpr int NW = ScoreSmem<D>::NW;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int bg = blockIdx.x;
    const int g = bg % Hkv;
    const int64_t t = c.pos[bg];
    const int64_t u = c.next_unscored[bg];
    const int slot = int(t % w);
    const int ring0 = s + C;
    const long ring_row = (long(bg) * S + ring0 + slot) * D;

    // ---- 1. eviction decision for the token leaving the window -------------------
    const int64_t jl = t - w;
    int target = -1;
    float rj = 0.0f;
    int cnt = 0;
    if (jl >= s) {
        rj = c.ring_score[long(bg) * w + slot];
        if (rj != rj) {
            if (tid == 0) c.flags[bg] |= 1;                 // left the window unscored
        } else if (rj > 0.5f && C > 0) {
            cnt = c.count[bg];
            if (cnt < C) {
                target = cnt;
            } else {
                // weakest entry: lowest score, then highest token index
                float bs = INFINITY;
                int bt = -1, bx = -1;
                for (int x = tid; x < C; x += 256) {
                    const float sc = c.ret_score[long(bg) * C + x];
                    const int tk = c.ret_idx[long(bg) * C + x];
                    if (sc < bs || (sc == bs && tk > bt)) { bs = sc; bt = tk; bx = x; }
                }
#pragma unroll
                for (int d = 32; d >= 1; d >>= 1) {
                    const float os = __shfl_xor(bs, d, 64);
                    const int ot = __shfl_xor(bt, d, 64);
                    const int ox = __shfl_xor(bx, d, 64);
                    if (os < bs || (os == bs && ot > bt)) { bs = os; bt = ot; bx = ox; }
                }
                if (lane == 0) { red_s[wave] = bs; red_tok[wave] = bt; red_slot[wave] = bx; }
                __syncthreads();
                bs = red_s[0]; bt = red_tok[0]; bx = red_slot[0];
#pragma unroll
                for (int q = 1; q < 4; ++q) {
                    if (red_s[q] < bs || (red_s[q] == bs && red_tok[q] > bt)) {
                        bs = red_s[q]; bt = red_tok[q]; bx = red_slot[q];
                    }
                }
                // the newcomer has the highest index, so it must score strictly higher
                if (rj > bs) target = bx;
            }
        }
    }
    if (target >= 0) {
        const long dst = (long(bg) * S + s + target) * D;
        for (int ch = tid; ch < D / 8; ch += 256) {
            *reinterpret_cast<uint4*>(c.k + dst + ch * 8) =
                *reinterpret_cast<const uint4*>(c.k + ring_row + ch * 8);
            *reinterpret_cast<uint4*>(c.v + dst + ch * 8) =
                *reinterpret_cast<const uint4*>(c.v + ring_row + ch * 8);
        }
        if (tid == 0) {
            c.ret_idx[long(bg) * C + target] = int(jl);
            c.ret_score[long(bg) * C + target] = rj;
            if (target == cnt && cnt < C) c.count[bg] = cnt + 1;
        }
    }
    __syncthreads();                                        // ring slot read before overwrite

    // ---- 2. append token t -----------------------------------------------------
    for (int ch = tid; ch < D / 8; ch += 256) {
        const uint4 kv = *reinterpret_cast<const uint4*>(k_t + long(bg) * D + ch * 8);
        const uint4 vv = *reinterpret_cast<const uint4*>(v_t + long(bg) * D + ch * 8);
        *reinterpret_cast<uint4*>(c.k + ring_row + ch * 8) = kv;
        *reinterpret_cast<uint4*>(c.v + ring_row + ch * 8) = vv;
        if (t < s) {
            const long srow = (long(bg) * S + t) * D;
            *reinterpret_cast<uint4*>(c.k + srow + ch * 8) = kv;
            *reinterpret_cast<uint4*>(c.v + srow + ch * 8) = vv;
        }
    }
    if (tid == 0) c.ring_score[long(bg) * w + slot] = __builtin_nanf("");

    // ---- 3. deferred batched scoring ----------------------------------------------
    if (t == u + w - 3) {
        __threadfence_block();
        __syncthreads();
        for (int x = tid; x < kHidden * 3; x += 256) w2s[x] = w2[g * kHidden * 3 + x];
        const uint16_t* kring = c.k + (long(bg) * S + ring0) * D;
        const uint16_t* vring = c.v + (long(bg) * S + ring0) * D;
        float* rs = c.ring_score + long(bg) * w;
        const int tt = int(t);
        for (int t0 = int(u); t0 <= tt - 2; t0 += kScoreTile) {
            // stage this head's W1 as packed bf16 MFMA operands
            bf16x8* wl = reinterpret_cast<bf16x8*>(buf);
            for (int x = tid; x < NW; x += 256) {
                int tap, kk, ln;
                w1p_coords(x, KK, tap, kk, ln);
                const int o = ln % 32;
                const int c0 = kk * 16 + (ln / 32) * 8;
                const float* src = w1 + ((long(g) * kHidden + o) * (2 * D) + c0) * 3 + tap;
                bf16x8 e8;
#pragma unroll
                for (int e = 0; e < 8; ++e) e8[e] = (__bf16)src[e * 3];
                wl[x] = e8;
            }
            score_chunk<D>(
                buf, w2s, b1 + g * kHidden, b2[g], t0, int(u), tt - 2,
                [&](int x, const uint16_t*& kp, const uint16_t*& vp) {
                    if (x < 0 || x > tt) return false;
                    kp = kring + long(x % w) * D;
                    vp = vring + long(x % w) * D;
                    return true;
                },
                [&](int x) { return x < 0; },
                [&](int tok, float r) { rs[tok % w] = r; });
        }
        if (tid == 0) c.next_unscored[bg] = t - 1;
    }
    if (tid == 0) c.pos[bg] = t + 1;
}

// Split-K attention of q_t over the cache.  Workgroup = (split, batch, KV head).
template <int D>
__global__ __launch_bounds__(256) void decode_attend_kernel(
    int Hq, int Hkv, int G, int s, int w, int C, int S, int nsplit,
    const uint16_t* __restrict__ q_t, CacheView c, float* __restrict__ part) {
    __shared__ float qs[kMaxG][D];
    __shared__ float sl[kMaxG][kDecodeSplitKeys];
    __shared__ float red[4][kMaxG][D];
    __shared__ int valid[kDecodeSplitKeys];
    __shared__ float mh[kMaxG], lh[kMaxG];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sp = blockIdx.x % nsplit;
    const int bg = blockIdx.x / nsplit;
    const int b = bg / Hkv;
    const int g = bg % Hkv;
    const int64_t t = c.pos[bg] - 1;
    const int cnt = c.count[bg];
    const int slot0 = sp * kDecodeSplitKeys;
    const float csc = kLog2e * rsqrtf(float(D));
    const uint16_t* kc = c.k + long(bg) * S * D;
    const uint16_t* vc = c.v + long(bg) * S * D;

    for (int x = tid; x < G * D; x += 256) {
        const int hh = x / D;
        const int d = x % D;
        const uint16_t qb = q_t[(long(b) * Hq + g * G + hh) * D + d];
        qs[hh][d] = __uint_as_float(uint32_t(qb) << 16);
    }
    if (tid < kDecodeSplitKeys) {
        const int slot = slot0 + tid;
        bool ok = false;
        if (slot < S && t >= 0) {
            if (slot < s) {
                ok = slot <= t;
            } else if (slot < s + C) {
                ok = (slot - s) < cnt;
            } else {
                const int r = slot - s - C;
                const int64_t x = t - (((t - r) % w) + w) % w;   // newest token in ring slot r
                ok = x >= 0 && x >= s;
            }
        }
        valid[tid] = ok ? 1 : 0;
    }
    __syncthreads();

    // ---- logits: 16 lanes per key, 4 keys per wave step -----------------------------
    constexpr int DL = D / 16;                 // dims per lane
    {
        const int kl = lane >> 4;
        const int dl = lane & 15;
        for (int it = 0; it < 8; ++it) {
            const int key = wave * 32 + it * 4 + kl;
            float acc[kMaxG];
#pragma unroll
            for (int hh = 0; hh < kMaxG; ++hh) acc[hh] = 0.0f;
            const bool ok = valid[key] != 0;
            if (ok) {
                const uint16_t* kr = kc + long(slot0 + key) * D + dl * DL;
                float kf[DL];
                if constexpr (DL == 8) {
                    const uint4 raw = *reinterpret_cast<const uint4*>(kr);
                    const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kf[2 * e] = __uint_as_float(r4[e] << 16);
                        kf[2 * e + 1] = __uint_as_float(r4[e] & 0xffff0000u);
                    }
                } else {
                    const uint2 raw = *reinterpret_cast<const uint2*>(kr);
                    const uint32_t r2[2] = {raw.x, raw.y};
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        kf[2 * e] = __uint_as_float(r2[e] << 16);
                        kf[2 * e + 1] = __uint_as_float(r2[e] & 0xffff0000u);
                    }
                }
#pragma unroll
                for (int hh = 0; hh < kMaxG; ++hh) {
                    if (hh < G) {
                        float a = 0.0f;
#pragma unroll
                        for (int e = 0; e < DL; ++e) a += kf[e] * qs[hh][dl * DL + e];
                        acc[hh] = a;
                    }
                }
            }
#pragma unroll
            for (int hh = 0; hh < kMaxG; ++hh) {
                if (hh < G) {
                    float a = acc[hh];
                    a += __shfl_xor(a, 8, 64);
                    a += __shfl_xor(a, 4, 64);
                    a += __shfl_xor(a, 2, 64);
                    a += __shfl_xor(a, 1, 64);
                    if (dl == hh) sl[hh][key] = ok ? a * csc : -INFINITY;
                }
            }
        }
    }
    __syncthreads();

    // ---- softmax statistics per head (one wave per head) ----------------------------
    for (int hh = wave; hh < G; hh += 4) {
        const float x0 = sl[hh][lane];
        const float x1 = sl[hh][lane + 64];
        float m = fmaxf(x0, x1);
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
        const float msafe = (m == -INFINITY) ? 0.0f : m;
        const float p0 = __builtin_amdgcn_exp2f(x0 - msafe);
        const float p1 = __builtin_amdgcn_exp2f(x1 - msafe);
        float l = p0 + p1;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) l += __shfl_xor(l, d, 64);
        sl[hh][lane] = p0;
        sl[hh][lane + 64] = p1;
        if (lane == 0) { mh[hh] = m; lh[hh] = l; }
    }
    __syncthreads();

    // ---- P V: each lane owns 2 dims; D/2 lanes per key row ------------------------------
    {
        constexpr int LPR = D / 2;                 // lanes per key row
        constexpr int KPI = 64 / LPR;              // keys per wave step
        const int kl = lane / LPR;
        const int d0 = (lane % LPR) * 2;
        float acc0[kMaxG], acc1[kMaxG];
#pragma unroll
        for (int hh = 0; hh < kMaxG; ++hh) { acc0[hh] = 0.0f; acc1[hh] = 0.0f; }
        for (int it = 0; it < 32 / KPI; ++it) {
            const int key = wave * 32 + it * KPI + kl;
            if (valid[key]) {
                const uint32_t raw = *reinterpret_cast<const uint32_t*>(
                    vc + long(slot0 + key) * D + d0);
                const float v0 = __uint_as_float(raw << 16);
                const float v1 = __uint_as_float(raw & 0xffff0000u);
#pragma unroll
                for (int hh = 0; hh < kMaxG; ++hh) {
                    if (hh < G) {
                        const float p = sl[hh][key];
                        acc0[hh] += p * v0;
                        acc1[hh] += p * v1;
                    }
                }
            }
        }
        // fold the KPI key lanes of a wave, then the 4 waves through LDS
#pragma unroll
        for (int hh = 0; hh < kMaxG; ++hh) {
            if (hh < G) {
                float a0 = acc0[hh], a1 = acc1[hh];
                for (int d = LPR; d < 64; d <<= 1) {
                    a0 += __shfl_xor(a0, d, 64);
                    a1 += __shfl_xor(a1, d, 64);
                }
                if (lane < LPR) { red[wave][hh][d0] = a0; red[wave][hh][d0 + 1] = a1; }
            }
        }
    }
    __syncthreads();
    float* pbase = part + (long(bg) * nsplit + sp) * G * (D + 2);
    for (int x = tid; x < G * D; x += 256) {
        const int hh = x / D;
        const int d = x % D;
        pbase[hh * (D + 2) + 2 + d] = red[0][hh][d] + red[1][hh][d] + red[2][hh][d] + red[3][hh][d];
    }
    if (tid < G) {
        pbase[tid * (D + 2) + 0] = mh[tid];
        pbase[tid * (D + 2) + 1] = lh[tid];
    }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(int Hq, int Hkv, int G, int nsplit,
                                                           const float* __restrict__ part,
                                                           uint16_t* __restrict__ out_t) {
    const int bh = blockIdx.x;                 // (b, g, hh)
    const int hh = bh % G;
    const int bg = bh / G;
    const int b = bg / Hkv;
    const int g = bg % Hkv;
    const int d = threadIdx.x;
    const float* p = part + long(bg) * nsplit * G * (D + 2) + hh * (D + 2);
    const long stride = long(G) * (D + 2);
    float M = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, p[sp * stride]);
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
        for (int sp = 0; sp < nsplit; ++sp) {
            const float m = p[sp * stride];
            if (m == -INFINITY) continue;
            const float f = __builtin_amdgcn_exp2f(m - M);
            L += p[sp * stride + 1] * f;
            O += p[sp * stride + 2 + d] * f;
        }
    }
    const float o = (L > 0.0f) ? O / L : 0.0f;
    reinterpret_cast<__bf16*>(out_t)[(long(b) * Hq + g * G + hh) * D + d] = (__bf16)o;
}

}  // namespace

hipError_t launch_score_evict(const Shape& sh, const lte_cnn& cnn, const uint16_t* k_t,
                              const uint16_t* v_t, const CacheView& cache, hipStream_t st) {
    dim3 grid(unsigned(sh.B * sh.Hkv));
    if (sh.D == 128) {
        hipLaunchKernelGGL(score_evict_kernel<128>, grid, dim3(256), 0, st, sh.Hkv, sh.s, sh.w,
                           sh.C, sh.S, k_t, v_t, cnn.w1, cnn.b1, cnn.w2, cnn.b2, cache);
    } else {
        hipLaunchKernelGGL(score_evict_kernel<64>, grid, dim3(256), 0, st, sh.Hkv, sh.s, sh.w,
                           sh.C, sh.S, k_t, v_t, cnn.w1, cnn.b1, cnn.w2, cnn.b2, cache);
    }
    return hipGetLastError();
}

hipError_t launch_decode_attend(const Shape& sh, const uint16_t* q_t, const CacheView& cache,
                                float* part, uint16_t* out_t, hipStream_t st) {
    const int nsplit = decode_nsplit(sh);
    dim3 grid(unsigned(sh.B * sh.Hkv * nsplit));
    dim3 cgrid(unsigned(sh.B * sh.Hq));
    if (sh.D == 128) {
        hipLaunchKernelGGL(decode_attend_kernel<128>, grid, dim3(256), 0, st, sh.Hq, sh.Hkv, sh.G,
                           sh.s, sh.w, sh.C, sh.S, nsplit, q_t, cache, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(decode_combine_kernel<128>, cgrid, dim3(128), 0, st, sh.Hq, sh.Hkv,
                           sh.G, nsplit, part, out_t);
    } else {
        hipLaunchKernelGGL(decode_attend_kernel<64>, grid, dim3(256), 0, st, sh.Hq, sh.Hkv, sh.G,
                           sh.s, sh.w, sh.C, sh.S, nsplit, q_t, cache, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(decode_combine_kernel<64>, cgrid, dim3(64), 0, st, sh.Hq, sh.Hkv,
                           sh.G, nsplit, part, out_t);
    }
    return hipGetLastError();
}

}  // namespace lte
