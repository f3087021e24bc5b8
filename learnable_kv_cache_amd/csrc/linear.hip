// Linear-attention layer of the hybrid: S_t = a_t S_{t-1} + v_t k_t^T,
// o_t = S_t q_t, one decay a_t per head and step.
//
// "Sparse Linear Attention: Viewing SWA from the Perspective of Linear
// Attention", section "Background: Linear attention": the state is decayed by
// A_t, written with v_t k_t^T and read with q_t.  A_t = a_t I here, given as
// log a_t; no scaling or feature map of q and k.
//
// Prefill, chunkwise (64 tokens per chunk, one workgroup per (batch, head),
// the state S^T in MFMA accumulators across chunks).  With G_t the running sum
// of log a over the chunk up to t (inclusive) and S0 the state before it:
//   o_t   = exp(G_t) S0 q_t + sum_{j <= t in chunk} exp(G_t - G_j) (q_t.k_j) v_j
//   S_end = exp(G_last) S0 + sum_j exp(G_last - G_j) v_j k_j^T
// Every exponent is <= 0.  Four MFMA products per chunk (v_mfma_f32_32x32x16_bf16):
//   P^T = K Q^T (masked and decayed, bf16, shared through LDS);
//   O  += P V (intra-chunk);  O' = Q S0^T (inter-chunk, S0 rounded to bf16);
//   S^T = exp(G_last) S^T + (w K)^T V  with w_j = exp(G_last - G_j).
// 2 D/32 waves, two per SIMD: wave w takes dims [32 dw, 32 dw + 32), dw = w/2,
// of the output rows [32 x, 32 x + 32), x = w%2, and the S^T tiles kt of its
// dims with kt in [x D/64, (x+1) D/64); the state is shared as bf16 through
// LDS for the inter-chunk product.  Two barriers per chunk: q and k are
// double-buffered, so the next chunk's are stored before the second barrier;
// its v and the state copy, which it reads only after its first barrier, after
// the second.  An MFMA
// accumulator holds its column in lane & 31 and rows (e/4)*8 + (lane/32)*4 +
// e%4; read as a 16-wide k operand, element i of lane-half h is then row
// 16c + (i<4 ? 4h + i : 8 + 4h + i-4) of step c, and every other operand is
// read in that same k order.
#include "lte_internal.h"

namespace lte {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;
constexpr float kLogAMin = -80.0f;     // a < 1.8e-35 acts as a reset

// 16-byte chunk swizzles.  Row-strided b128 reads of 16 consecutive rows (Q,
// K) and transposing b64 reads of 4 consecutive rows x 64 bytes (V, w K)
// each spread over all banks.
template <int D>
__device__ __forceinline__ int rswz(int r) {
    if constexpr (D == 128) return (((r & 1) * 10) | ((r & 2) << 1)) ^ ((r >> 2) & 3);
    else return ((r & 3) << 1) | ((r >> 2) & 1);
}
template <int D>
__device__ __forceinline__ int tswz(int r) {
    if constexpr (D == 128) return (r & 3) << 2;
    else return ((r >> 1) & 1) << 2;
}
// P tile [64 t][64 j]: 8 chunks per 128-byte row
__device__ __forceinline__ int pswz(int t) { return (t >> 1) & 7; }

template <int D>
__global__ __launch_bounds__(128 * (D / 32)) void linear_prefill_kernel(
    int T, int H, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ log_a,
    const float* __restrict__ state_in, float* __restrict__ state_out,
    uint16_t* __restrict__ out) {
    constexpr int DT = D / 32;              // 32-row tiles over D
    constexpr int NW = 2 * DT;              // waves
    constexpr int NT = 64 * NW;
    constexpr int CPR = D / 8;              // 16-byte chunks per row
    constexpr int KK = D / 16;              // k-steps over D
    constexpr int KTW = DT / 2;             // state tiles per wave
    // q and k tiles double-buffered: the next chunk's are stored before the chunk's last
    // barrier, while its own are still read
    __shared__ __align__(16) u32x4 Qs0[kChunk * CPR];
    __shared__ __align__(16) u32x4 Ks0[kChunk * CPR];
    __shared__ __align__(16) u32x4 Qs1[kChunk * CPR];
    __shared__ __align__(16) u32x4 Ks1[kChunk * CPR];
    __shared__ __align__(16) u32x4 Vs[kChunk * CPR];
    __shared__ __align__(16) u32x4 Ws[kChunk * CPR];     // w_j K[j]
    __shared__ __align__(16) u32x4 Ps[kChunk * 8];       // P[t][j] bf16
    __shared__ __align__(16) u32x4 Sb[KK * 2 * D];       // S^T as bf16 k operands
    __shared__ __align__(16) uint16_t Os[kChunk * D];     // the chunk's outputs, bf16 rows
    __shared__ __align__(16) float Gb[2][kChunk];         // G_t (two chunks)
    __shared__ __align__(16) float Eb[2][kChunk];         // exp(G_t)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int bh = blockIdx.x;
    const int b = bh / H;
    const int h = bh % H;
    const long rs = long(H) * D;                          // row stride of q, k, v, out

    const int dw = wave >> 1;                             // dim tile
    const int xw = wave & 1;                              // row tile; half of the state tiles
    // ---- state S^T: tile i holds S^T[(xw KTW + i)*32 + row(e)][32 dw + lane&31] ------
    f32x16 st[KTW];
    const float* sin = state_in ? state_in + long(bh) * D * D : nullptr;
    const int dcol = 32 * dw + (lane & 31);
#pragma unroll
    for (int i = 0; i < KTW; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int kr = (xw * KTW + i) * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
            st[i][e] = sin ? sin[long(dcol) * D + kr] : 0.0f;      // S[d][k]
        }
    }
    // its bf16 copy for the other waves: k-step kk, lane-half h of column d is
    // 16-byte piece (2 kk + h) * D + d
    auto share_state = [&]() {
#pragma unroll
        for (int i = 0; i < KTW; ++i) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int kk = 2 * (xw * KTW + i) + s2;
                bf16x8 sv;
#pragma unroll
                for (int u = 0; u < 8; ++u) sv[u] = (__bf16)st[i][s2 * 8 + u];
                Sb[(2 * kk + half) * D + dcol] = __builtin_bit_cast(u32x4, sv);
            }
        }
    };
    // per-lane pieces of the transposing reads (see the attention kernel): lane
    // (16-group G, index i) reads rows 4*(G>>1) + (i>>2) (+16c + 8r) at dims
    // (G&1)*16 + 4*(i&3) of a 32-wide tile
    uint32_t trd[DT];
    {
        const int grp = lane >> 4;
        const int i = lane & 15;
        const int key0 = 4 * (grp >> 1) + (i >> 2);
        const int c_lo = 2 * (grp & 1) + ((i & 3) >> 1);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            trd[dt] = uint32_t(key0 * CPR * 16 + ((4 * dt + c_lo) ^ tswz<D>(key0)) * 16 + 8 * (i & 1));
    }
    auto tr_operand = [&](const u32x4* tile, int dt, int c) {
        const char* base = reinterpret_cast<const char*>(tile);
        bf16x8 a;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const v4i16 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16*)(base + trd[dt] +
                                                           (c * 16 + 8 * r) * CPR * 16));
            const bf16x4 b4 = __builtin_bit_cast(bf16x4, t4);
            a[4 * r + 0] = b4[0];
            a[4 * r + 1] = b4[1];
            a[4 * r + 2] = b4[2];
            a[4 * r + 3] = b4[3];
        }
        return a;
    };

    // ---- chunk loads, one chunk ahead into registers: q, k (and log a) at a chunk's
    //      top, stored to LDS before its second barrier; v after its first barrier,
    //      stored after its second (rows zero past T; log a clamped, zero past T) -----
    constexpr int LPT = kChunk * CPR / NT;               // 16-byte pieces per thread
    u32x4 pq[LPT], pk[LPT], pv[LPT];
    float pg = 0.0f;
    auto fetch = [&](int c0) {
        const int nr = min(kChunk, T - c0);
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int x = tid + u * NT;
            const int r = x / CPR;
            const int c = x % CPR;
            pq[u] = pk[u] = u32x4{0u, 0u, 0u, 0u};
            if (r < nr) {
                const long src = (long(b) * T + c0 + r) * rs + long(h) * D + c * 8;
                pq[u] = *reinterpret_cast<const u32x4*>(q + src);
                pk[u] = *reinterpret_cast<const u32x4*>(k + src);
            }
        }
        if (wave == NW - 1) pg = (lane < nr) ? log_a[(long(b) * T + c0 + lane) * H + h] : 0.0f;
    };
    // running sums of the fetched chunk's log a (clamped), by the last wave, into
    // G buffer gbuf
    auto scan_g = [&](int gbuf) {
        if (wave == NW - 1) {
            // inclusive prefix sum over the wave by DPP moves: shifts by 1, 2, 4, 8 within
            // rows of 16 lanes, then each row's last lane into the rows after it; a lane
            // whose source is out of range adds the +0.0 passed as the old value
            float g = fmaxf(pg, kLogAMin);
            g += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(g), 0x111, 0xf, 0xf, false));
            g += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(g), 0x112, 0xf, 0xf, false));
            g += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(g), 0x114, 0xf, 0xf, false));
            g += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(g), 0x118, 0xf, 0xf, false));
            g += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(g), 0x142, 0xa, 0xf, false));
            g += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(g), 0x143, 0xc, 0xf, false));
            Gb[gbuf][lane] = g;
            Eb[gbuf][lane] = __expf(g);
        }
    };
    // the LDS offsets are recomputed on every call: hoisted out of the chunk loop they
    // were spilled, and their reloads serialised the stores
    auto stash_qk = [&](u32x4* Qd, u32x4* Kd) __attribute__((always_inline)) {
        int tx = tid;
        asm volatile("" : "+v"(tx));
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int x = tx + u * NT;
            const int r = x / CPR;
            const int c = x % CPR;
            Qd[r * CPR + (c ^ rswz<D>(r))] = pq[u];
            Kd[r * CPR + (c ^ rswz<D>(r))] = pk[u];
        }
    };
    auto stash_v = [&]() __attribute__((always_inline)) {
        int tx = tid;
        asm volatile("" : "+v"(tx));
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int x = tx + u * NT;
            const int r = x / CPR;
            const int c = x % CPR;
            Vs[r * CPR + (c ^ tswz<D>(r))] = pv[u];
        }
    };

    const int nchunk = (T + kChunk - 1) / kChunk;
    auto fetch_v = [&](int c0) {
        const int nr = min(kChunk, T - c0);
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int x = tid + u * NT;
            const int r = x / CPR;
            const int c = x % CPR;
            pv[u] = u32x4{0u, 0u, 0u, 0u};
            if (r < nr)
                pv[u] = *reinterpret_cast<const u32x4*>(v + (long(b) * T + c0 + r) * rs +
                                                        long(h) * D + c * 8);
        }
    };
    fetch(0);
    fetch_v(0);
    stash_qk(Qs0, Ks0);
    stash_v();
    scan_g(0);
    share_state();
    __syncthreads();
    // a chunk's outputs go through LDS and leave as whole rows after the chunk's last
    // barrier, ahead of the next chunk's loads
    constexpr int LPO = kChunk * CPR / NT;               // 16-byte output pieces per thread
    uint16_t opend[16];
    for (int ch = 0; ch < nchunk; ++ch) {
        const u32x4* Qs = (ch & 1) ? Qs1 : Qs0;
        const u32x4* Ks = (ch & 1) ? Ks1 : Ks0;
        u32x4* QN = (ch & 1) ? Qs0 : Qs1;
        u32x4* KN = (ch & 1) ? Ks0 : Ks1;
        const int t0 = ch * kChunk;
        const int nrow = min(kChunk, T - t0);
        if (ch + 1 < nchunk) fetch(t0 + kChunk);          // in flight during this chunk
        const float* Gs = Gb[ch & 1];
        const float* Es = Eb[ch & 1];
        // ---- w K: row j scaled by exp(G_last - G_j) ------------------------------------
        const float g_last = Gs[kChunk - 1];
        // (with 8 waves by waves 4-7, which take no q.k tile; with 4 by all)
        constexpr int WW0 = NW > 4 ? 4 : 0;
        for (int x = tid - WW0 * 64; x >= 0 && x < kChunk * CPR; x += NT - WW0 * 64) {
            const int r = x / CPR;
            const float wj = __expf(g_last - Gs[r]);
            const int pc = x % CPR;                       // physical chunk of Ks row r
            const int c = pc ^ rswz<D>(r);                // its logical chunk
            const bf16x8 kv = __builtin_bit_cast(bf16x8, Ks[r * CPR + pc]);
            bf16x8 wv;
#pragma unroll
            for (int u = 0; u < 8; ++u) wv[u] = (__bf16)(float(kv[u]) * wj);
            Ws[r * CPR + (c ^ tswz<D>(r))] = __builtin_bit_cast(u32x4, wv);
        }
        // ---- P^T = K Q^T for the tiles (jt, tt) of this wave; mask, decay, to LDS ----
        for (int tile = wave; tile < 4; tile += 4) {
            const int jt = tile & 1;
            const int tt = tile >> 1;
            f32x16 sacc = f32x16{};
            const int jr = jt * 32 + (lane & 31);
            const int tr = tt * 32 + (lane & 31);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, Ks[jr * CPR + ((2 * kk + half) ^ rswz<D>(jr))]);
                const bf16x8 bq = __builtin_bit_cast(
                    bf16x8, Qs[tr * CPR + ((2 * kk + half) ^ rswz<D>(tr))]);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, sacc, 0, 0, 0);
            }
            // operands two k-steps ahead of the MFMA that takes them
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
            for (int x = 0; x < KK - 2; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
            const float gt = Gs[tr];
            // G of this lane's keys: 4 runs of 4 consecutive rows
            float4 gj[4];
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                gj[e4] = *reinterpret_cast<const float4*>(&Gs[jt * 32 + e4 * 8 + half * 4]);
            bf16x8 pf[2];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = jt * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
                const float g4[4] = {gj[e >> 2].x, gj[e >> 2].y, gj[e >> 2].z, gj[e >> 2].w};
                const float p = (j <= tr) ? sacc[e] * __expf(gt - g4[e & 3]) : 0.0f;
                pf[e >> 3][e & 7] = (__bf16)p;
            }
            // P row tr, k-step c = 2jt + s, lane-half h: chunk 2c + h
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const int pc = (2 * (2 * jt + s2) + half) ^ pswz(tr);
                Ps[tr * 8 + pc] = __builtin_bit_cast(u32x4, pf[s2]);
            }
        }
        __syncthreads();

        if (ch + 1 < nchunk) fetch_v(t0 + kChunk);       // needed after the second barrier
        // ---- V operands of this wave's dims, k-steps c = 0..3 (P V and the update) ----
        bf16x8 vop[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) vop[c] = tr_operand(Vs, dw, c);
        // ---- O = P V + exp(G_t) Q S0^T for this wave's row tile -------------------------
        {
            const int tt = xw;
            const int tr = tt * 32 + (lane & 31);
            f32x16 oi = f32x16{}, ox = f32x16{};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bf16x8 pa = __builtin_bit_cast(bf16x8, Ps[tr * 8 + ((2 * c + half) ^ pswz(tr))]);
                oi = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vop[c], oi, 0, 0, 0);
            }
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                // q[tr][16kk + 4h .. +4] and q[tr][16kk + 8 + 4h .. +4]: halves of chunks
                const uint16_t* row = reinterpret_cast<const uint16_t*>(Qs + tr * CPR);
                const bf16x4 lo = *reinterpret_cast<const bf16x4*>(
                    row + ((2 * kk) ^ rswz<D>(tr)) * 8 + 4 * half);
                const bf16x4 hi = *reinterpret_cast<const bf16x4*>(
                    row + ((2 * kk + 1) ^ rswz<D>(tr)) * 8 + 4 * half);
                const bf16x8 qa = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                const bf16x8 sop = __builtin_bit_cast(bf16x8, Sb[(2 * kk + half) * D + dcol]);
                ox = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sop, ox, 0, 0, 0);
            }
            // operands (two q halves, one state piece) two k-steps ahead
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 2);
#pragma unroll
            for (int x = 0; x < KK - 2; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
                __builtin_amdgcn_sched_group_barrier(0x100, 3, 2);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 2);
            // element e: row t = tt*32 + (e/4)*8 + h*4 + e%4, dim 32*wave + lane&31
            float4 ev[4];                                 // exp(G_t) of this lane's rows
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                ev[e4] = *reinterpret_cast<const float4*>(&Es[tt * 32 + e4 * 8 + half * 4]);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float e4v[4] = {ev[e >> 2].x, ev[e >> 2].y, ev[e >> 2].z, ev[e >> 2].w};
                opend[e] = __builtin_bit_cast(uint16_t, (__bf16)(oi[e] + e4v[e & 3] * ox[e]));
            }
        }
        // ---- S^T = exp(G_last) S^T + (w K)^T V for this wave's state tiles ------------
        const float decay = __expf(g_last);
#pragma unroll
        for (int i = 0; i < KTW; ++i) {
            st[i] *= decay;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bf16x8 wa = tr_operand(Ws, xw * KTW + i, c);
                st[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, vop[c], st[i], 0, 0, 0);
            }
        }
        if (ch + 1 < nchunk) scan_g((ch + 1) & 1);       // the next chunk's G, other buffer
        // element e: row t = xw*32 + (e/4)*8 + h*4 + e%4, dim 32 dw + lane&31
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int t = xw * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
            Os[t * D + dcol] = opend[e];
        }
        if (ch + 1 < nchunk) stash_qk(QN, KN);           // the other q, k buffers
        __syncthreads();                                  // the chunk's tiles and Sb are free
        // the next chunk reads v and Sb only after its first barrier
        if (ch + 1 < nchunk) {
            stash_v();
            share_state();
        }
        {
            uint16_t* ob = out + (long(b) * T + t0) * rs + long(h) * D;
#pragma unroll
            for (int u = 0; u < LPO; ++u) {
                const int x = tid + u * NT;
                const int r = x / CPR;
                const int c = x % CPR;
                if (r < nrow)
                    *reinterpret_cast<u32x4*>(ob + long(r) * rs + c * 8) =
                        *reinterpret_cast<const u32x4*>(&Os[r * D + c * 8]);
            }
        }
    }
    float* so = state_out + long(bh) * D * D;
#pragma unroll
    for (int i = 0; i < KTW; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int kr = (xw * KTW + i) * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
            so[long(dcol) * D + kr] = st[i][e];
        }
}

// One step: S <- a S + v k^T, o = S q.  A workgroup of 256 threads takes 32
// rows of one (batch, head)'s S (D/32 workgroups per head, so a step spreads
// over enough waves to keep the state streaming); thread x owns 8 threads'
// share, D/8 consecutive elements, of one row.
template <int D>
__global__ __launch_bounds__(256) void linear_step_kernel(int H, const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const float* __restrict__ log_a,
                                                          float* __restrict__ state,
                                                          uint16_t* __restrict__ out) {
    constexpr int RW = 32;                                // rows per workgroup
    constexpr int TPR = 256 / RW;                         // threads per row
    constexpr int PER = D / TPR;                          // elements per thread
    const int bh = blockIdx.x / (D / RW);
    const int tid = threadIdx.x;
    const int d = (blockIdx.x % (D / RW)) * RW + tid / TPR;   // row of S (value dim)
    const int k0 = (tid % TPR) * PER;                     // first key dim
    const float a = __expf(fmaxf(log_a[bh], kLogAMin));
    const float vd = float(__builtin_bit_cast(__bf16, v[long(bh) * D + d]));
    float* srow = state + long(bh) * D * D + long(d) * D + k0;
    const uint16_t* kp = k + long(bh) * D + k0;
    const uint16_t* qp = q + long(bh) * D + k0;
    float4 s4[PER / 4];
#pragma unroll
    for (int x = 0; x < PER / 4; ++x) s4[x] = *reinterpret_cast<const float4*>(srow + 4 * x);
    float acc = 0.0f;
#pragma unroll
    for (int x = 0; x < PER / 4; ++x) {
        const bf16x4 k4 = *reinterpret_cast<const bf16x4*>(kp + 4 * x);
        const bf16x4 q4 = *reinterpret_cast<const bf16x4*>(qp + 4 * x);
        s4[x].x = fmaf(a, s4[x].x, vd * float(k4[0]));
        s4[x].y = fmaf(a, s4[x].y, vd * float(k4[1]));
        s4[x].z = fmaf(a, s4[x].z, vd * float(k4[2]));
        s4[x].w = fmaf(a, s4[x].w, vd * float(k4[3]));
        acc = fmaf(s4[x].x, float(q4[0]), acc);
        acc = fmaf(s4[x].y, float(q4[1]), acc);
        acc = fmaf(s4[x].z, float(q4[2]), acc);
        acc = fmaf(s4[x].w, float(q4[3]), acc);
        *reinterpret_cast<float4*>(srow + 4 * x) = s4[x];
    }
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (tid % TPR == 0) out[long(bh) * D + d] = __builtin_bit_cast(uint16_t, (__bf16)acc);
}

}  // namespace

hipError_t launch_linear_prefill(int B, int H, int D, int64_t T, const uint16_t* q,
                                 const uint16_t* k, const uint16_t* v, const float* log_a,
                                 const float* state_in, float* state_out, uint16_t* out,
                                 hipStream_t st) {
    dim3 grid(unsigned(B * H));
    if (D == 128)
        hipLaunchKernelGGL(linear_prefill_kernel<128>, grid, dim3(512), 0, st, int(T), H, q, k, v,
                           log_a, state_in, state_out, out);
    else
        hipLaunchKernelGGL(linear_prefill_kernel<64>, grid, dim3(256), 0, st, int(T), H, q, k, v,
                           log_a, state_in, state_out, out);
    return hipGetLastError();
}

hipError_t launch_linear_step(int B, int H, int D, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const float* log_a, float* state, uint16_t* out,
                              hipStream_t st) {
    dim3 grid(unsigned(B * H * (D / 32)));
    if (D == 128)
        hipLaunchKernelGGL(linear_step_kernel<128>, grid, dim3(256), 0, st, H, q, k, v, log_a,
                           state, out);
    else
        hipLaunchKernelGGL(linear_step_kernel<64>, grid, dim3(256), 0, st, H, q, k, v, log_a,
                           state, out);
    return hipGetLastError();
}

}  // namespace lte
