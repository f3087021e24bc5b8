// A-plus-column sparse causal attention for a whole prompt on gfx950.
//
// LTE paper (arXiv 2510.20787) summary page, Figure 2 caption (right panel):
// each head attends to the sink columns, the diagonal band of the sliding
// window ("A") and vertical stripes for the retained tokens ("column").
// Query row i sees V(i) = [0, min(s, i+1)) U [i-w+1, i] U R_i, with
// j in R_i <=> j <= i-w and rank[j] <= thr[i-w] (selection kernel).
//
// Tiling (one workgroup = 4 waves = 128 MFMA rows):
//   * GQA packing: the G = Hq/Hkv query heads of a group share their keys, so
//     a tile is P = 128/G consecutive positions x G heads of one KV head.
//     Its band of keys is [i0-w+1, i0+P-1] (P+w-1 keys for P rows).
//   * keys are processed in blocks of 64: first the gathered columns below the
//     band (sink + retained tokens alive at the tile's first row, via the
//     per-head rank/thr lists), then the band blocks.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K rows from LDS are the A
//     operand, each wave's 32 query rows stay in registers as the B operand.
//     A lane then owns one query row, so the row max/sum of the online
//     softmax is a 32-value local reduction plus one lane swap.
//   * O^T += V^T P^T: P^T comes straight from the S^T accumulator (converted
//     to bf16); V is stored transposed in LDS with the key order permuted to
//     match the accumulator's row order, so no data moves between lanes.
//   * fp32 softmax with exp2 and max subtraction; masked keys are -inf.
#include "lte_internal.h"

namespace lte {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, int G>
__global__ __launch_bounds__(256) void attend_prefill_kernel(
    int T, int Hq, int Hkv, int s, int w, int ntile, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ thr,
    uint16_t* __restrict__ out) {
    constexpr int P = 128 / G;          // positions per tile
    constexpr int KK = D / 16;          // MFMA k-steps of q.k
    constexpr int DT = D / 32;          // 32-wide output tiles of o
    constexpr int KST = D + 8;          // LDS row stride of K (bf16)
    constexpr int VST = 64 + 8;         // LDS row stride of V^T (bf16)
    constexpr int kMaxList = kMaxSink + kMaxCapacity;
    constexpr int DV = D / 8;           // 16-byte chunks per key row

    __shared__ __align__(16) __bf16 Ks[64 * KST];
    __shared__ __align__(16) __bf16 Vt[D * VST];
    __shared__ __align__(16) uint32_t lst[kMaxList];   // (rank << 16) | token index
    __shared__ __align__(16) int32_t brank[64];
    __shared__ int wsum[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;          // which half of the MFMA k-dimension a lane holds

    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so map
    // each XCD's share to a contiguous run of tiles (neighbouring tiles of a
    // head share most of their band keys in that XCD's L2).
    const int nblk = gridDim.x;
    int lin = blockIdx.x;
    if ((nblk & 7) == 0) lin = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    const int bg = lin / ntile;
    const int tile = lin % ntile;
    const int b = bg / Hkv;
    const int g = bg % Hkv;
    const int i0 = tile * P;
    const int i_last = min(i0 + P, T) - 1;
    const int band_lo = max(0, i0 - w + 1);
    const int band_hi = i_last;
    const int32_t* rk = rank + long(bg) * T;
    const int32_t* th = thr + long(bg) * T;
    const long kv_row = long(Hkv) * D;                           // elements between tokens
    const uint16_t* kbase = k + (long(b) * T * Hkv + g) * D;
    const uint16_t* vbase = v + (long(b) * T * Hkv + g) * D;

    // ---- gathered columns below the band: sink, then retained tokens ----------
    int len = 0;
    int ns = 0;                                   // leading sink entries: always visible
    if (band_lo > 0) {
        const int thr0 = th[i0 - w];
        ns = min(s, band_lo);
        for (int j = tid; j < ns; j += 256) lst[j] = uint32_t(j);
        len = ns;
        // candidates j in [s, band_lo) alive at the first row, in index order
        for (int base = s; base < band_lo; base += 256 * 16) {
            uint32_t ent[16];
            int cnt = 0;
            const int j0 = base + tid * 16;
            int rr[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) rr[u] = (j0 + u < band_lo) ? rk[j0 + u] : kNotCand;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (rr[u] <= thr0) ent[cnt++] = (uint32_t(rr[u]) << 16) | uint32_t(j0 + u);
            }
            // block exclusive scan of cnt
            int incl = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                int y = __shfl_up(incl, d, 64);
                if (lane >= d) incl += y;
            }
            if (lane == 63) wsum[wave] = incl;
            __syncthreads();
            int woff = 0, tot = 0;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                woff += (x < wave) ? wsum[x] : 0;
                tot += wsum[x];
            }
            const int off = len + woff + incl - cnt;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (u < cnt) lst[off + u] = ent[u];
            }
            len += tot;
            __syncthreads();
        }
    }
    __syncthreads();

    // ---- this lane's query row --------------------------------------------------
    const int rtile = wave * 32 + (lane & 31);
    const int p_row = rtile / G;
    const int hh = rtile % G;
    const int i_row = i0 + p_row;
    const bool row_ok = i_row <= i_last;
    const int irow = row_ok ? i_row : i_last;
    const int h = g * G + hh;
    bf16x8 qf[KK];
    {
        const uint16_t* qrow = q + ((long(b) * T + irow) * Hq + h) * D;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + kk * 16 + half * 8);
    }
    const int thr_row = (irow - w >= 0) ? th[irow - w] : -2;
    const float csc = kLog2e * rsqrtf(float(D));

    float m_run = -INFINITY;
    float l_run = 0.0f;
    f32x16 acc_o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x16{};

    const int nlist = (len + 63) / 64;
    const int nband = (band_hi - band_lo + 1 + 63) / 64;

    for (int blk = 0; blk < nlist + nband; ++blk) {
        const bool is_list = blk < nlist;
        const int jb0 = band_lo + (blk - nlist) * 64;     // first key of a band block

        // ---- stage K (row-major) and V^T (permuted key order) into LDS ---------
#pragma unroll
        for (int x = 0; x < (64 * DV) / 256; ++x) {
            const int c16 = tid + 256 * x;
            const int t = c16 / DV;
            const int col = c16 % DV;
            int j;
            if (is_list) {
                const int e = blk * 64 + t;
                j = (e < len) ? int(lst[e] & 0xffffu) : 0;
            } else {
                j = min(jb0 + t, band_hi);
            }
            *reinterpret_cast<uint4*>(&Ks[t * KST + col * 8]) =
                *reinterpret_cast<const uint4*>(kbase + long(j) * kv_row + col * 8);
        }
        if (tid < 16 * DV) {
            const int kg = tid / DV;          // 4 consecutive keys 4kg .. 4kg+3
            const int dg = tid % DV;          // 8 consecutive dims 8dg .. 8dg+7
            uint4 rows[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = 4 * kg + u;
                int j;
                if (is_list) {
                    const int e = blk * 64 + t;
                    j = (e < len) ? int(lst[e] & 0xffffu) : 0;
                } else {
                    j = min(jb0 + t, band_hi);
                }
                rows[u] = *reinterpret_cast<const uint4*>(vbase + long(j) * kv_row + dg * 8);
            }
            // keys 4q..4q+3 of each 16-key chunk go to positions (q&1)*8 + (q>>1)*4,
            // so lane half 0 reads keys {0-3, 8-11} and half 1 keys {4-7, 12-15}
            const int qq = kg & 3;
            const int pos = (kg >> 2) * 16 + (qq & 1) * 8 + (qq >> 1) * 4;
            const uint16_t* r0 = reinterpret_cast<const uint16_t*>(&rows[0]);
            const uint16_t* r1 = reinterpret_cast<const uint16_t*>(&rows[1]);
            const uint16_t* r2 = reinterpret_cast<const uint16_t*>(&rows[2]);
            const uint16_t* r3 = reinterpret_cast<const uint16_t*>(&rows[3]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint2 pk;
                pk.x = uint32_t(r0[e]) | (uint32_t(r1[e]) << 16);
                pk.y = uint32_t(r2[e]) | (uint32_t(r3[e]) << 16);
                *reinterpret_cast<uint2*>(&Vt[(dg * 8 + e) * VST + pos]) = pk;
            }
        }
        if (!is_list && tid < 64) {
            const int j = jb0 + tid;
            brank[tid] = (j <= band_hi) ? rk[j] : kNotCand;
        }
        __syncthreads();

        // ---- S^T = K Q^T for 64 keys x this wave's 32 rows -----------------------
        f32x16 sacc[2];
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    &Ks[(ks * 32 + (lane & 31)) * KST + kk * 16 + half * 8]);
                sacc[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[ks], 0, 0, 0);
            }
        }

        // ---- mask and scale: element e of subtile ks is key slot
        //      ks*32 + (e/4)*8 + half*4 + e%4 of this block ---------------------------
        float x[2][16];
        if (is_list) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int t0 = ks * 32 + e4 * 8 + half * 4;
                    const uint4 ent = *reinterpret_cast<const uint4*>(&lst[blk * 64 + t0]);
                    const uint32_t ev[4] = {ent.x, ent.y, ent.z, ent.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int eidx = blk * 64 + t0 + u;
                        const bool vis = (eidx < ns) || (eidx < len && int(ev[u] >> 16) <= thr_row);
                        x[ks][e4 * 4 + u] = vis ? sacc[ks][e4 * 4 + u] * csc : -INFINITY;
                    }
                }
            }
        } else {
            const bool full = (jb0 >= i_last - w + 1) && (jb0 + 63 <= i0);
            if (full) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int e = 0; e < 16; ++e) x[ks][e] = sacc[ks][e] * csc;
            } else {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        const int t0 = ks * 32 + e4 * 8 + half * 4;
                        const int4 br = *reinterpret_cast<const int4*>(&brank[t0]);
                        const int bv[4] = {br.x, br.y, br.z, br.w};
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int j = jb0 + t0 + u;
                            const bool vis =
                                (j <= irow) &&
                                (j >= irow - w + 1 || j < s || (j <= irow - w && bv[u] <= thr_row));
                            x[ks][e4 * 4 + u] = vis ? sacc[ks][e4 * 4 + u] * csc : -INFINITY;
                        }
                    }
                }
            }
        }

        // ---- online softmax (row = this lane's query; keys split with lane^32) -----
        float mloc = x[0][0];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, x[ks][e]);
        const float mrow = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const float m_new = fmaxf(m_run, mrow);
        const float msafe = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - msafe);
        float lsum = 0.0f;
        bf16x8 pf[4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = fast_exp2(x[ks][e] - msafe);
                lsum += p;
                pf[ks * 2 + (e >> 3)][e & 7] = (__bf16)p;
            }
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc_o[dt] *= alpha;

        // ---- O^T += V^T P^T ------------------------------------------------------
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    &Vt[(dt * 32 + (lane & 31)) * VST + cc * 16 + half * 8]);
                acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[cc], acc_o[dt], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- normalise and store: element e of d-tile dt is dim dt*32 + (e/4)*8 + half*4 + e%4
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (row_ok) {
        const float inv = 1.0f / l_tot;
        uint16_t* orow = out + ((long(b) * T + i_row) * Hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                bf16x4 o4;
#pragma unroll
                for (int u = 0; u < 4; ++u) o4[u] = (__bf16)(acc_o[dt][e4 * 4 + u] * inv);
                *reinterpret_cast<bf16x4*>(orow + dt * 32 + e4 * 8 + half * 4) = o4;
            }
        }
    }
}

template <int D>
hipError_t launch_attend_d(const Shape& sh, int64_t T, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const int32_t* rank, const int32_t* thr,
                           uint16_t* out, hipStream_t st) {
    const int G = sh.G;
    const int P = 128 / G;
    const int ntile = int((T + P - 1) / P);
    dim3 grid(unsigned(long(sh.B) * sh.Hkv * ntile));
#define LTE_ATTEND_CASE(GG)                                                                   \
    case GG:                                                                                  \
        hipLaunchKernelGGL((attend_prefill_kernel<D, GG>), grid, dim3(256), 0, st, int(T),    \
                           sh.Hq, sh.Hkv, sh.s, sh.w, ntile, q, k, v, rank, thr, out);        \
        break;
    switch (G) {
        LTE_ATTEND_CASE(1)
        LTE_ATTEND_CASE(2)
        LTE_ATTEND_CASE(4)
        LTE_ATTEND_CASE(8)
        LTE_ATTEND_CASE(16)
        default:
            return hipErrorInvalidValue;
    }
#undef LTE_ATTEND_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attend_prefill(const Shape& sh, int64_t T, const uint16_t* q,
                                 const uint16_t* k, const uint16_t* v, const int32_t* rank,
                                 const int32_t* thr, uint16_t* out, hipStream_t st) {
    if (sh.D == 128) return launch_attend_d<128>(sh, T, q, k, v, rank, thr, out, st);
    return launch_attend_d<64>(sh, T, q, k, v, rank, thr, out, st);
}

}  // namespace lte
