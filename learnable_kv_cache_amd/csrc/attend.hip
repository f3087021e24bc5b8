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
//     to bf16).  V stays row-major in LDS; its MFMA operand (8 keys of one
//     dim per lane) is read with ds_read_b64_tr_b16, whose 16-lane transpose
//     turns four 4-dim row pieces into four keys of one dim per lane.
//   * K and V tiles sit in LDS as 16-byte chunks XOR-swizzled by row, so the
//     row-strided MFMA operand reads hit distinct banks.
//   * the next block's K/V rows are fetched into registers while the current
//     block computes, then written to LDS between two barriers.
//   * fp32 online softmax on raw logits, the 1/sqrt(D) scale and log2(e)
//     folded into one FMA before exp2; masked keys are -inf; the running
//     output is rescaled only when some row's maximum moved.
#include "lte_internal.h"

namespace lte {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS chunk swizzle of tile row r (a key): bits (r&3)<<1 | (r>>2)&1, a
// permutation of 0..7 over any 8 consecutive rows starting at a multiple of 8.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

template <int D, int G>
__global__ __launch_bounds__(256, 2) void attend_prefill_kernel(
    int T, int Hq, int Hkv, int s, int w, int ntile, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ thr,
    uint16_t* __restrict__ out) {
    constexpr int P = 128 / G;          // positions per tile
    constexpr int KK = D / 16;          // MFMA k-steps of q.k
    constexpr int DT = D / 32;          // 32-wide output tiles of o
    constexpr int CPR = D / 8;          // 16-byte chunks per key row
    constexpr int NCH = 64 * CPR / 256; // chunks of one 64-key tile per thread
    constexpr int kMaxList = kMaxSink + kMaxCapacity;

    __shared__ __align__(16) u32x4 Ks[64 * CPR];          // swizzled row-major K tile
    __shared__ __align__(16) u32x4 Vs[64 * CPR];          // swizzled row-major V tile
    // (field << 16) | token index; field = rank + 1 of a retained token, 0 for
    // a sink token, 0xffff for padding
    __shared__ __align__(16) uint32_t lst[kMaxList];
    __shared__ __align__(16) int32_t brank[128];
    __shared__ int wsum[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;          // which half of the MFMA k-dimension a lane holds

    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so map
    // each XCD's share to a contiguous run of tiles (neighbouring tiles of a
    // head share most of their band keys in that XCD's L2).
    const int ngrid = gridDim.x;
    int lin = blockIdx.x;
    if ((ngrid & 7) == 0) lin = (blockIdx.x & 7) * (ngrid >> 3) + (blockIdx.x >> 3);
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
        for (int j = tid; j < ns; j += 256) lst[j] = uint32_t(j);     // field 0: always visible
        len = ns;
        // candidates j in [s, band_lo) alive at the first row, in index order
        for (int base = s; base < band_lo; base += 256 * 16) {
            const int j0 = base + tid * 16;
            int rr[16];
            int cnt = 0;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                rr[u] = (j0 + u < band_lo) ? rk[j0 + u] : kNotCand;
                cnt += (rr[u] <= thr0) ? 1 : 0;
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
            int o = len + woff + incl - cnt;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (rr[u] <= thr0) lst[o++] = (uint32_t(rr[u] + 1) << 16) | uint32_t(j0 + u);
            }
            len += tot;
            __syncthreads();
        }
        // pad to whole blocks with entries no row sees (field 0xffff, key 0)
        for (int e = len + tid; e < ((len + 63) & ~63); e += 256) lst[e] = 0xffff0000u;
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
    // list entry e is visible to this row iff e <= lim (field <= thr_row + 1)
    const uint32_t lim = (uint32_t(min(max(thr_row + 1, 0), 0xfffe)) << 16) | 0xffffu;
    const float csc = kLog2e * rsqrtf(float(D));

    float m_run = -INFINITY;
    float l_run = 0.0f;
    f32x16 acc_o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x16{};

    const int nlist = (len + 63) / 64;
    const int nband = (band_hi - band_lo + 1 + 63) / 64;

    // ranks of the first 128 band keys: a band key j can be a retained column
    // of a row of the tile only if j <= i_last - w < band_lo + P - 1 <= band_lo + 127
    if (tid < 128) {
        const int j = band_lo + tid;
        brank[tid] = (j < s) ? -1 : ((j <= band_hi) ? rk[j] : kNotCand);   // sink always passes
    }

    // Chunk c = tid + 256x of a 64-key tile is stored chunk c % CPR of tile row
    // c / CPR and holds that key's 8-dim chunk (c % CPR) ^ swz(row).  swz puts
    // 8 consecutive rows on 8 distinct bank groups (row-strided K reads) and
    // the 4-row x 2-chunk patch of one 16-lane transposing V read likewise.
    // The list entry is read for band blocks too (clamped, unused) so that the
    // fetch stays branch-free.
    int frow[NCH], fchk[NCH];
#pragma unroll
    for (int x = 0; x < NCH; ++x) {
        const int c = tid + 256 * x;
        frow[x] = c / CPR;
        fchk[x] = ((c % CPR) ^ swz(frow[x])) * 8;
    }
    const int nblk = nlist + nband;
    u32x4 kpre[NCH], vpre[NCH];
#define LTE_FETCH(BLK)                                                                   \
    {                                                                                    \
        const int fb = (BLK);                                                            \
        _Pragma("unroll") for (int x = 0; x < NCH; ++x) {                                \
            const int e = fb * 64 + frow[x];                                             \
            const int lrow = int(lst[min(e, kMaxList - 1)] & 0xffffu);                   \
            const int brow = min(band_lo + (fb - nlist) * 64 + frow[x], band_hi);        \
            const int row = (fb < nlist) ? lrow : brow;                                  \
            const long off = long(row) * kv_row + fchk[x];                               \
            kpre[x] = *reinterpret_cast<const u32x4*>(kbase + off);                        \
            vpre[x] = *reinterpret_cast<const u32x4*>(vbase + off);                        \
        }                                                                                \
    }
#define LTE_STAGE()                                                                      \
    {                                                                                    \
        _Pragma("unroll") for (int x = 0; x < NCH; ++x) {                                \
            Ks[tid + 256 * x] = kpre[x];                                                 \
            Vs[tid + 256 * x] = vpre[x];                                                 \
        }                                                                                \
    }
    LTE_FETCH(0)
    __syncthreads();                              // band ranks visible
    LTE_STAGE()
    __syncthreads();

    for (int blk = 0; blk < nblk; ++blk) {
        const bool is_list = blk < nlist;
        const int jb0 = band_lo + (blk - nlist) * 64;     // first key of a band block
        if (blk + 1 < nblk) LTE_FETCH(blk + 1)            // in flight during this block

        // ---- S^T = K Q^T for 64 keys x this wave's 32 rows -----------------------
        f32x16 sacc[2];
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int row = ks * 32 + (lane & 31);
                const bf16x8 a = __builtin_bit_cast(bf16x8, Ks[row * CPR + ((2 * kk + half) ^ swz(row))]);
                sacc[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[ks], 0, 0, 0);
            }
        }
        // ---- mask: element e of subtile ks is key slot
        //      ks*32 + (e/4)*8 + half*4 + e%4 of this block ----------------------------
        float x[2][16];
        if (is_list) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int t0 = ks * 32 + e4 * 8 + half * 4;
                    const u32x4 ent = *reinterpret_cast<const u32x4*>(&lst[blk * 64 + t0]);
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        x[ks][e4 * 4 + u] = (ent[u] <= lim) ? sacc[ks][e4 * 4 + u] : -INFINITY;
                }
            }
        } else {
            const bool full = (jb0 >= i_last - w + 1) && (jb0 + 63 <= i0);
            if (full) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int e = 0; e < 16; ++e) x[ks][e] = sacc[ks][e];
            } else {
                // d = irow - j: visible iff 0 <= d < w, or d >= w and j passes
                // (sink ranks read -1); blocks past the second hold no d >= w
                const int rb = min(blk - nlist, 1) * 64;
                const int dbase = irow - jb0 - half * 4;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        const int t0 = ks * 32 + e4 * 8 + half * 4;
                        const int4 br = *reinterpret_cast<const int4*>(&brank[rb + t0]);
                        const int bv[4] = {br.x, br.y, br.z, br.w};
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int d = dbase - (ks * 32 + e4 * 8 + u);
                            const bool vis = (unsigned(d) < unsigned(w)) |
                                             ((d >= 0) & (bv[u] <= thr_row));
                            x[ks][e4 * 4 + u] = vis ? sacc[ks][e4 * 4 + u] : -INFINITY;
                        }
                    }
                }
            }
        }

        // ---- online softmax in raw logits (scale folded into the exponent; row =
        //      this lane's query, keys split with lane^32) ------------------------------
        float mloc = x[0][0];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, x[ks][e]);
        const float mrow = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const float m_new = fmaxf(m_run, mrow);
        const float msafe = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = fast_exp2((m_run - msafe) * csc);
        const float moff = -msafe * csc;
        float lsum = 0.0f;
        bf16x8 pf[4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = fast_exp2(fmaf(x[ks][e], csc, moff));
                lsum += p;
                pf[ks * 2 + (e >> 3)][e & 7] = (__bf16)p;
            }
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc_o[dt] *= alpha;
        }

        // ---- O^T += V^T P^T ------------------------------------------------------
        // operand element e of lane (16-group G, index i) is V[key][dt*32 + (G&1)*16 + i]
        // with key = cc*16 + (e<4 ? 4h + e : 8 + 4h + e-4), h = lane/32: two
        // transposing reads, each of 4 keys, from rows that lane i of the group names
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                bf16x8 a;
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int grp = lane >> 4;
                    const int i = lane & 15;
                    const int key = cc * 16 + 8 * r + 4 * (grp >> 1) + (i >> 2);
                    const int d0 = dt * 32 + (grp & 1) * 16 + 4 * (i & 3);
                    const int chunk = (d0 >> 3) ^ swz(key);
                    const __bf16* src = reinterpret_cast<const __bf16*>(&Vs[key * CPR + chunk]) + (d0 & 7);
                    typedef short v4i16 __attribute__((ext_vector_type(4)));
                    const v4i16 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16*)(src));
                    const bf16x4 b4 = __builtin_bit_cast(bf16x4, t4);
                    a[4 * r + 0] = b4[0];
                    a[4 * r + 1] = b4[1];
                    a[4 * r + 2] = b4[2];
                    a[4 * r + 3] = b4[3];
                }
                acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[cc], acc_o[dt], 0, 0, 0);
            }
        }
        __syncthreads();                          // every wave is done with the tiles
        if (blk + 1 < nblk) {
            LTE_STAGE()
            __syncthreads();
        }
    }
#undef LTE_FETCH
#undef LTE_STAGE

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
