// Keep/evict selection of a whole prompt on gfx950.
//
// LTE paper (arXiv 2510.20787) summary page, Figure 2 caption: whether a KV
// pair is evicted is decided when it moves out of the sliding window, from its
// retention score; the abstract and TL;DR cap the retained set per head (a
// budget).  Keep rule taken here: token j >= s is a candidate iff r_j > 0.5;
// at most C are kept; on overflow the C best by (score desc, index asc) stay.
//
// Retained set at query i: R_i = TopC{candidates j <= i - w}.  Because the
// order is a strict total order, a streaming top-C equals this closed form,
// so the sequential eviction process is replaced by a parallel one:
//   rank[j]  = position of candidate j in the (score desc, index asc) order,
//   thr[m]   = the C-th smallest rank among candidates j <= m
//              (kAllPass when at most C such candidates exist),
// and j is in R_i  <=>  j <= i - w  and  rank[j] <= thr[i - w].
//
// One workgroup (1024 threads) per (batch, KV head):
//   1. compact the candidates in index order;
//   2. stable LSD radix sort of their fp32 score bits (descending, ties keep
//      index order) -> sorted index array sidx, rank[sidx[p]] = p;
//   3. cumulative position bitmaps: snapshot kb holds every candidate of rank
//      < (kb+1) * RBS; per-word prefix popcounts, and M[kb] = the position of
//      the C-th set bit of snapshot kb (non-increasing in kb);
//   4. for each prefix end m: the first snapshot kb with M[kb] <= m contains
//      the C-th smallest rank; scan that rank block for the exact rank.
#include "lte_internal.h"

namespace lte {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
// Prompts of up to kSelLdsT tokens keep the whole per-(b, g) scratch (sort
// buffers, snapshot bitmaps and their prefix counts: 128 KB) in LDS, which
// turns every phase's global round trips into LDS ones; longer prompts use the
// workspace.
constexpr int kSelLdsT = 4096;
constexpr int kSelLdsWords = 4 * kSelLdsT + 2 * (kSelLdsT / 64) * (kSelLdsT / 32);

__device__ __forceinline__ unsigned long long lanemask_lt(int lane) {
    return lane == 0 ? 0ull : ((~0ull) >> (64 - lane));
}

// Lanes of this wave that are valid and hold the digit d (8 bits) of this lane.
__device__ __forceinline__ unsigned long long same_digit(int d, bool valid) {
    unsigned long long mask = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const unsigned long long bb = __ballot((d >> bit) & 1);
        mask &= ((d >> bit) & 1) ? bb : ~bb;
    }
    return mask;
}

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ __forceinline__ int block_excl_scan(int x, int* wsum, int* total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int incl = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int q = 0; q < kSelWaves; ++q) {
        int c = wsum[q];
        woff += (q < wave) ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return woff + incl - x;
}

template <int ELEMS, bool LDS>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    int T, int Hkv, int s, int w, int C, int rbs, int nsnap_max, long scratch_words,
    const int32_t* __restrict__ seq_lens, const float* __restrict__ scores,
    int32_t* __restrict__ rank_out,
    int32_t* __restrict__ thr_out, int32_t* __restrict__ ncand_out,
    uint32_t* __restrict__ scratch) {
    __shared__ int wsum[kSelWaves];
    __shared__ int hist[256];
    __shared__ int wcnt[kSelWaves][256];
    __shared__ int dbase[256];
    __shared__ int Msnap[1024];
    __shared__ int skipf[4];                        // per radix pass: every key has one digit
    __shared__ __align__(16) uint32_t lsc[LDS ? kSelLdsWords : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int bg = blockIdx.x;
    if (tid < 4) skipf[tid] = 0;                   // read after the barriers below
    const float* r = scores + long(bg) * T;
    int32_t* rk = rank_out + long(bg) * T;
    int32_t* th = thr_out + long(bg) * T;
    uint32_t* sc;
    if constexpr (LDS) sc = lsc;
    else sc = scratch + long(bg) * scratch_words;
    const long Tp = (long(T) + 63) & ~63L;           // 256-byte aligned array stride
    uint32_t* cidx = sc;
    uint32_t* ckey = sc + Tp;
    uint32_t* tidx = sc + 2L * Tp;
    uint32_t* tkey = sc + 3L * Tp;
    const int W = (T + 31) / 32;
    uint32_t* bm = sc + 4L * Tp;                     // [nsnap][W]
    uint32_t* pre = bm + long(nsnap_max) * W;        // [nsnap][W]

    // ---- 1. candidates in index order -------------------------------------
    const int Tb = seq_len_of(seq_lens, bg / Hkv, T);    // this sequence's length
    const int last_leaving = Tb - 1 - w;             // last token that leaves the window
    int n = 0;
    float r_next = (tid < T) ? r[tid] : 0.0f;       // scores read one group ahead
    for (int base = 0; base < T; base += kSelThreads) {
        const int j = base + tid;
        const float rj = r_next;
        if (j + kSelThreads < T) r_next = r[j + kSelThreads];
        bool cand = false;
        if (j < T) {
            cand = (j >= s) && (j <= last_leaving) && (rj > 0.5f);
            rk[j] = kNotCand;
        }
        int tot;
        int off = block_excl_scan(cand ? 1 : 0, wsum, &tot);
        if (cand) {
            cidx[n + off] = uint32_t(j);
            ckey[n + off] = ~__float_as_uint(rj);    // ascending key = descending score
        }
        n += tot;
    }
    if (tid == 0) ncand_out[bg] = n;

    if (C == 0 || n <= C) {
        // nothing or everything is kept: rank 0 for each candidate
        __syncthreads();
        for (int p = tid; p < n; p += kSelThreads) rk[cidx[p]] = (C == 0) ? kNotCand : 0;
        const int32_t tv = (C == 0) ? -1 : kAllPass;
        for (int m = tid; m < T; m += kSelThreads) th[m] = tv;
        return;
    }

    // ---- 2. stable LSD radix sort, 8 bits per pass ---------------------------
    // Wave w holds sequence positions [w*ELEMS*64, (w+1)*ELEMS*64), element e of
    // lane l at position (w*ELEMS + e)*64 + l.  A pass ranks each wave's
    // elements against its own digit counters, 64 at a time in position order
    // (no block barrier between groups), then one scan over (digit, wave)
    // turns the counters into each (wave, digit)'s first output position and
    // the same walk places the elements: the order within a digit is kept.
    uint32_t key[ELEMS], idx[ELEMS];
    const int wbase = wave * ELEMS * 64;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < ELEMS; ++e) {
        const int p = wbase + e * 64 + lane;
        key[e] = p < n ? ckey[p] : 0u;
        idx[e] = p < n ? cidx[p] : 0u;
    }
    bool in_tmp = false;                                // where the sorted data lives
    for (int shift = 0; shift < 32; shift += 8) {
        int* wc = wcnt[wave];
        for (int x = lane; x < 256; x += 64) wc[x] = 0;
#pragma unroll
        for (int e = 0; e < ELEMS; ++e) {
            if (wbase + e * 64 >= n) break;             // uniform across the wave
            const bool valid = wbase + e * 64 + lane < n;
            const int d = int((key[e] >> shift) & 255);
            const unsigned long long mask = same_digit(d, valid);
            const int before = valid ? wc[d] : 0;       // this digit in earlier groups
            if (valid && __popcll(mask & lanemask_lt(lane)) == 0) wc[d] = before + __popcll(mask);
        }
        __syncthreads();
        // digit totals; a pass in which every key has the same digit leaves the
        // order as is
        if (tid < 256) {
            int tot = 0;
#pragma unroll
            for (int q = 0; q < kSelWaves; ++q) tot += wcnt[q][tid];
            hist[tid] = tot;
            if (tot == n) skipf[shift >> 3] = 1;
        }
        __syncthreads();
        if (skipf[shift >> 3]) continue;
        // exclusive scan of the 256 digit totals (wave 0, 4 digits per lane)
        if (wave == 0) {
            int h0 = hist[lane * 4 + 0], h1 = hist[lane * 4 + 1];
            int h2 = hist[lane * 4 + 2], h3 = hist[lane * 4 + 3];
            int sum = h0 + h1 + h2 + h3;
            int incl = sum;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                int y = __shfl_up(incl, d, 64);
                if (lane >= d) incl += y;
            }
            int ex = incl - sum;
            dbase[lane * 4 + 0] = ex;
            dbase[lane * 4 + 1] = ex + h0;
            dbase[lane * 4 + 2] = ex + h0 + h1;
            dbase[lane * 4 + 3] = ex + h0 + h1 + h2;
        }
        __syncthreads();
        // first output position of (wave q, digit): digit base plus the digit's
        // count in the waves before q
        if (tid < 256) {
            int run = dbase[tid];
#pragma unroll
            for (int q = 0; q < kSelWaves; ++q) {
                const int c = wcnt[q][tid];
                wcnt[q][tid] = run;
                run += c;
            }
        }
        __syncthreads();
        uint32_t* okey = in_tmp ? ckey : tkey;
        uint32_t* oidx = in_tmp ? cidx : tidx;
#pragma unroll
        for (int e = 0; e < ELEMS; ++e) {
            if (wbase + e * 64 >= n) break;
            const bool valid = wbase + e * 64 + lane < n;
            const int d = int((key[e] >> shift) & 255);
            const unsigned long long mask = same_digit(d, valid);
            const int lrank = __popcll(mask & lanemask_lt(lane));
            const int at = valid ? wc[d] : 0;           // next free position of the digit
            if (valid) {
                okey[at + lrank] = key[e];
                oidx[at + lrank] = idx[e];
                if (lrank == 0) wc[d] = at + __popcll(mask);
            }
        }
        in_tmp = !in_tmp;
        __threadfence_block();
        __syncthreads();
#pragma unroll
        for (int e = 0; e < ELEMS; ++e) {
            const int p = wbase + e * 64 + lane;
            key[e] = p < n ? okey[p] : 0u;
            idx[e] = p < n ? oidx[p] : 0u;
        }
        __syncthreads();
    }
    // key/idx registers now hold the sorted order: element e of this lane is at
    // position wbase + e*64 + lane.
    const uint32_t* sidx = in_tmp ? tidx : cidx;
#pragma unroll
    for (int e = 0; e < ELEMS; ++e) {
        int p = wbase + e * 64 + lane;
        if (p < n) rk[idx[e]] = p;
    }

    // ---- 3. cumulative rank-block bitmaps --------------------------------------
    const int nsnap = (n + rbs - 1) / rbs;
    for (long x = tid; x < long(nsnap) * W; x += kSelThreads) bm[x] = 0u;
    __threadfence_block();
    __syncthreads();
#pragma unroll
    for (int e = 0; e < ELEMS; ++e) {
        int p = wbase + e * 64 + lane;
        if (p < n) {
            uint32_t j = idx[e];
            atomicOr(&bm[long(p / rbs) * W + (j >> 5)], 1u << (j & 31));
        }
    }
    __threadfence_block();
    __syncthreads();
    for (int wd = tid; wd < W; wd += kSelThreads) {     // prefix-OR over snapshots
        uint32_t acc = 0u;
        for (int kb = 0; kb < nsnap; ++kb) {
            acc |= bm[long(kb) * W + wd];
            bm[long(kb) * W + wd] = acc;
        }
    }
    __threadfence_block();
    __syncthreads();
    // one wave per snapshot: exclusive prefix popcounts and the C-th set bit
    for (int kb = wave; kb < nsnap; kb += kSelWaves) {
        int running = 0;
        int found = 0x7fffffff;
        for (int c0 = 0; c0 < W; c0 += 64) {
            const int wd = c0 + lane;
            const uint32_t word = wd < W ? bm[long(kb) * W + wd] : 0u;
            const int pc = __popc(word);
            int incl = pc;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                int y = __shfl_up(incl, d, 64);
                if (lane >= d) incl += y;
            }
            const int ex = running + incl - pc;
            if (wd < W) pre[long(kb) * W + wd] = ex;
            if (ex < C && ex + pc >= C) {               // the C-th set bit is in this word
                int need = C - ex;
                uint32_t x = word;
                int bit = 0;
                for (;;) {
                    bit = __ffs(x) - 1;
                    if (--need == 0) break;
                    x &= x - 1;
                }
                found = wd * 32 + bit;
            }
            running += __shfl(incl, 63, 64);
        }
        // at most one lane found it
        for (int d = 32; d >= 1; d >>= 1) {
            int y = __shfl_xor(found, d, 64);
            found = min(found, y);
        }
        if (lane == 0) Msnap[kb] = found;
    }
    __threadfence_block();
    __syncthreads();

    // ---- 4. thr[m] ---------------------------------------------------------------
    const int mlast = Msnap[nsnap - 1];                 // first m with >= C candidates <= m
    for (int m = tid; m < T; m += kSelThreads) {
        if (m < mlast) { th[m] = kAllPass; continue; }
        int lo = 0, hi = nsnap - 1;                     // smallest kb with Msnap[kb] <= m
        while (lo < hi) {
            int mid = (lo + hi) >> 1;
            if (Msnap[mid] <= m) hi = mid; else lo = mid + 1;
        }
        const int wd = m >> 5;
        const int bit = m & 31;
        const uint32_t low = (bit == 31) ? 0xffffffffu : ((2u << bit) - 1u);
        int basecnt = 0;
        if (lo > 0) basecnt = pre[long(lo - 1) * W + wd] + __popc(bm[long(lo - 1) * W + wd] & low);
        int need = C - basecnt;                         // >= 1
        const int p0 = lo * rbs;
        const int p1 = min(n, p0 + rbs);
        int res = p1 - 1;
        // the rank block in chunks of 64 entries, each chunk's loads issued together
        for (int c = p0; c < p1 && need > 0; c += 64) {
            uint4 v[16];
            const uint4* src = reinterpret_cast<const uint4*>(sidx + c);
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = src[q];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const uint32_t e4[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    // branch-free: need keeps counting down past zero, so it equals
                    // zero right after exactly one hit, the need-th
                    const int p = c + 4 * q + u;
                    const int hit = (p < p1 && e4[u] <= uint32_t(m)) ? 1 : 0;
                    need -= hit;
                    res = (hit != 0 && need == 0) ? p : res;
                }
            }
        }
        th[m] = res;
    }
}

}  // namespace

hipError_t launch_select(const Shape& sh, int64_t T, const int32_t* seq_lens, const float* scores,
                         int32_t* rank, int32_t* thr, int32_t* ncand, uint32_t* scratch,
                         hipStream_t st) {
    const int rbs = select_rbs(T);
    const int nsnap_max = int(select_nsnap_max(T));
    const long words = long(select_scratch_words(T));
    dim3 grid(unsigned(sh.B * sh.Hkv));
    if (T <= kSelLdsT && words <= kSelLdsWords) {
        static_assert(kSelLdsT <= 4 * kSelThreads, "four sort elements per thread");
        hipLaunchKernelGGL((select_kernel<4, true>), grid, dim3(kSelThreads), 0, st, int(T),
                           sh.Hkv, sh.s, sh.w, sh.C, rbs, nsnap_max, words, seq_lens, scores,
                           rank, thr, ncand, scratch);
    } else if (T <= 4 * kSelThreads) {
        hipLaunchKernelGGL((select_kernel<4, false>), grid, dim3(kSelThreads), 0, st, int(T),
                           sh.Hkv, sh.s, sh.w, sh.C, rbs, nsnap_max, words, seq_lens, scores,
                           rank, thr, ncand, scratch);
    } else {
        hipLaunchKernelGGL((select_kernel<32, false>), grid, dim3(kSelThreads), 0, st, int(T),
                           sh.Hkv, sh.s, sh.w, sh.C, rbs, nsnap_max, words, seq_lens, scores,
                           rank, thr, ncand, scratch);
    }
    return hipGetLastError();
}

}  // namespace lte
