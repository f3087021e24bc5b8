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
//   1. compact the candidates in index order (four tokens per thread a round),
//      with the AND and OR of their keys;
//   2. stable LSD radix sort of their fp32 score bits (descending, ties keep
//      index order) -> sorted index array sidx, rank[sidx[p]] = p.  Digits that
//      every key shares are skipped, and so are key bits that never differ;
//   3. cumulative position bitmaps: snapshot kb holds every candidate of rank
//      < (kb+1) * RBS; per-word prefix popcounts, and M[kb] = the position of
//      the C-th set bit of snapshot kb (non-increasing in kb).  rank_out is
//      written once, coalesced, from the inverse permutation kept in LDS;
//   4. for each prefix end m: the first snapshot kb with M[kb] <= m contains
//      the C-th smallest rank; search that rank block for the exact rank, 64
//      entries at a time across the wave.
// The work is VALU-bound on the compute units it occupies: wave scans use DPP
// moves rather than LDS permutes, and same-digit masks take one ballot and two
// bitwise ops per varying key bit.
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

// Lanes of this wave that are valid and hold the digit d (8 bits) of this lane: a lane
// differs where any bit's ballot differs from this lane's bit.  Bits clear in vbits
// (wave-uniform) are alike in every key and are not looked at.
__device__ __forceinline__ unsigned long long same_digit(int d, bool valid, uint32_t vbits) {
    uint32_t dlo = 0u, dhi = 0u;                    // the two halves of the difference mask
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        if (((vbits >> bit) & 1u) == 0u) continue;
        const int sb = (d << (31 - bit)) >> 31;     // this lane's bit as 0 or all ones
        const unsigned long long bb = __ballot(sb != 0);
        dlo |= uint32_t(bb) ^ uint32_t(sb);
        dhi |= uint32_t(bb >> 32) ^ uint32_t(sb);
    }
    return __ballot(valid) & ~((static_cast<unsigned long long>(dhi) << 32) | dlo);
}

// OR of a value over the wave, by the same DPP pattern (lane 63 ends with all lanes).
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
    int x = int(v);
    x |= __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
    x |= __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
    x |= __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
    x |= __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
    x |= __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
    x |= __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
    return uint32_t(__builtin_amdgcn_readlane(x, 63));
}

// Position of the need-th set bit (need in [1, popcount]) of a 32-bit word, by
// halving: each step keeps the half that holds it.
__device__ __forceinline__ int nth_set_bit32(uint32_t x, int need) {
    int pos = 0;
#pragma unroll
    for (int half = 16; half >= 1; half >>= 1) {
        const int c = __popc(x & ((1u << half) - 1u));
        const bool up = need > c;
        need = up ? need - c : need;
        pos = up ? pos + half : pos;
        x = up ? (x >> half) : x;
    }
    return pos;
}

__device__ __forceinline__ int nth_set_bit64(unsigned long long x, int need) {
    const int c = __popc(uint32_t(x));
    const bool up = need > c;
    return (up ? 32 : 0) + nth_set_bit32(up ? uint32_t(x >> 32) : uint32_t(x), up ? need - c : need);
}

// Block-wide exclusive scan of one int per thread (1024 threads).
__device__ __forceinline__ int block_excl_scan(int x, int* wsum, int* total) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int incl = wave_incl_sum(x);
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
    __shared__ uint32_t wand[kSelWaves], wor[kSelWaves];   // per-wave AND / OR of the keys
    __shared__ __align__(16) uint32_t lsc[LDS ? kSelLdsWords : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int bg = blockIdx.x;
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
    // Four consecutive tokens per thread per round (one block scan per 4096 tokens), the
    // next round's scores read ahead; the AND and OR of the candidate keys tell which
    // radix digits vary at all.
    int n = 0;
    uint32_t kand = ~0u, kor = 0u;
    float r_next[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r_next[u] = (4 * tid + u < T) ? r[4 * tid + u] : 0.0f;
    for (int base = 0; base < T; base += 4 * kSelThreads) {
        const int j0 = base + 4 * tid;
        float rj[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            rj[u] = r_next[u];
            const int jn = j0 + 4 * kSelThreads + u;
            if (jn < T) r_next[u] = r[jn];
        }
        bool cand[4];
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + u;
            cand[u] = (j < T) && (j >= s) && (j <= last_leaving) && (rj[u] > 0.5f);
            cnt += cand[u] ? 1 : 0;
        }
        int tot;
        int off = n + block_excl_scan(cnt, wsum, &tot);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (cand[u]) {
                const uint32_t key = ~__float_as_uint(rj[u]);   // ascending key = descending score
                cidx[off] = uint32_t(j0 + u);
                ckey[off] = key;
                kand &= key;
                kor |= key;
                ++off;
            }
        }
        n += tot;
    }
    if (tid == 0) ncand_out[bg] = n;

    if (C == 0 || n <= C) {
        // nothing or everything is kept: rank 0 for each candidate
        for (int j = tid; j < T; j += kSelThreads) rk[j] = kNotCand;
        __syncthreads();                            // the candidate list, and the stores above first
        if (C != 0)
            for (int p = tid; p < n; p += kSelThreads) rk[cidx[p]] = 0;
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
    kand = ~wave_or(~kand);
    kor = wave_or(kor);
    if (lane == 0) { wand[wave] = kand; wor[wave] = kor; }
    __syncthreads();
    uint32_t vary = 0u;                                 // key bits that differ between candidates
    {
        uint32_t a = ~0u, o = 0u;
#pragma unroll
        for (int q = 0; q < kSelWaves; ++q) { a &= wand[q]; o |= wor[q]; }
        vary = a ^ o;
    }
#pragma unroll
    for (int e = 0; e < ELEMS; ++e) {
        const int p = wbase + e * 64 + lane;
        key[e] = p < n ? ckey[p] : 0u;
        idx[e] = p < n ? cidx[p] : 0u;
    }
    bool in_tmp = false;                                // where the sorted data lives
    // Offsets of each element among its wave's keys of the same digit, kept from the
    // counting walk for the placing walk (for ELEMS = 4; the 32-element form recounts
    // to stay within its registers).
    constexpr bool kKeepOffs = ELEMS <= 4;
    int offs[kKeepOffs ? ELEMS : 1];
    for (int shift = 0; shift < 32; shift += 8) {
        // a digit every key shares leaves the order as it is
        if (((vary >> shift) & 255u) == 0u) continue;
        const uint32_t vbits = (vary >> shift) & 255u;
        int* wc = wcnt[wave];
        for (int x = lane; x < 256; x += 64) wc[x] = 0;
#pragma unroll
        for (int e = 0; e < ELEMS; ++e) {
            if (wbase + e * 64 >= n) break;             // uniform across the wave
            const bool valid = wbase + e * 64 + lane < n;
            const int d = int((key[e] >> shift) & 255);
            const unsigned long long mask = same_digit(d, valid, vbits);
            const int before = valid ? wc[d] : 0;       // this digit in earlier groups
            const int lrank = __popcll(mask & lanemask_lt(lane));
            if constexpr (kKeepOffs) offs[e] = before + lrank;
            if (valid && lrank == 0) wc[d] = before + __popcll(mask);
        }
        __syncthreads();
        // digit totals
        if (tid < 256) {
            int tot = 0;
#pragma unroll
            for (int q = 0; q < kSelWaves; ++q) tot += wcnt[q][tid];
            hist[tid] = tot;
        }
        __syncthreads();
        // exclusive scan of the 256 digit totals (wave 0, 4 digits per lane)
        if (wave == 0) {
            int h0 = hist[lane * 4 + 0], h1 = hist[lane * 4 + 1];
            int h2 = hist[lane * 4 + 2], h3 = hist[lane * 4 + 3];
            int sum = h0 + h1 + h2 + h3;
            int ex = wave_incl_sum(sum) - sum;
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
            if constexpr (kKeepOffs) {
                if (valid) {
                    const int at = wc[d] + offs[e];     // (wave, digit) start + offset
                    okey[at] = key[e];
                    oidx[at] = idx[e];
                }
            } else {
                const unsigned long long mask = same_digit(d, valid, vbits);
                const int lrank = __popcll(mask & lanemask_lt(lane));
                const int at = valid ? wc[d] : 0;       // next free position of the digit
                if (valid) {
                    okey[at + lrank] = key[e];
                    oidx[at + lrank] = idx[e];
                    if (lrank == 0) wc[d] = at + __popcll(mask);
                }
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
    // the inverse permutation (each candidate's rank, by index) goes into the key
    // buffer, free now; rank_out is written from it in one coalesced pass below
    uint32_t* inv = ckey;
#pragma unroll
    for (int e = 0; e < ELEMS; ++e) {
        int p = wbase + e * 64 + lane;
        if (p < n) inv[idx[e]] = uint32_t(p);
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
        for (int kb0 = 0; kb0 < nsnap; kb0 += 8) {     // eight loads in flight
            uint32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = (kb0 + u < nsnap) ? bm[long(kb0 + u) * W + wd] : 0u;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                acc |= v[u];
                if (kb0 + u < nsnap) bm[long(kb0 + u) * W + wd] = acc;
            }
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
            const int incl = wave_incl_sum(pc);
            const int ex = running + incl - pc;
            if (wd < W) pre[long(kb) * W + wd] = ex;
            // at most one word holds the C-th set bit
            const unsigned long long hit = __ballot(ex < C && ex + pc >= C);
            if (hit != 0ull) {
                const int hl = __ffsll((unsigned long long)hit) - 1;
                const uint32_t hw = uint32_t(__builtin_amdgcn_readlane(int(word), hl));
                const int hex = __builtin_amdgcn_readlane(ex, hl);
                found = (c0 + hl) * 32 + nth_set_bit32(hw, C - hex);
            }
            running += __builtin_amdgcn_readlane(incl, 63);
        }
        if (lane == 0) Msnap[kb] = found;
    }
    __threadfence_block();
    __syncthreads();

    // rank_out: the candidates are the bits of the last (cumulative) snapshot
    {
        const uint32_t* all = bm + long(nsnap - 1) * W;
        for (int j = tid; j < T; j += kSelThreads)
            rk[j] = ((all[j >> 5] >> (j & 31)) & 1u) ? int32_t(inv[j]) : kNotCand;
    }

    // ---- 4. thr[m] ---------------------------------------------------------------
    // Lanes hold consecutive m (a wave covers [mb, mb + 64)).  Per m: the snapshot lo,
    // the count of candidates j <= m of rank < lo * rbs, and need = C - that count >= 1;
    // thr[m] is the rank of the need-th entry of rank block lo, in rank order, whose
    // index is <= m.  The wave takes its lanes' blocks one at a time, 64 entries per
    // round with entry q in lane q.  Entries of index below mb are hits for every lane,
    // those at mb + 64 or above for none; the few in between are tested lane by lane.
    const int mlast = Msnap[nsnap - 1];                 // first m with >= C candidates <= m
    for (int mb = wave * 64; mb < T; mb += kSelThreads) {
        const int m = mb + lane;
        const bool active = m < T && m >= mlast;
        if (m < T && m < mlast) th[m] = kAllPass;
        // lo = the smallest kb with Msnap[kb] <= m = the count of kb with Msnap[kb] > m
        // (Msnap does not increase with kb): values at mb + 64 or above count for every
        // lane, those at mb or below for none, the few in between lane by lane
        int lo = 0, need = 0;
        for (int kb0 = 0; kb0 < nsnap; kb0 += 64) {
            const int kb = kb0 + lane;
            const int v = kb < nsnap ? Msnap[kb] : -1;
            lo += __popcll(__ballot(v >= mb + 64));
            unsigned long long win = __ballot(v > mb && v < mb + 64);
            while (win != 0ull) {
                const int l = __ffsll((unsigned long long)win) - 1;
                win &= win - 1ull;
                lo += (m < __builtin_amdgcn_readlane(v, l)) ? 1 : 0;
            }
        }
        if (active) {
            const int wd = m >> 5;
            const int bit = m & 31;
            const uint32_t low = (bit == 31) ? 0xffffffffu : ((2u << bit) - 1u);
            int basecnt = 0;
            if (lo > 0) basecnt = pre[long(lo - 1) * W + wd] + __popc(bm[long(lo - 1) * W + wd] & low);
            need = C - basecnt;
        }
        int res = 0;
        unsigned long long todo = __ballot(active);
        while (todo != 0ull) {
            const int blo = __builtin_amdgcn_readlane(lo, __ffsll((long long)todo) - 1);
            const bool mine = active && lo == blo;
            const int p0 = blo * rbs;
            const int p1 = min(n, p0 + rbs);
            int nd = need;
            int r = p1 - 1;
            bool done = !mine;
            for (int c = p0; c < p1; c += 64) {
                if (__ballot(!done) == 0ull) break;
                const int q = c + lane;
                const uint32_t e = q < p1 ? sidx[q] : 0xffffffffu;
                unsigned long long hits = __ballot(q < p1 && e < uint32_t(mb));
                unsigned long long mids = __ballot(q < p1 && e >= uint32_t(mb) && e < uint32_t(mb + 64));
                while (mids != 0ull) {
                    const int qq = __ffsll((long long)mids) - 1;
                    mids &= mids - 1ull;
                    const uint32_t eq = uint32_t(__builtin_amdgcn_readlane(int(e), qq));
                    if (eq <= uint32_t(m)) hits |= 1ull << qq;
                }
                const int cnt = __popcll(hits);
                if (!done) {
                    if (nd <= cnt) { r = c + nth_set_bit64(hits, nd); done = true; }
                    else nd -= cnt;
                }
            }
            if (mine) res = r;
            todo &= ~__ballot(mine);
        }
        if (active) th[m] = res;
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
