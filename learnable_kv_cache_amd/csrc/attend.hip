// A-plus-column sparse causal attention for a whole prompt on gfx950.
//
// LTE paper (arXiv 2510.20787) summary page, Figure 2 caption (right panel):
// each head attends to the sink columns, the diagonal band of the sliding
// window ("A") and vertical stripes for the retained tokens ("column").
// Query row i sees V(i) = [0, min(s, i+1)) U [i-w+1, i] U R_i, with
// j in R_i <=> j <= i-w and rank[j] <= thr[i-w] (selection kernel).
//
// Tiling (one workgroup = 8 waves = 256 MFMA rows, one workgroup per CU):
//   * GQA packing: the G = Hq/Hkv query heads of a group share their keys, so
//     a tile is P = 256/G consecutive positions x G heads of one KV head.
//     Its band of keys is [i0-w+1, i0+P-1] (P+w-1 keys for P rows).
//   * keys are processed in blocks of 64: first the band blocks, then the
//     gathered columns below the band (sink + retained tokens alive at the
//     tile's first row, via the per-head rank/thr lists).  With two band
//     blocks or more the list is built after the first one, whose compute
//     hides the rank loads' latency.  Entries that every row of the tile sees
//     come first, so only the last list blocks need a mask.
//   * K/V tiles are double-buffered in LDS.  The next block is copied straight
//     from global memory into the free buffer while the current one is
//     computed (global_load_lds, issued from inline assembly so that the
//     compiler does not make the current buffer's operand reads wait for it);
//     each wave waits for its own copies at the end of the block, and one
//     barrier per block publishes them.  The first block's copy is issued
//     behind the rank loads, so the gathered list is built while it is in
//     flight.  Scheduling groups keep three k-steps of K operands and four V
//     operands in flight ahead of the MFMAs.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K rows from LDS are the A
//     operand, each wave's 32 query rows stay in registers as the B operand.
//     A lane then owns one query row, so the row max/sum of the online
//     softmax is a 32-value local reduction plus one lane swap.
//   * O^T += V^T P^T: P^T comes straight from the S^T accumulator (converted
//     to bf16).  V stays row-major in LDS; its MFMA operand (8 keys of one
//     dim per lane) is read with ds_read_b64_tr_b16, whose 16-lane transpose
//     turns four 4-dim row pieces into four keys of one dim per lane.
//   * K and V tiles sit in LDS as 16-byte chunks XOR-swizzled by row (each
//     tensor its own pattern), so the row-strided MFMA operand reads hit
//     distinct banks.
//   * A block that needs a mask gets it as the first k-step's accumulator (0,
//     or -inf for a hidden key), built before its MFMAs: the logits then leave
//     the MFMAs in the registers the softmax reads, where a mask applied
//     afterwards made the compiler move all 32 of them on every unmasked block.
//   * fp32 online softmax on raw logits, the 1/sqrt(D) scale and log2(e)
//     folded into one FMA before exp2; masked keys are -inf.  p is taken
//     against a lazy reference maximum: a lane's sum of its block's p bounds
//     each of them, so the block maximum is computed (and the reference moved,
//     when exceeded by more than 2^8 in the exponent) only when that sum
//     passes 2^8; the running output is rarely rescaled.
//   * the output is staged through LDS and stored as whole rows.
#include "lte_internal.h"

#pragma clang diagnostic ignored "-Winline-asm"   // M0 on the clobber list of the tile copies

namespace lte {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max of x over lanes l and l ^ 32, by one cross-half swap (no LDS round trip)
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS chunk swizzle of tile row r (a key): the 16-byte chunk c of row r is
// stored at chunk position c ^ swz(r).  Two access patterns must spread over
// the banks: the K operand reads one chunk of 8 (or 16) consecutive rows, the
// transposing V read two (or four) adjacent chunks of 4 consecutive rows.
// D = 128 (256-byte rows): swz(r) = T[r & 3] ^ ((r >> 2) & 3) with
// T = {0, 10, 4, 14}, which maps any aligned 8 rows to distinct positions mod
// 8 and 16 rows to distinct positions mod 16, and (row, chunk) of both V
// patterns likewise.  D = 64 (128-byte rows): 3 bits, (r&3)<<1 | (r>>2)&1.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return (((r & 1) * 10) | ((r & 2) << 1)) ^ ((r >> 2) & 3);
    else return ((r & 3) << 1) | ((r >> 2) & 1);
}

// LDS chunk swizzle of V tile row r.  The transposing V read takes, for one
// output tile of 32 dims, 4 consecutive keys x 64 bytes per 32 lanes; XOR-ing
// bits 2-3 of the chunk index with the key's position in its group of 4 (D =
// 128: 256-byte rows) or bit 1 of the key (D = 64: 128-byte rows, two per
// 256-byte bank line) puts those 4 key pieces in different 64-byte bank
// quarters, and leaves a lane's read address affine in the key and in the
// dim tile but for one XOR of the tile index.
template <int D>
__device__ __forceinline__ int vswz(int r) {
    if constexpr (D == 128) return (r & 3) << 2;
    else return ((r >> 1) & 1) << 2;
}

template <int D, int G>
__global__ __launch_bounds__(512) void attend_prefill_kernel(
    int T, int Hq, int Hkv, int s, int w, int ntile, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ q_lo, int q_rows, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ thr,
    const int32_t* __restrict__ ncand, uint16_t* __restrict__ out) {
    constexpr int NW = 8;                   // waves
    constexpr int P = NW * 32 / G;          // positions per tile
    constexpr int KK = D / 16;              // MFMA k-steps of q.k
    constexpr int DT = D / 32;              // 32-wide output tiles of o
    constexpr int CPR = D / 8;              // 16-byte chunks per key row
    constexpr int TCH = 64 * CPR;           // chunks of one 64-key tile
    constexpr int LPW = TCH / 64 / NW;      // direct loads per wave per tile and tensor
    constexpr int kMaxList = kMaxSink + kMaxCapacity + P;    // sink, retained, transient room
    constexpr int kListTop = kMaxList + 63;       // transient entries gather below it
    constexpr int kBr = P > 64 ? P : 64;    // band keys whose rank can matter, rounded up
    static_assert(LPW >= 1 && LPW * 64 * NW == TCH, "tile split");

    // double-buffered swizzled K and V tiles, one object per buffer so that the
    // compiler can tell a tile being read from the one being loaded
    __shared__ __align__(16) u32x4 K0[TCH];
    __shared__ __align__(16) u32x4 V0[TCH];
    __shared__ __align__(16) u32x4 K1[TCH];
    __shared__ __align__(16) u32x4 V1[TCH];
    // (field << 16) | token index; field = rank + 1 of a retained token, 0 for
    // a sink token, 0xffff for padding
    __shared__ __align__(16) uint32_t lst[kMaxList + 64];
    __shared__ __align__(16) int32_t brank[kBr];
    __shared__ int lfull[kMaxList / 64];            // list block visible to every row of the tile
    __shared__ int wcnt[2][64];                     // per (pass slot, wave) counts, stable | transient << 16
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;          // which half of the MFMA k-dimension a lane holds
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);

    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so map
    // each XCD's share to a contiguous run of tiles (neighbouring tiles of a
    // head share most of their band keys in that XCD's L2).  Each run is taken
    // from its end: a head's later tiles carry the longer gathered lists, so the
    // cheapest tiles come last and the launch's tail is short.
    const int ngrid = gridDim.x;
    int lin = ngrid - 1 - blockIdx.x;
    if ((ngrid & 7) == 0) lin = (blockIdx.x & 7) * (ngrid >> 3) + ((ngrid >> 3) - 1 - (blockIdx.x >> 3));
    const int bg = lin / ntile;
    const int tile = lin % ntile;
    const int b = bg / Hkv;
    const int g = bg % Hkv;
    const int i0 = tile * P;
    const int Tb = seq_len_of(seq_lens, b, T);      // this sequence's length
    if (i0 >= Tb) return;                           // every row of the tile is padding
    const int i_last = min(i0 + P, Tb) - 1;
    // with q_lo, only rows >= q_lo[b] are queries: q and out then hold q_rows rows
    // per sequence, row i at i - q_lo[b]
    const int qlo = q_lo ? q_lo[b] : 0;
    if (i_last < qlo) return;
    const long qrows = q_lo ? long(q_rows) : long(T);
    const int band_lo = max(0, i0 - w + 1);
    const int band_hi = i_last;
    const int nband = (band_hi - band_lo + 1 + 63) / 64;
    const int32_t* rk = rank + long(bg) * T;
    const int32_t* th = thr + long(bg) * T;
    // a (b, g) without candidates retains nothing: its ranks are not read and the
    // gathered list is the sink alone
    const bool has_cand = !(ncand != nullptr && ncand[bg] == 0);
    const int scan_hi = has_cand ? band_lo : s;
    // key rows of this (batch, KV head): byte offsets fit 32 bits (T * Hkv * D
    // * 2 < 2^31 is checked on the host) and row * kv_bytes fits 24-bit factors
    const char* kbytes = reinterpret_cast<const char*>(k + (long(b) * T * Hkv + g) * D);
    const char* vbytes = reinterpret_cast<const char*>(v + (long(b) * T * Hkv + g) * D);
    const uint32_t kv_bytes = uint32_t(Hkv * D * 2);

    // Blocks: the band blocks first, then the gathered columns below the band.
    // Block fb is copied straight from global memory into the tile buffers KB, VB:
    // load x of wave wv covers tile chunks [64x', 64x'+64), x' = wv*LPW + x, lane l
    // chunk 64x'+l; chunk c is tile row c / CPR at position c % CPR and holds that
    // key's chunk (c % CPR) ^ swz(row) (K) or ^ vswz(row) (V).  The copies are
    // global_load_lds written as inline assembly: the compiler, which cannot tell
    // their LDS writes from the operand reads of the other buffer, would otherwise
    // make every LDS read wait for them.  The end of each block waits for them
    // (LTE_WAIT_COPIES).  The kernel sets M0 only here.
#define LTE_COPY(BLK, KB, VB)                                                               \
    {                                                                                      \
        const int fb = (BLK);                                                              \
        _Pragma("unroll") for (int x = 0; x < LPW; ++x) {                                  \
            const int c = (wave * LPW + x) * 64 + lane;                                    \
            const int trow = c / CPR;                                                      \
            int row;                                                                       \
            if (fb < nband) row = min(band_lo + fb * 64 + trow, band_hi);                  \
            else row = int(lst[min((fb - nband) * 64 + trow, kMaxList - 1)] & 0xffffu);    \
            const uint32_t roff = __umul24(uint32_t(row), kv_bytes);                       \
            const char* ks_ = kbytes + roff + uint32_t(((c % CPR) ^ swz<D>(trow)) * 16);   \
            const char* vs_ = vbytes + roff + uint32_t(((c % CPR) ^ vswz<D>(trow)) * 16);  \
            const uint32_t kl_ = uint32_t(reinterpret_cast<uintptr_t>(                     \
                (__attribute__((address_space(3))) void*)(&KB[(wave_u * LPW + x) * 64]))); \
            const uint32_t vl_ = uint32_t(reinterpret_cast<uintptr_t>(                     \
                (__attribute__((address_space(3))) void*)(&VB[(wave_u * LPW + x) * 64]))); \
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"    \
                         :: "v"(ks_), "s"(kl_) : "memory", "m0");                           \
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"    \
                         :: "v"(vs_), "s"(vl_) : "memory", "m0");                           \
        }                                                                                  \
    }
#define LTE_WAIT_COPIES() asm volatile("s_waitcnt vmcnt(0)" ::: "memory")

    // ---- this lane's query row (its loads first: they come from HBM) ---------------
    const int rtile = wave * 32 + (lane & 31);
    const int p_row = rtile / G;
    const int hh = rtile % G;
    const int i_row = i0 + p_row;
    const int irow = i_row <= i_last ? i_row : i_last;
    const int h = g * G + hh;
    bf16x8 qf[KK];
    {
        const uint16_t* qrow = q + ((long(b) * qrows + max(irow - qlo, 0)) * Hq + h) * D;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + kk * 16 + half * 8);
    }
    // ---- prologue: every global load first, then the LDS work ----------------------
    constexpr int NT = NW * 64;
    constexpr int LU = 8;                         // list candidates per thread and pass
    static_assert(LU * NW == 64, "one wave scans the per-(pass slot, wave) counts");
    const int ns = min(s, band_lo);               // sink tokens below the band
    const int thr0 = (band_lo > 0) ? th[i0 - w] : -2;    // list threshold at the first row
    const int thr_last = (band_lo > 0) ? th[i_last - w] : -2;
    // rank of band key band_lo + tid: a band key j can be a retained column of a
    // row of the tile only if j <= i_last - w <= band_lo + P - 2
    int brv = kNotCand;
    if (tid < kBr) {
        const int j = band_lo + tid;
        brv = (j < s) ? -1 : ((j <= band_hi && has_cand) ? rk[j] : kNotCand);   // sink always passes
    }
    // list candidates j = s + u*NT + tid of the first pass (coalesced)
    int rr[LU];
#pragma unroll
    for (int u = 0; u < LU; ++u) {
        const int j = s + u * NT + tid;
        rr[u] = (j < scan_hi) ? rk[j] : kNotCand;
    }

    const int thr_row = (irow - w >= 0) ? th[irow - w] : -2;
    // list entry e is visible to this row iff e <= lim (field <= thr_row + 1)
    const uint32_t lim = (uint32_t(min(max(thr_row + 1, 0), 0xfffe)) << 16) | 0xffffu;
    const float csc = kLog2e * rsqrtf(float(D));
    // the first band block (needs no list), copied behind the rank loads so that the
    // list is built while it is in flight
    LTE_COPY(0, K0, V0)

    if (tid < kBr) brank[tid] = brv;
    // ---- gathered columns below the band: the sink, then the candidates alive at the
    //      tile's first row.  Entries every row of the tile sees (rank within the last
    //      row's threshold) come first, so the blocks they fill need no mask; the at
    //      most P-1 entries that leave the retained set inside the tile follow them.
    //      Ballot compaction (order by pass slot u, then wave, then lane); transient
    //      entries are collected downward from the top of lst and moved after the
    //      stable ones at the end -------------------------------------------------------
    int nblk = nband;                             // the list's blocks join once it is built
    bool listed = false;
    auto build_list = [&]() {
    int len = ns;                                 // sink + stable entries so far
    int ntr = 0;                                  // transient entries so far
    int par = 0;                                  // count buffer of this pass
    for (int j = tid; j < ns; j += NT) lst[j] = uint32_t(j);           // field 0: always visible
    for (int base = s; base < scan_hi; base += LU * NT) {
        if (base != s) {
#pragma unroll
            for (int u = 0; u < LU; ++u) {
                const int j = base + u * NT + tid;
                rr[u] = (j < scan_hi) ? rk[j] : kNotCand;
            }
        }
        uint32_t pre[LU];
#pragma unroll
        for (int u = 0; u < LU; ++u) {
            const bool st = rr[u] <= thr_last;
            const bool tr = !st && rr[u] <= thr0;
            const unsigned long long ms = __ballot(st);
            const unsigned long long mt = __ballot(tr);
            const unsigned long long m = st ? ms : mt;
            pre[u] = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                               __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
            if (lane == 0) wcnt[par][u * NW + wave] = __popcll(ms) | (__popcll(mt) << 16);
        }
        __syncthreads();                          // the pass's counts
        // every wave scans the 64 packed counts itself (each total < 2^13), so no
        // second barrier; the counts alternate between two buffers, so the next
        // pass's writes wait only for its own barrier
        const int c = wcnt[par][lane];
        const int incl = wave_incl_sum(c);
        const int excl = incl - c;
        const int tot = __builtin_amdgcn_readlane(incl, 63);
#pragma unroll
        for (int u = 0; u < LU; ++u) {
            const int off = __builtin_amdgcn_readlane(excl, u * NW + wave);
            const uint32_t ent = (uint32_t(rr[u] + 1) << 16) | uint32_t(base + u * NT + tid);
            if (rr[u] <= thr_last)
                lst[len + (off & 0xffff) + int(pre[u])] = ent;
            else if (rr[u] <= thr0)
                lst[kListTop - (ntr + (off >> 16) + int(pre[u]))] = ent;
        }
        len += tot & 0xffff;
        ntr += tot >> 16;
        par ^= 1;
    }
    __syncthreads();                              // every entry placed
    // transient entries after the stable ones, and the padding to whole blocks with
    // entries no row sees (field 0xffff, key 0), in one pass: the transient entries sit
    // at or above kMaxList + 64 - P, past both (len + ntr <= s + C and ntr < P)
    for (int e = tid; e < ntr; e += NT) lst[len + e] = lst[kListTop - e];
    len += ntr;
    for (int e = len + tid; e < ((len + 63) & ~63); e += NT) lst[e] = 0xffff0000u;
    const int nlist = (len + 63) / 64;
    nblk = nband + nlist;
    __syncthreads();                              // list complete
    // thr is non-increasing, so the tile's last row has the strictest list
    // threshold: a block whose entries all pass it needs no mask
    if (nlist > 0) {
        const uint32_t lim_last = (uint32_t(min(max(thr_last + 1, 0), 0xfffe)) << 16) | 0xffffu;
        for (int bl = wave; bl < nlist; bl += NW) {
            const bool ok = lst[bl * 64 + lane] <= lim_last;
            const bool all = __ballot(ok) == ~0ull;
            if (lane == 0) lfull[bl] = all ? 1 : 0;
        }
    }

        listed = true;
    };
    // with two band blocks or more the list is built after the first block, whose
    // compute hides the rank loads' latency; block 1 is then a band block
    if (nband < 2) build_list();

    float m_run = -INFINITY;
    float l_run = 0.0f;
    f32x16 acc_o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x16{};

    LTE_WAIT_COPIES();
    __syncthreads();                              // block 0, brank (and lfull when listed)

    uint32_t vrd[DT];           // this lane's byte offsets of its V operand pieces
    {
        const int grp = lane >> 4;
        const int i = lane & 15;
        const int key0 = 4 * (grp >> 1) + (i >> 2);
        const int c_lo = 2 * (grp & 1) + ((i & 3) >> 1);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            vrd[dt] = uint32_t(key0 * CPR * 16 + ((4 * dt + c_lo) ^ vswz<D>(key0)) * 16 + 8 * (i & 1));
    }

    // one block: copy the next block into (KN, VN), compute on (KC, VC)
    auto step = [&](const int blk, u32x4* KC, u32x4* VC, u32x4* KN, u32x4* VN) {
        if (blk + 1 < nblk) LTE_COPY(blk + 1, KN, VN)      // in flight during this block
        const bool is_list = blk >= nband;
        const int lb = blk - nband;                        // list block index
        const int jb0 = band_lo + blk * 64;                // first key of a band block

        // ---- S^T = K Q^T for 64 keys x this wave's 32 rows.  Hidden keys enter as
        //      -inf through the first k-step's accumulator, built (only for blocks that
        //      need a mask) before the MFMAs; element e of subtile ks is key slot
        //      ks*32 + (e/4)*8 + half*4 + e%4 of this block --------------------------------
        const bool list_full =
            is_list && __builtin_amdgcn_readfirstlane(lfull[min(lb, kMaxList / 64 - 1)]);
        // d = irow - j: visible iff 0 <= d < w, or d >= w and j passes (sink ranks read
        // -1); band blocks past kBr keys hold no d >= w
        const bool causal_ok = jb0 + 63 <= i0;               // d >= 0 on every row
        const bool in_window = jb0 >= i_last - w + 1;        // d < w on every row
        const bool masked = is_list ? !list_full : !(causal_ok && in_window);
        f32x16 sacc[2];
        {
            bf16x8 a0[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int row = ks * 32 + (lane & 31);
                a0[ks] = __builtin_bit_cast(bf16x8, KC[row * CPR + (half ^ swz<D>(row))]);
            }
            if (masked) {
                f32x16 bias[2];
                bias[0] = f32x16{};
                bias[1] = f32x16{};
                if (is_list) {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                        for (int e4 = 0; e4 < 4; ++e4) {
                            const int t0 = ks * 32 + e4 * 8 + half * 4;
                            const u32x4 ent = *reinterpret_cast<const u32x4*>(&lst[lb * 64 + t0]);
#pragma unroll
                            for (int u = 0; u < 4; ++u)
                                if (!(ent[u] <= lim)) bias[ks][e4 * 4 + u] = -INFINITY;
                        }
                    }
                } else {
                    const int dbase = irow - jb0 - half * 4;
                    if (in_window) {                         // the causal edge only
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                            for (int e = 0; e < 16; ++e) {
                                const int d = dbase - (ks * 32 + (e >> 2) * 8 + (e & 3));
                                if (d < 0) bias[ks][e] = -INFINITY;
                            }
                    } else {                                 // the window edge, maybe both
                        const int rb = min(blk, kBr / 64 - 1) * 64;
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
                                    if (!vis) bias[ks][e4 * 4 + u] = -INFINITY;
                                }
                            }
                        }
                    }
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    sacc[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[ks], qf[0], bias[ks], 0, 0, 0);
            } else {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    sacc[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[ks], qf[0], f32x16{}, 0, 0, 0);
            }
        }
#pragma unroll
        for (int kk = 1; kk < KK; ++kk) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int row = ks * 32 + (lane & 31);
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, KC[row * CPR + ((2 * kk + half) ^ swz<D>(row))]);
                sacc[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[ks], 0, 0, 0);
            }
        }
        // schedule (k-steps 1 .. KK-1): the K operands of the next three k-steps are
        // in flight while this one's MFMAs run
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);
#pragma unroll
        for (int x = 0; x < KK - 4; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 1);

        // ---- online softmax in raw logits, scale folded into the exponent; row =
        //      this lane's query, keys split with lane^32.  p is taken against the
        //      reference m_run; the lane's block sum bounds every p, so the row
        //      maximum is needed only when that sum exceeds 2^8 (a new maximum, or
        //      inf/NaN) or the row has no reference yet.  m_run then moves only when
        //      exceeded by more than 2^8 in the exponent, so p <= 256 and the output
        //      is rarely rescaled; the final division by l_run cancels the choice of
        //      m_run exactly.
        float moff = (m_run == -INFINITY) ? 0.0f : -m_run * csc;
        float pv[32];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 16; ++e) pv[ks * 16 + e] = fast_exp2(fmaf(sacc[ks][e], csc, moff));
        auto tree = [&]() {
            float t[16];
#pragma unroll
            for (int x = 0; x < 16; ++x) t[x] = pv[2 * x] + pv[2 * x + 1];
#pragma unroll
            for (int x = 0; x < 8; ++x) t[x] = t[2 * x] + t[2 * x + 1];
#pragma unroll
            for (int x = 0; x < 4; ++x) t[x] = t[2 * x] + t[2 * x + 1];
            return (t[0] + t[1]) + (t[2] + t[3]);
        };
        float lsum = tree();
        // the fast path needs a finite reference: until a row has seen a visible key
        // its reference is undefined (and p was taken against 0)
        if (__ballot(!(lsum <= 256.0f) || m_run == -INFINITY) != 0ull) {
            float mloc = sacc[0][0];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, sacc[ks][e]);
            const float mrow = max_xor32(mloc);
            // NaN (both -inf: nothing visible yet) compares false: no move
            const bool move = (mrow - m_run) * csc > 8.0f;
            const float m_new = move ? mrow : m_run;
            const float alpha = move ? fast_exp2((m_run - m_new) * csc) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc_o[dt] *= alpha;
            m_run = m_new;
            moff = (m_run == -INFINITY) ? 0.0f : -m_run * csc;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    pv[ks * 16 + e] = fast_exp2(fmaf(sacc[ks][e], csc, moff));
            lsum = tree();
        }
        l_run += lsum;
        bf16x8 pf[4];
#pragma unroll
        for (int x = 0; x < 32; ++x) pf[x >> 3][x & 7] = (__bf16)pv[x];

        // ---- O^T += V^T P^T ------------------------------------------------------
        // operand element e of lane (16-group G, index i) is V[key][dt*32 + (G&1)*16 + i]
        // with key = cc*16 + (e<4 ? 4h + e : 8 + 4h + e-4), h = lane/32: two
        // transposing reads, each of 4 keys, from rows that lane i of the group
        // names, at byte vrd[dt] + (cc*16 + 8r) * row bytes of the tile
        const char* vb = reinterpret_cast<const char*>(VC);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                bf16x8 a;
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    typedef short v4i16 __attribute__((ext_vector_type(4)));
                    const v4i16 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16*)(vb + vrd[dt] +
                                                                   (cc * 16 + 8 * r) * CPR * 16));
                    const bf16x4 b4 = __builtin_bit_cast(bf16x4, t4);
                    a[4 * r + 0] = b4[0];
                    a[4 * r + 1] = b4[1];
                    a[4 * r + 2] = b4[2];
                    a[4 * r + 3] = b4[3];
                }
                acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[cc], acc_o[dt], 0, 0, 0);
            }
        }
        // schedule: four V operands in flight ahead of the MFMA that takes them
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 2);
#pragma unroll
        for (int x = 0; x < 4 * DT - 4; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 2);
        LTE_WAIT_COPIES();                        // this wave's copies of the next block
        __syncthreads();                          // everyone's copies; and the current tiles are free
    };
    step(0, K0, V0, K1, V1);
    if (!listed) build_list();
    for (int blk = 1; blk < nblk; blk += 2) {
        step(blk, K1, V1, K0, V0);
        if (blk + 1 < nblk) step(blk + 1, K0, V0, K1, V1);
    }
#undef LTE_COPY
#undef LTE_WAIT_COPIES

    // ---- normalise, stage the wave's 32 rows as bf16 in LDS (the K/V tiles are free
    //      after the last block's barrier), then store whole rows: the G heads of one
    //      position are G*D contiguous elements of out, so 64 lanes write 1 KB runs
    //      instead of 32 rows x 16 bytes per store.  Element e of d-tile dt is dim
    //      dt*32 + (e/4)*8 + half*4 + e%4; the staged row r holds its 16-byte piece c at
    //      position c ^ (r mod CPR), so the 32 rows of one write spread over the banks.
    const float inv = 1.0f / add_xor32(l_run);
    constexpr int SROW = CPR * 16;                // staged bytes per row
    char* stg = reinterpret_cast<char*>(wave < 2 ? K0 : (wave < 4 ? V0 : (wave < 6 ? K1 : V1))) +
                (wave & 1) * 32 * SROW;
    {
        const int r = lane & 31;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                bf16x4 o4;
#pragma unroll
                for (int u = 0; u < 4; ++u) o4[u] = (__bf16)(acc_o[dt][e4 * 4 + u] * inv);
                *reinterpret_cast<bf16x4*>(stg + r * SROW + (((dt * 4 + e4) ^ (r & (CPR - 1))) * 16) +
                                           half * 8) = o4;
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int x = 0; x < 32 * CPR / 64; ++x) {
        const int c = x * 64 + lane;
        const int rr = c / CPR;                   // staged row: tile row wave*32 + rr
        const int ch = c % CPR;
        const int rt = wave * 32 + rr;
        const int i = i0 + rt / G;
        const u32x4 val = *reinterpret_cast<const u32x4*>(stg + rr * SROW + ((ch ^ (rr & (CPR - 1))) * 16));
        if (i <= i_last && i >= qlo)
            *reinterpret_cast<u32x4*>(out + ((long(b) * qrows + (i - qlo)) * Hq + g * G + rt % G) * D +
                                      ch * 8) = val;
    }
}

template <int D>
hipError_t launch_attend_d(const Shape& sh, int64_t T, const int32_t* seq_lens,
                           const int32_t* q_lo, int q_rows, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const int32_t* rank, const int32_t* thr,
                           const int32_t* ncand, uint16_t* out, hipStream_t st) {
    const int G = sh.G;
    const int P = 256 / G;
    const int ntile = int((T + P - 1) / P);
    dim3 grid(unsigned(long(sh.B) * sh.Hkv * ntile));
#define LTE_ATTEND_CASE(GG)                                                                   \
    case GG:                                                                                  \
        hipLaunchKernelGGL((attend_prefill_kernel<D, GG>), grid, dim3(512), 0, st, int(T),    \
                           sh.Hq, sh.Hkv, sh.s, sh.w, ntile, seq_lens, q_lo, q_rows, q, k, v, \
                           rank, thr, ncand, out);                                           \
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

hipError_t launch_attend_prefill(const Shape& sh, int64_t T, const int32_t* seq_lens,
                                 const int32_t* q_lo, int q_rows, const uint16_t* q,
                                 const uint16_t* k, const uint16_t* v, const int32_t* rank,
                                 const int32_t* thr, const int32_t* ncand, uint16_t* out,
                                 hipStream_t st) {
    if (sh.D == 128)
        return launch_attend_d<128>(sh, T, seq_lens, q_lo, q_rows, q, k, v, rank, thr, ncand, out,
                                    st);
    return launch_attend_d<64>(sh, T, seq_lens, q_lo, q_rows, q, k, v, rank, thr, ncand, out, st);
}

}  // namespace lte
