// KV-cache construction after a prefill, and cache reset.
//
// LTE paper (arXiv 2510.20787) summary page, Figure 3 caption: the inference
// cache is a circular segment for the in-window KVs plus an out-of-window
// segment of capped capacity holding the LTE-retained KVs and the attention
// sink.  "Sparse Linear Attention: Viewing SWA from the Perspective of Linear
// Attention", section "Viewing SWA from the linear-state perspective": the
// window is a FIFO of slots, one slot overwritten per token -- token j lives
// in ring slot j mod w.
//
// After a T-token prompt the cache holds: the sink tokens [0, min(s, T)), the
// retained set R_{T-1} compacted in token order, the last min(w, T) tokens in
// the ring, the scores of ring tokens whose right neighbours exist (j <= T-3),
// pos = T and next_unscored = max(T-2, s).
//
// After a chunked prefill the rows are those of the extended sequence (see
// chunk.hip) and the kernels map them to tokens: row e is token e, or, past
// the sink of a cache that had lost tokens from its window, the segment's
// sorted token e - s (rows [s, s + C)) or token e + off (later rows).
#include "lte_internal.h"

namespace lte {
namespace {

__global__ void cache_init_kernel(int BG, int w, int s, CacheView c) {
    const long n = long(BG) * w;
    const float qnan = __builtin_nanf("");
    for (long x = blockIdx.x * long(blockDim.x) + threadIdx.x; x < n;
         x += long(gridDim.x) * blockDim.x)
        c.ring_score[x] = qnan;
    for (long x = blockIdx.x * long(blockDim.x) + threadIdx.x; x < BG;
         x += long(gridDim.x) * blockDim.x) {
        c.count[x] = 0;
        c.pos[x] = 0;
        c.next_unscored[x] = s;
        c.flags[x] = 0;
        c.weak[x] = -1;
        c.nx_slot[x] = -1;
        c.nx_score[x] = 0.0f;
        c.arrive[x] = 0;
    }
}

// One workgroup (256 threads) per (batch, KV head): bookkeeping of the cache.
__global__ __launch_bounds__(256) void cache_meta_kernel(int Tmax, int Hkv, int s, int w, int C,
                                                         const int32_t* __restrict__ seq_lens,
                                                         ChunkView xv,
                                                         const float* __restrict__ scores,
                                                         const int32_t* __restrict__ rank,
                                                         const int32_t* __restrict__ thr,
                                                         CacheView c) {
    __shared__ int wsum[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int bg = blockIdx.x;
    const int b = bg / Hkv;
    const int T = seq_len_of(seq_lens, b, Tmax);            // rows of this sequence
    const float* r = scores + long(bg) * Tmax;
    const int32_t* rk = rank + long(bg) * Tmax;
    const float qnan = __builtin_nanf("");
    // row -> token map of a chunked prefill (identity otherwise)
    const bool warm = xv.warm != nullptr && xv.warm[b] != 0;
    const int off = warm ? xv.tok_off[b] : 0;
    const int Tn = T + off;                                  // tokens of the sequence
    auto tok = [&](int e) {
        if (!warm || e < s) return e;
        if (e < s + C) return int(xv.seg_tok[long(bg) * C + (e - s)]);
        return e + off;
    };

    // ring scores: the ring's tokens are the last w rows
    for (int slot = tid; slot < w; slot += 256) {
        const int j = Tn - 1 - ((Tn - 1 - slot) % w + w) % w;   // newest token in this slot
        float sc = qnan;
        if (j >= 0 && j >= s && j <= Tn - 3) sc = r[j - off];
        c.ring_score[long(bg) * w + slot] = sc;
    }

    // R_{T-1}: tokens j <= T-1-w with rank[j] <= thr[T-1-w], in token order
    const int m = T - 1 - w;
    int len = 0;
    if (m >= 0 && C > 0) {
        const int th = thr[long(bg) * Tmax + m];
        for (int base = s; base <= m; base += 256 * 8) {
            int cnt = 0;
            int ent[8];
            const int j0 = base + tid * 8;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                if (j <= m && rk[j] <= th) ent[cnt++] = j;
            }
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
            const int o = len + woff + incl - cnt;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (u < cnt) {
                    c.ret_idx[long(bg) * C + o + u] = tok(ent[u]);
                    c.ret_score[long(bg) * C + o + u] = r[ent[u]];
                    if (xv.seg_row != nullptr) xv.seg_row[long(bg) * C + o + u] = ent[u];
                }
            }
            len += tot;
            __syncthreads();
        }
    }
    // weakest entry of a full segment: lowest score, then highest token index
    int wx = -1;
    if (C > 0 && len == C) {
        __threadfence_block();
        __syncthreads();
        float bs = INFINITY;
        int bt = -1;
        for (int x = tid; x < C; x += 256) {
            const float sc = c.ret_score[long(bg) * C + x];
            const int tk = c.ret_idx[long(bg) * C + x];
            if (sc < bs || (sc == bs && tk > bt)) { bs = sc; bt = tk; wx = x; }
        }
        __shared__ float rs[4];
        __shared__ int rt[4], rx[4];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const float os = __shfl_xor(bs, d, 64);
            const int ot = __shfl_xor(bt, d, 64);
            const int ox = __shfl_xor(wx, d, 64);
            if (os < bs || (os == bs && ot > bt)) { bs = os; bt = ot; wx = ox; }
        }
        if (lane == 0) { rs[wave] = bs; rt[wave] = bt; rx[wave] = wx; }
        __syncthreads();
        bs = rs[0]; bt = rt[0]; wx = rx[0];
        for (int q = 1; q < 4; ++q) {
            if (rs[q] < bs || (rs[q] == bs && rt[q] > bt)) { bs = rs[q]; bt = rt[q]; wx = rx[q]; }
        }
    }
    if (tid == 0) {
        c.count[bg] = len;
        c.pos[bg] = Tn;
        c.next_unscored[bg] = max(Tn - 2, s);
        c.flags[bg] = 0;
        c.weak[bg] = wx;
        // decision for the token Tn-w that leaves at the first decode step (its
        // score is final: its right neighbours Tn-w+1, Tn-w+2 exist)
        int nx = -1;
        float rl = 0.0f;
        const int jl = Tn - w;
        if (jl >= s) {
            rl = r[jl - off];
            if (rl > 0.5f && C > 0) {
                if (len < C) nx = len;
                else if (wx >= 0 && rl > c.ret_score[long(bg) * C + wx]) nx = wx;
            }
        }
        c.nx_slot[bg] = nx;
        c.nx_score[bg] = rl;
        c.arrive[bg] = 0;
    }
}

// Copies K/V rows into the cache slots: sink, retained segment, ring.
// Work items are (batch, KV head) x slot groups, one 16-byte chunk per thread;
// the grid walks them with a stride (one item per workgroup when the grid
// covers them all).
__global__ __launch_bounds__(256) void cache_copy_kernel(int Tmax, int Hkv, int D, int s, int w,
                                                         int C, int S, int slots_per_block, int nblk,
                                                         const int32_t* __restrict__ seq_lens,
                                                         ChunkView xv,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         CacheView c) {
    const int nsb = (S + slots_per_block - 1) / slots_per_block;
    for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int bg = blk / nsb;
        const int sb = blk % nsb;
        const int b = bg / Hkv;
        const int g = bg % Hkv;
        const int T = seq_len_of(seq_lens, b, Tmax);            // rows of this sequence
        const bool warm = xv.warm != nullptr && xv.warm[b] != 0;
        const int off = warm ? xv.tok_off[b] : 0;
        const int Tn = T + off;                                  // tokens of the sequence
        const int chunks = D / 8;
        const int cnt = c.count[bg];
        for (int x = threadIdx.x; x < slots_per_block * chunks; x += blockDim.x) {
            const int slot = sb * slots_per_block + x / chunks;
            const int ch = x % chunks;
            if (slot >= S) continue;
            int j = -1;                                      // source row
            if (slot < s) {
                if (slot < T) j = slot;
            } else if (slot < s + C) {
                if (slot - s < cnt)
                    j = xv.seg_row != nullptr ? xv.seg_row[long(bg) * C + (slot - s)]
                                              : c.ret_idx[long(bg) * C + (slot - s)];
            } else {
                const int rs = slot - s - C;
                const int jj = Tn - 1 - ((Tn - 1 - rs) % w + w) % w;   // token
                if (jj >= 0) j = jj - off;
            }
            if (j < 0) continue;
            const long src = ((long(b) * Tmax + j) * Hkv + g) * D + ch * 8;
            const long dst = (long(bg) * S + slot) * D + ch * 8;
            *reinterpret_cast<uint4*>(c.k + dst) = *reinterpret_cast<const uint4*>(k + src);
            *reinterpret_cast<uint4*>(c.v + dst) = *reinterpret_cast<const uint4*>(v + src);
        }
    }
}

}  // namespace

hipError_t launch_cache_init(const Shape& sh, const CacheView& cache, hipStream_t st) {
    const long n = long(sh.B) * sh.Hkv * sh.w;
    int blocks = int((n + 255) / 256);
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(cache_init_kernel, dim3(blocks), dim3(256), 0, st, sh.B * sh.Hkv, sh.w,
                       sh.s, cache);
    return hipGetLastError();
}

hipError_t launch_build_cache(const Shape& sh, int64_t T, const int32_t* seq_lens,
                              const ChunkView* chunk, const uint16_t* k, const uint16_t* v,
                              const float* scores, const int32_t* rank, const int32_t* thr,
                              const CacheView& cache, hipStream_t st, int copy_wgs) {
    const int BG = sh.B * sh.Hkv;
    const ChunkView x = chunk ? *chunk : ChunkView{};
    hipLaunchKernelGGL(cache_meta_kernel, dim3(BG), dim3(256), 0, st, int(T), sh.Hkv, sh.s, sh.w,
                       sh.C, seq_lens, x, scores, rank, thr, cache);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int spb = 32;                                  // slots per workgroup
    const int nsb = (sh.S + spb - 1) / spb;
    const int nblk = BG * nsb;
    const int grid = (copy_wgs > 0 && copy_wgs < nblk) ? copy_wgs : nblk;
    hipLaunchKernelGGL(cache_copy_kernel, dim3(unsigned(grid)), dim3(256), 0, st,
                       int(T), sh.Hkv, sh.D, sh.s, sh.w, sh.C, sh.S, spb, nblk, seq_lens, x, k, v,
                       cache);
    return hipGetLastError();
}

}  // namespace lte
