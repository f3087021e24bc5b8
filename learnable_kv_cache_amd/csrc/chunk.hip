// Chunked prefill onto an existing cache: lays the cache and a chunk of n new
// tokens out as one extended sequence that the prefill kernels then process.
//
// LTE paper (arXiv 2510.20787) summary page, Figure 2 caption: a token's
// eviction is decided when it leaves the window, from its score alone, and
// at most C tokens are kept, so the retained set after a prefix is the top-C
// of that prefix's candidates; under the strict order (score desc, index asc)
// top-C of a union equals top-C of (top-C of one part) U (the other part).
// The cache's segment already is the top-C of every token that left the
// window before the chunk, so the chunk continues exactly from it.
//
// Extended layout of one (batch, KV head), E rows:
//   * the cache still holds the whole history (pos < s + w: no token past
//     the sink has left the window): rows [0, pos) are tokens 0..pos-1 (sink
//     slots, ring slots), rows [pos, pos + n) the chunk; token = row;
//   * otherwise: rows [0, s) the sink, rows [s, s + C) the segment sorted by
//     token (count valid rows, then empty rows that are never candidates),
//     rows [s + C, s + C + w) the ring's tokens pos-w .. pos-1 in order, then
//     the chunk; token = row + off with off = pos - w - s - C past the
//     segment.
// In both layouts the ring and the chunk are contiguous and in token order,
// so a chunk query's window is its last w rows, the sink is rows [0, s), and
// the candidates order by (score, row) as by (score, token).
#include "lte_internal.h"

namespace lte {
namespace {

constexpr int kSortMax = kMaxCapacity;     // segment entries sorted in LDS

// One workgroup per (batch, KV head): per-sequence layout data, the segment
// sorted by token, and the extended rows' known scores.
__global__ __launch_bounds__(256) void chunk_meta_kernel(int Hkv, int s, int w, int C, int n,
                                                         CacheView c, ChunkView x,
                                                         float* __restrict__ ext_scores,
                                                         int Emax) {
    __shared__ unsigned long long key[kSortMax];
    const int bg = blockIdx.x;
    const int b = bg / Hkv;
    const int tid = threadIdx.x;
    const int P = int(c.pos[bg]);
    const int u = int(c.next_unscored[bg]);
    const bool warm = P >= s + w;
    const int off = warm ? P - w - s - C : 0;
    float* sc = ext_scores + long(bg) * Emax;
    if (tid == 0) {
        x.score_lo[bg] = warm ? u - off : u;
        if (bg % Hkv == 0) {
            x.ext_len[b] = warm ? s + C + w + n : P + n;
            x.q_lo[b] = warm ? s + C + w : P;
            x.tok_off[b] = off;
            x.warm[b] = warm ? 1 : 0;
        }
    }
    const float* rs = c.ring_score + long(bg) * w;
    if (!warm) {
        for (int e = tid; e < P; e += 256) sc[e] = (e < s) ? 0.0f : rs[e % w];
        return;
    }
    for (int e = tid; e < s; e += 256) sc[e] = 0.0f;
    for (int i = tid; i < w; i += 256) {
        const int j = P - w + i;                         // ring token
        sc[s + C + i] = rs[j % w];
    }
    // segment: bitonic sort of (token, slot) over the next power of two
    const int cnt = c.count[bg];
    int N = 1;
    while (N < cnt) N <<= 1;
    const int32_t* ri = c.ret_idx + long(bg) * C;
    for (int e = tid; e < N; e += 256)
        key[e] = (e < cnt) ? ((unsigned long long)(unsigned(ri[e])) << 32) | unsigned(e)
                           : ~0ull;
    __syncthreads();
    for (int k = 2; k <= N; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int e = tid; e < N; e += 256) {
                const int p = e ^ j;
                if (p > e) {
                    const bool up = (e & k) == 0;
                    const unsigned long long a = key[e], bb = key[p];
                    if ((a > bb) == up) {
                        key[e] = bb;
                        key[p] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    const float* rsc = c.ret_score + long(bg) * C;
    for (int r = tid; r < C; r += 256) {
        if (r < cnt) {
            const int slot = int(key[r] & 0xffffffffu);
            x.seg_tok[long(bg) * C + r] = int(key[r] >> 32);
            x.seg_slot[long(bg) * C + r] = slot;
            sc[s + r] = rsc[slot];
        } else {
            x.seg_slot[long(bg) * C + r] = -1;
            sc[s + r] = 0.0f;                            // empty row: never a candidate
        }
    }
}

// Extended K/V rows: grid.x = (batch, KV head) x groups of 32 rows; one 16-byte
// chunk per thread and pass.
__global__ __launch_bounds__(256) void chunk_rows_kernel(int Hkv, int D, int s, int w, int C,
                                                         int S, int n, int Emax, int ngroups,
                                                         const uint16_t* __restrict__ kc,
                                                         const uint16_t* __restrict__ vc,
                                                         CacheView c, ChunkView x,
                                                         uint16_t* __restrict__ ek,
                                                         uint16_t* __restrict__ ev) {
    const int bg = blockIdx.x / ngroups;
    const int grp = blockIdx.x % ngroups;
    const int b = bg / Hkv;
    const int g = bg % Hkv;
    const int P = int(c.pos[bg]);
    const bool warm = x.warm[b] != 0;
    const int E = x.ext_len[b];
    const int chunks = D / 8;
    for (int t = threadIdx.x; t < 32 * chunks; t += 256) {
        const int e = grp * 32 + t / chunks;
        const int ch = t % chunks;
        if (e >= E) continue;
        const uint16_t* sk = nullptr;                    // source row
        const uint16_t* sv = nullptr;
        int slot = -1;
        int crow = -1;
        if (!warm) {
            if (e < P) slot = (e < s) ? e : s + C + e % w;
            else crow = e - P;
        } else if (e < s) {
            slot = e;
        } else if (e < s + C) {
            const int r = x.seg_slot[long(bg) * C + (e - s)];
            if (r >= 0) slot = s + r;
        } else if (e < s + C + w) {
            const int j = P - w + (e - s - C);
            slot = s + C + j % w;
        } else {
            crow = e - (s + C + w);
        }
        if (slot >= 0) {
            sk = c.k + (long(bg) * S + slot) * D;
            sv = c.v + (long(bg) * S + slot) * D;
        } else if (crow >= 0) {
            sk = kc + ((long(b) * n + crow) * Hkv + g) * D;
            sv = vc + ((long(b) * n + crow) * Hkv + g) * D;
        }
        const long dst = ((long(b) * Emax + e) * Hkv + g) * D + ch * 8;
        uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
        if (sk != nullptr) {
            kv = *reinterpret_cast<const uint4*>(sk + ch * 8);
            vv = *reinterpret_cast<const uint4*>(sv + ch * 8);
        }
        *reinterpret_cast<uint4*>(ek + dst) = kv;
        *reinterpret_cast<uint4*>(ev + dst) = vv;
    }
}

}  // namespace

hipError_t launch_chunk_gather(const Shape& sh, int n, int Emax, const uint16_t* k,
                               const uint16_t* v, const CacheView& cache, const ChunkView& x,
                               float* ext_scores, uint16_t* ek, uint16_t* ev, hipStream_t st) {
    const int BG = sh.B * sh.Hkv;
    hipLaunchKernelGGL(chunk_meta_kernel, dim3(BG), dim3(256), 0, st, sh.Hkv, sh.s, sh.w, sh.C, n,
                       cache, x, ext_scores, Emax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ngroups = (Emax + 31) / 32;
    hipLaunchKernelGGL(chunk_rows_kernel, dim3(unsigned(long(BG) * ngroups)), dim3(256), 0, st,
                       sh.Hkv, sh.D, sh.s, sh.w, sh.C, sh.S, n, Emax, ngroups, k, v, cache, x,
                       ek, ev);
    return hipGetLastError();
}

}  // namespace lte
