// Retention scoring CNN over a whole prompt on gfx950.
//
// LTE paper (arXiv 2510.20787) summary page, Figure 2 caption: the
// retention score r_{j,h} of token j in head h comes from a stack of
// convolutions over the keys/values of the few tokens on either side of j.
// Shape used here:
// per KV head, conv1d(2D -> 32, kernel 3, zero pad 1) over concat(k, v),
// GELU, conv1d(32 -> 1, kernel 3, zero pad 1), sigmoid.  x is bf16 (the
// layer's input dtype), W1 is rounded to bf16, accumulation is fp32; the GELU
// (erf by Abramowitz and Stegun 7.1.26, absolute error at most 1.5e-7), the
// 96-term second layer and the sigmoid run in fp32.
//
// Grid: a few workgroups of 8 waves per (batch, KV head), each over a
// contiguous run of 224-token chunks (8 waves x 28 tokens), with the head's W1
// staged in LDS once.  Two workgroups fit a CU (16 waves), which hide each
// other's load latency.  Tokens outside [0, T_b) read as zero (first layer's
// padding) and their hidden activations are zero (second layer's padding);
// T_b is the sequence's length (seq_lens[b], or T for every sequence).  With
// score_lo (per (b, g)), rows below it are not written: they hold scores
// already known.
#include "score_core.h"

namespace lte {
namespace {

// W1 [Hkv][32][2D][3] fp32 -> w1p [Hkv][3][2D/16][64 lanes][8] bf16: the B
// operand of v_mfma_f32_32x32x16_bf16 for output column o = lane % 32 and
// input channels c = 16 kk + 8 (lane / 32) + e.
__global__ void pack_w1_kernel(int Hkv, int D, const float* __restrict__ w1,
                               __bf16* __restrict__ w1p) {
    const int KK = (2 * D) / 16;
    const long total = long(Hkv) * 3 * KK * 64 * 8;
    for (long x = blockIdx.x * long(blockDim.x) + threadIdx.x; x < total;
         x += long(gridDim.x) * blockDim.x) {
        const int e = int(x % 8);
        int tap, kk, lane;
        w1p_coords(int((x / 8) % (3L * KK * 64)), KK, tap, kk, lane);
        const int g = int(x / (8L * 64 * KK * 3));
        const int o = lane % 32;
        const int c = kk * 16 + (lane / 32) * 8 + e;
        w1p[x] = (__bf16)w1[((long(g) * kHidden + o) * (2 * D) + c) * 3 + tap];
    }
}

template <int D>
__global__ __launch_bounds__(64 * kScoreWaves) __attribute__((amdgpu_waves_per_eu(4))) void score_prefill_kernel(
    int T, int Hkv, int nchunk, int nsplit, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ score_lo, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v,
    const bf16x8* __restrict__ w1p, const float* __restrict__ b1, const float* __restrict__ w2,
    const float* __restrict__ b2, float* __restrict__ scores) {
    constexpr int NW = ScoreSmem<D>::NW;
    __shared__ bf16x8 wl[NW];
    __shared__ float w2s[kHidden * 3];
    __shared__ float act[kScoreWaves][kActRows * kActPitch];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int bg = blockIdx.x / nsplit;
    const int part = blockIdx.x % nsplit;
    const int b = bg / Hkv;
    const int g = bg % Hkv;
    const int Tb = seq_len_of(seq_lens, b, T);
    const int lo = score_lo ? score_lo[bg] : 0;              // rows below keep their scores
    // this workgroup's chunks, without those wholly past T_b or below lo
    const int per = (nchunk + nsplit - 1) / nsplit;
    const int c_begin = max(part * per, lo / kChunkTokens);
    const int c_end = min(min(nchunk, (part + 1) * per), (Tb + kChunkTokens - 1) / kChunkTokens);
    if (c_begin >= c_end) return;

    const long row_stride = long(Hkv) * D;
    const uint16_t* kb = k + (long(b) * T * Hkv + g) * D;
    const uint16_t* vb = v + (long(b) * T * Hkv + g) * D;
    // this lane's row of the first pass: its first operand half loads while W1 is staged
    int tok = c_begin * kChunkTokens + wave * kPassTokens - 2 + (lane & 31);
    bf16x8 a0[ScoreSmem<D>::KK / 2];
    score_load_half<D>(a0, kb + long(tok) * row_stride, vb + long(tok) * row_stride,
                       tok >= 0 && tok < Tb, 0);

    const bf16x8* wsrc = w1p + long(g) * NW;
    for (int x = tid; x < NW; x += 64 * kScoreWaves) wl[x] = wsrc[x];
    for (int x = tid; x < kHidden * 3; x += 64 * kScoreWaves) w2s[x] = w2[g * kHidden * 3 + x];
    const float b1o = b1[g * kHidden + (lane & 31)];
    const float b2g = b2[g];

    float* out = scores + long(bg) * T;
    __syncthreads();                                         // W1 and W2 staged
    float* my_act = act[wave];
    for (int c = c_begin; c < c_end; ++c, tok += kChunkTokens) {
        const int t0 = c * kChunkTokens + wave * kPassTokens;
        const int ntok = tok + kChunkTokens;                 // the same row of the next pass
        score_pass<D>(
            wl, w2s, b1o, b2g, a0, kb + long(tok) * row_stride, vb + long(tok) * row_stride,
            tok >= 0 && tok < Tb, kb + long(ntok) * row_stride, vb + long(ntok) * row_stride,
            c + 1 < c_end && ntok < Tb, my_act, t0, 0, Tb - 1,
            [&](int x) { return x < 0 || x >= Tb; },
            [&](int t, float r) { if (t >= lo) out[t] = r; });
    }
}

}  // namespace

hipError_t launch_pack_w1(const Shape& sh, const float* w1, uint16_t* w1p, hipStream_t st) {
    long total = long(sh.Hkv) * 3 * (2 * sh.D / 16) * 64 * 8;
    int blocks = int((total + 255) / 256);
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(pack_w1_kernel, dim3(blocks), dim3(256), 0, st, sh.Hkv, sh.D, w1,
                       reinterpret_cast<__bf16*>(w1p));
    return hipGetLastError();
}

hipError_t launch_score_prefill(const Shape& sh, int64_t T, const int32_t* seq_lens,
                                const int32_t* score_lo, const uint16_t* k, const uint16_t* v,
                                const uint16_t* w1p, const lte_cnn& cnn, float* scores,
                                hipStream_t st) {
    // about two workgroups per CU over the whole grid (256 CUs), each (b, g)
    // split into nsplit runs of chunks
    const int nchunk = int((T + kChunkTokens - 1) / kChunkTokens);
    const long bgs = long(sh.B) * sh.Hkv;
    long nsplit = (512 + bgs - 1) / bgs;
    if (nsplit > nchunk) nsplit = nchunk;
    if (nsplit < 1) nsplit = 1;
    dim3 grid(unsigned(bgs * nsplit));
    const bf16x8* wp = reinterpret_cast<const bf16x8*>(w1p);
    if (sh.D == 128) {
        hipLaunchKernelGGL(score_prefill_kernel<128>, grid, dim3(64 * kScoreWaves), 0, st, int(T), sh.Hkv,
                           nchunk, int(nsplit), seq_lens, score_lo, k, v, wp, cnn.b1, cnn.w2,
                           cnn.b2, scores);
    } else {
        hipLaunchKernelGGL(score_prefill_kernel<64>, grid, dim3(64 * kScoreWaves), 0, st, int(T), sh.Hkv,
                           nchunk, int(nsplit), seq_lens, score_lo, k, v, wp, cnn.b1, cnn.w2,
                           cnn.b2, scores);
    }
    return hipGetLastError();
}

}  // namespace lte
