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
// Grid: about one workgroup of 8 waves per CU, a few per (batch, KV head),
// each over an even share of the head's tokens in 224-token chunks (8 waves x
// 28 tokens), with
// the head's W1 converted to bf16 and staged in LDS once.  Every wave holds the
// next pass's rows in registers while it computes the current one.  Tokens outside [0, T_b) read as zero (first layer's
// padding) and their hidden activations are zero (second layer's padding);
// T_b is the sequence's length (seq_lens[b], or T for every sequence).  With
// score_lo (per (b, g)), rows below it are not written: they hold scores
// already known.
#include "score_core.h"

namespace lte {
namespace {

// One wave's pass over 32 rows (tokens t0-2 .. t0+29), scoring tokens [t0, t0+28)
// clipped to [tlo, thi]: layer 1 on v_mfma_f32_32x32x16_bf16 from the operands a
// (all 2D channels of the lane's row, loaded a pass ahead), the hidden activations
// through the wave's LDS tile, layer 2 and the sigmoid for lanes < 28, whose
// result (token t, score r) is returned for the caller to store.
//   wl, w2s  this head's packed W1 and W2 [32][3] in LDS; b1o: b1 of column lane % 32
//   act      wave-private LDS tile [kActRows][kActPitch]
//   a_zero(x) -> true where layer 2 sees zero padding (outside the sequence)
// The accumulator element e of lane l holds row 8 (e/4) + 4 (l/32) + e%4 and
// output column l % 32, so a row's neighbours are in the same lane except
// across groups of 4 rows, where they sit in lane l ^ 32.
template <int D, class AZero>
__device__ __forceinline__ bool score_rows(const bf16x8* wl, const float* w2s, float b1o,
                                           float b2g, const bf16x8 (&a)[ScoreSmem<D>::KK],
                                           float* act, int t0, int tlo, int thi, AZero a_zero,
                                           int& t_out, float& r_out) {
    constexpr int KK = ScoreSmem<D>::KK;
    const int lane = threadIdx.x & 63;
    const bool hi = (lane & 32) != 0;
    f32x16 acc[3];
#pragma unroll
    for (int tp = 0; tp < 3; ++tp) acc[tp] = f32x16{};
#pragma unroll
    for (int q = 0; q < KK; ++q) {
#pragma unroll
        for (int tp = 0; tp < 3; ++tp) {
            const bf16x8 bfrag = wl[(tp * KK + q) * 64 + lane];
            acc[tp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[q], bfrag, acc[tp], 0, 0, 0);
        }
    }
    // tap 0 of row-1 and tap 2 of row+1 where they sit in the other lane half
    float p0[4], p2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p0[i] = other_half(acc[0][4 * i + 3]);
        p2[i] = other_half(acc[2][4 * i]);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int i = e >> 2;
        const int j = e & 3;
        const int row = 8 * i + (hi ? 4 : 0) + j;
        // rows 0 and 31 (the outer halo) take no neighbour: they feed no score
        const float y0 = (j > 0) ? acc[0][e - 1] : (hi ? p0[i] : (i > 0 ? p0[i - 1] : 0.0f));
        const float y2 = (j < 3) ? acc[2][e + 1] : (hi ? (i < 3 ? p2[i + 1] : 0.0f) : p2[i]);
        const float h = b1o + y0 + acc[1][e] + y2;
        if (row >= 1 && row <= kActRows)
            act[(row - 1) * kActPitch + (lane & 31)] = a_zero(t0 - 2 + row) ? 0.0f : gelu_erf(h);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // output layer + sigmoid for tokens t0 .. t0+27 (rows 2 .. 29)
    bool has = false;
    if (lane < kPassTokens) {
        const int t = t0 + lane;
        if (t >= tlo && t <= thi) {
            float z = b2g;
            const int r = lane + 1;                          // act row of token t
#pragma unroll 8
            for (int o = 0; o < kHidden; ++o) {
                z += w2s[o * 3 + 0] * act[(r - 1) * kActPitch + o] +
                     w2s[o * 3 + 1] * act[r * kActPitch + o] +
                     w2s[o * 3 + 2] * act[(r + 1) * kActPitch + o];
            }
            t_out = t;
            r_out = 1.0f / (1.0f + expf(-z));
            has = true;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return has;
}

// The layer-1 A operands of the lane's row: channels 16 kk + 8 (lane/32) .. +8 of
// concat(k, v) of the row at kp, vp (zeros where !ok).
template <int D>
__device__ __forceinline__ void score_load_row(bf16x8 (&a)[ScoreSmem<D>::KK], const uint16_t* kp,
                                               const uint16_t* vp, bool ok) {
    constexpr int KK = ScoreSmem<D>::KK;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < KK; ++q) {
        const int ch = q * 16 + (lane >> 5) * 8;
        a[q] = ok ? *reinterpret_cast<const bf16x8*>((ch < D) ? (kp + ch) : (vp + (ch - D)))
                  : bf16x8{};
    }
}

// One workgroup (8 waves, one per SIMD pair) per compute unit scores an even share
// of one (batch, KV head)'s tokens in 224-token chunks: each wave takes 28 tokens of a
// chunk per pass.  A pass's rows are loaded during the pass before it, into the
// second of two register sets, so every wave keeps a whole pass of loads in flight
// while it computes; the score of a pass is stored at the start of the next one,
// after its wait, so that the wait never covers a store.
template <int D>
__global__ __launch_bounds__(64 * kScoreWaves) __attribute__((amdgpu_waves_per_eu(2))) void score_prefill_kernel(
    int T, int Hkv, int nsplit, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ score_lo, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v,
    const float* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    const float* __restrict__ b2, float* __restrict__ scores) {
    constexpr int NW = ScoreSmem<D>::NW;
    constexpr int KK = ScoreSmem<D>::KK;
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
    // this workgroup's tokens: an even share of the head's T rows, without those past
    // T_b or below lo, in 224-token chunks from its first token
    const int per = (T + nsplit - 1) / nsplit;
    const int t_begin = max(part * per, lo);
    const int t_end = min((part + 1) * per, Tb);
    if (t_begin >= t_end) return;
    const int c_begin = 0;
    const int c_end = (t_end - t_begin + kChunkTokens - 1) / kChunkTokens;

    const long row_stride = long(Hkv) * D;
    const uint16_t* kb = k + (long(b) * T * Hkv + g) * D;
    const uint16_t* vb = v + (long(b) * T * Hkv + g) * D;
    // this lane's row of chunk c: token c * 224 + wave * 28 - 2 + lane % 32
    const int tok0 = wave * kPassTokens - 2 + (lane & 31);
    auto load = [&](bf16x8 (&a)[KK], int c) {
        const int tok = t_begin + c * kChunkTokens + tok0;
        // rows past t_end + 1 feed no score of this range: read as zero, no traffic
        score_load_row<D>(a, kb + long(tok) * row_stride, vb + long(tok) * row_stride,
                          tok >= 0 && tok < min(Tb, t_end + 2));
    };
    bf16x8 aA[KK], aB[KK];
    load(aA, c_begin);                                       // lands while W1 is staged

    // this head's W1 [32][2D][3] as the MFMA B operands: entry (tap, kk, lane) holds
    // W1[o = lane % 32][c = 16 kk + 8 (lane / 32) + e][tap], e < 8, in bf16; the 8
    // channels of one (kk, lane) are 24 consecutive floats over the three taps
    {
        const float* w1g = w1 + long(g) * kHidden * 2 * D * 3;
        const bool al16 = (reinterpret_cast<uintptr_t>(w1g) & 15) == 0;
        for (int x = tid; x < KK * 64; x += 64 * kScoreWaves) {
            const int kk = x / 64;
            const int ln = x % 64;
            const float* src = w1g + (long(ln % 32) * 2 * D + 16 * kk + 8 * (ln / 32)) * 3;
            float f[24];
            if (al16) {
#pragma unroll
                for (int u = 0; u < 6; ++u) {
                    const float4 t4 = *reinterpret_cast<const float4*>(src + 4 * u);
                    f[4 * u] = t4.x;
                    f[4 * u + 1] = t4.y;
                    f[4 * u + 2] = t4.z;
                    f[4 * u + 3] = t4.w;
                }
            } else {
#pragma unroll
                for (int u = 0; u < 24; ++u) f[u] = src[u];
            }
#pragma unroll
            for (int tp = 0; tp < 3; ++tp) {
                bf16x8 e8;
#pragma unroll
                for (int e = 0; e < 8; ++e) e8[e] = (__bf16)f[3 * e + tp];
                wl[(tp * KK + kk) * 64 + ln] = e8;
            }
        }
    }
    for (int x = tid; x < kHidden * 3; x += 64 * kScoreWaves) w2s[x] = w2[g * kHidden * 3 + x];
    const float b1o = b1[g * kHidden + (lane & 31)];
    const float b2g = b2[g];

    float* out = scores + long(bg) * T;
    __syncthreads();                                         // W1 and W2 staged
    float* my_act = act[wave];
    bool pend = false;                                       // a score not yet stored
    int pt = 0;
    float pr = 0.0f;
    auto pass = [&](int c, const bf16x8 (&a)[KK], bf16x8 (&an)[KK]) {
        __builtin_amdgcn_s_waitcnt(0);                       // a has landed
        __builtin_amdgcn_sched_barrier(0);
        if (pend) out[pt] = pr;
        if (c + 1 < c_end) load(an, c + 1);
        __builtin_amdgcn_sched_barrier(0);
        pend = score_rows<D>(wl, w2s, b1o, b2g, a, my_act, t_begin + c * kChunkTokens + wave * kPassTokens,
                             t_begin, t_end - 1, [&](int x) { return x < 0 || x >= Tb; }, pt, pr);
    };
    for (int c = c_begin; c < c_end; c += 2) {
        pass(c, aA, aB);
        if (c + 1 >= c_end) break;
        pass(c + 1, aB, aA);
    }
    if (pend) out[pt] = pr;
}

}  // namespace

hipError_t launch_score_prefill(const Shape& sh, int64_t T, const int32_t* seq_lens,
                                const int32_t* score_lo, const uint16_t* k, const uint16_t* v,
                                const lte_cnn& cnn, float* scores, hipStream_t st) {
    // about one workgroup per CU over the whole grid (256 CUs), each (b, g)
    // split into nsplit even token ranges
    const int nchunk = int((T + kChunkTokens - 1) / kChunkTokens);
    const long bgs = long(sh.B) * sh.Hkv;
    long nsplit = (256 + bgs - 1) / bgs;
    if (nsplit > nchunk) nsplit = nchunk;
    if (nsplit < 1) nsplit = 1;
    dim3 grid(unsigned(bgs * nsplit));
    if (sh.D == 128) {
        hipLaunchKernelGGL(score_prefill_kernel<128>, grid, dim3(64 * kScoreWaves), 0, st, int(T), sh.Hkv,
                           int(nsplit), seq_lens, score_lo, k, v, cnn.w1, cnn.b1, cnn.w2,
                           cnn.b2, scores);
    } else {
        hipLaunchKernelGGL(score_prefill_kernel<64>, grid, dim3(64 * kScoreWaves), 0, st, int(T), sh.Hkv,
                           int(nsplit), seq_lens, score_lo, k, v, cnn.w1, cnn.b1, cnn.w2,
                           cnn.b2, scores);
    }
    return hipGetLastError();
}

}  // namespace lte
