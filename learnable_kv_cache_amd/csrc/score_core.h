// Body of the retention-scoring CNN, shared by the prefill scorer (tokens read
// from the k/v prompt tensors) and the deferred batched scorer of the decode
// path (tokens read from the cache's ring slots).
//
// LTE paper (arXiv 2510.20787) summary page, Figure 2 caption: a CNN reads the
// keys/values of past and future neighbours and emits r_{j,h}; the score of a
// token is computable once its receptive field (tokens j-2 .. j+2 for two
// kernel-3 layers) is present.
//
// The prefill scorer (one wave per 28 tokens, W1 staged once per workgroup in
// LDS) builds on the constants and helpers here; score_wave: one wave scores 28
// tokens (decode), W1 read from global memory.
// Layer 1 is written as Y_tap = W1[:, :, tap] . x per token
// (v_mfma_f32_32x32x16_bf16, 32 tokens x 96 outputs per wave), then
// h[j] = b1 + Y_0[j-1] + Y_1[j] + Y_2[j+1].
#pragma once

#include "lte_internal.h"

namespace lte {

constexpr int kPassTokens = 28;      // tokens one wave scores per pass (32 rows with halos)
constexpr int kScoreWaves = 8;       // waves of a prefill scoring workgroup
constexpr int kChunkTokens = kScoreWaves * kPassTokens;   // per prefill workgroup pass
constexpr int kActPitch = 33;        // floats per activation row in LDS (bank spread)
constexpr int kActRows = 30;         // rows 1 .. 30 of a pass feed its scores

template <int D>
struct ScoreSmem {
    static constexpr int KK = (2 * D) / 16;          // MFMA k-steps over the 2D channels
    static constexpr int NW = 3 * KK * 64;           // bf16x8 entries of one head's packed W1
};

// erf by Abramowitz and Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: for x >= 0, erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5)
// exp(-x^2) with t = 1 / (1 + p x), absolute error at most 1.5e-7; erf is odd.
// Branch-free: one reciprocal, one exponential, five FMAs.
constexpr float kErfP = 0.3275911f;
constexpr float kErfA1 = 0.254829592f;
constexpr float kErfA2 = -0.284496736f;
constexpr float kErfA3 = 1.421413741f;
constexpr float kErfA4 = -1.453152027f;
constexpr float kErfA5 = 1.061405429f;
__device__ __forceinline__ float erf_as(float x) {
    const float ax = fabsf(x);
    const float t = 1.0f / fmaf(kErfP, ax, 1.0f);
    const float poly =
        t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, kErfA5, kErfA4), kErfA3), kErfA2), kErfA1);
    return copysignf(1.0f - poly * __expf(-ax * ax), x);
}

__device__ __forceinline__ float gelu_erf(float h) {
    return 0.5f * h * (1.0f + erf_as(h * 0.70710678118654752f));
}

// x held by lane l ^ 32 (one cross-half swap)
__device__ __forceinline__ float other_half(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    // first: every lane's copy of the low half's x; second: of the high half's
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// One wave scores tokens [t0, t0+28) clipped to [tlo, thi] (the decode
// path's deferred batches, split across the waves of a step).  Same
// arithmetic per token as score_pass: layer 1 on v_mfma_f32_32x32x16_bf16
// over the 32 rows t0-2 .. t0+29, with W1's bf16 operands built from the fp32
// weights; a token's score does not depend on how tokens are grouped.
//   Ya       LDS of kWaveScoreBytesA: layer-1 taps 0 and 1 [32 rows][64], wave-private
//   Yb       LDS of kWaveScoreBytesB: layer-1 tap 2 [32 rows][32], wave-private
//   w1g      fp32 W1 of this head [hidden][2D][3]; w2g [hidden][3]
constexpr int kWaveScoreTile = kPassTokens;
constexpr int kWaveScoreBytesA = 32 * 64 * 4;
constexpr int kWaveScoreBytesB = 32 * 32 * 4;

template <int D, class XRow, class AZero, class Store>
__device__ __forceinline__ void score_wave(float* Ya, float* Yb, const float* __restrict__ w1g,
                                           const float* __restrict__ b1g,
                                           const float* __restrict__ w2g, float b2g, int t0,
                                           int tlo, int thi, XRow x_row, AZero a_zero,
                                           Store store) {
    constexpr int KK = ScoreSmem<D>::KK;
    const int lane = threadIdx.x & 63;
    const int tok = t0 - 2 + (lane & 31);
    const uint16_t* kp = nullptr;
    const uint16_t* vp = nullptr;
    const bool ok = x_row(tok, kp, vp);
    // B operand of (tap, kk): element e of lane l is W1[o = l % 32][c = 16 kk + 8 (l/32) + e][tap];
    // one tap at a time (a rare path: registers matter more than reloads)
    const float* wrow = w1g + ((lane & 31) * (2 * D) + (lane >> 5) * 8) * 3;
    for (int tp = 0; tp < 3; ++tp) {
        f32x16 acc = f32x16{};
#pragma unroll 2
        for (int kk = 0; kk < KK; ++kk) {
            const int c = kk * 16 + (lane >> 5) * 8;
            bf16x8 a = bf16x8{};
            if (ok) a = *reinterpret_cast<const bf16x8*>((c < D) ? (kp + c) : (vp + (c - D)));
            bf16x8 bw;
#pragma unroll
            for (int e = 0; e < 8; ++e) bw[e] = (__bf16)wrow[(kk * 16 + e) * 3 + tp];
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw, acc, 0, 0, 0);
        }
        // accumulator element e of lane l: row 8 (e/4) + 4 (l/32) + e%4, column l % 32
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
            if (tp < 2) Ya[row * 64 + tp * 32 + (lane & 31)] = acc[e];
            else Yb[row * 32 + (lane & 31)] = acc[e];
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // hidden layer for rows 1..30 (tokens t0-1 .. t0+28); GELU(h) of row r
    // overwrites Y_1 of row r, which no other lane reads
    for (int x = lane; x < 30 * kHidden; x += 64) {
        const int r = x / kHidden + 1;
        const int o = x % kHidden;
        const int t = t0 - 2 + r;
        float a = 0.0f;
        if (!a_zero(t)) {
            const float h = b1g[o] + Ya[(r - 1) * 64 + o] + Ya[r * 64 + 32 + o] +
                            Yb[(r + 1) * 32 + o];
            a = gelu_erf(h);
        }
        Ya[r * 64 + 32 + o] = a;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // output layer + sigmoid for tokens t0 .. t0+27 (rows 2 .. 29)
    if (lane < kWaveScoreTile) {
        const int t = t0 + lane;
        if (t >= tlo && t <= thi) {
            float z = b2g;
            const float* a = Ya + 32;
            const int r = lane + 2;
#pragma unroll 8
            for (int o = 0; o < kHidden; ++o) {
                z += w2g[o * 3 + 0] * a[(r - 1) * 64 + o] + w2g[o * 3 + 1] * a[r * 64 + o] +
                     w2g[o * 3 + 2] * a[(r + 1) * 64 + o];
            }
            store(t, 1.0f / (1.0f + expf(-z)));
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace lte
