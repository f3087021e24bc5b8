// Body of the retention-scoring CNN, shared by the prefill scorer (tokens read
// from the k/v prompt tensors) and the deferred batched scorer of the decode
// path (tokens read from the cache's ring slots).
//
// LTE paper (arXiv 2510.20787) summary page, Figure 2 caption: a CNN reads the
// keys/values of past and future neighbours and emits r_{j,h}; the score of a
// token is computable once its receptive field (tokens j-2 .. j+2 for two
// kernel-3 layers) is present.
//
// score_chunk: one workgroup of 256 threads (4 waves) scores the 124 tokens
// [t0, t0+124) (prefill).  score_wave: one wave scores 28 tokens (decode).  Layer 1 is written as Y_tap = W1[:, :, tap] . x per token
// (v_mfma_f32_32x32x16_bf16, 32 tokens x 96 outputs per wave), then
// h[j] = b1 + Y_0[j-1] + Y_1[j] + Y_2[j+1].
#pragma once

#include "lte_internal.h"

namespace lte {

constexpr int kScoreTile = 124;        // scored tokens per workgroup call
constexpr int kScoreRows = 128;        // tokens whose Y a call computes

template <int D>
struct ScoreSmem {
    static constexpr int KK = (2 * D) / 16;          // MFMA k-steps over the 2D channels
    static constexpr int NW = 3 * KK * 64;           // bf16x8 entries of one head's packed W1
    static constexpr int kBytes = (NW * 16 > kScoreRows * 96 * 4) ? NW * 16 : kScoreRows * 96 * 4;
};

__device__ __forceinline__ float gelu_erf(float h) {
    return 0.5f * h * (1.0f + erff(h * 0.70710678118654752f));
}

// Packed-W1 entry index x (bf16x8 units) -> (tap, kk, lane); element e of the
// entry holds W1[o = lane % 32][c = 16 kk + 8 (lane / 32) + e][tap].
__device__ __forceinline__ void w1p_coords(int x, int KK, int& tap, int& kk, int& lane) {
    lane = x % 64;
    kk = (x / 64) % KK;
    tap = x / (64 * KK);
}

// Scores tokens [t0, t0+124) clipped to [tlo, thi] and hands each to store(t, r).
//   buf      LDS of ScoreSmem<D>::kBytes, already holding this head's packed W1
//   w2s      LDS copy of this head's W2 [32][3]
//   x_row(x, kp, vp) -> true and row pointers of token x, or false: x reads as 0
//   a_zero(x)        -> true where layer 2 sees zero padding (outside the sequence)
// Ends with the LDS buffer overwritten (holds Y); callers re-stage W1 to reuse it.
template <int D, class XRow, class AZero, class Store>
__device__ __forceinline__ void score_chunk(unsigned char* buf, const float* w2s,
                                            const float* __restrict__ b1g, float b2g, int t0,
                                            int tlo, int thi, XRow x_row, AZero a_zero,
                                            Store store) {
    constexpr int KK = ScoreSmem<D>::KK;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bf16x8* wl = reinterpret_cast<const bf16x8*>(buf);

    // A operands: token (lane % 32) of this wave's 32, channels 16 kk + 8 (lane/32) .. +8
    const int tok = t0 - 2 + wave * 32 + (lane & 31);
    const uint16_t* kp = nullptr;
    const uint16_t* vp = nullptr;
    const bool ok = x_row(tok, kp, vp);
    bf16x8 afrag[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const int c = kk * 16 + (lane >> 5) * 8;
        if (ok) {
            const uint16_t* src = (c < D) ? (kp + c) : (vp + (c - D));
            afrag[kk] = *reinterpret_cast<const bf16x8*>(src);
        } else {
            afrag[kk] = bf16x8{};
        }
    }
    __syncthreads();                                  // W1 staged by the caller

    f32x16 acc[3];
#pragma unroll
    for (int tp = 0; tp < 3; ++tp) acc[tp] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int tp = 0; tp < 3; ++tp) {
            const bf16x8 bfrag = wl[(tp * KK + kk) * 64 + lane];
            acc[tp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[kk], bfrag, acc[tp], 0, 0, 0);
        }
    }
    __syncthreads();                                  // W1 no longer read: reuse for Y

    // accumulator element e of lane l: row (token) 8 (e/4) + 4 (l/32) + e%4,
    // column (output) l % 32
    float* Y = reinterpret_cast<float*>(buf);         // [128][96]
#pragma unroll
    for (int tp = 0; tp < 3; ++tp) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = wave * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
            Y[row * 96 + tp * 32 + (lane & 31)] = acc[tp][e];
        }
    }
    __syncthreads();

    // hidden layer for local rows 1..126 (tokens t0-1 .. t0+124).  GELU(h) of
    // row r overwrites Y_1 of row r: that element is read by this thread only.
    for (int x = tid; x < (kScoreRows - 2) * kHidden; x += 256) {
        const int r = x / kHidden + 1;
        const int o = x % kHidden;
        const int t = t0 - 2 + r;
        float a = 0.0f;
        if (!a_zero(t)) {
            const float h = b1g[o] + Y[(r - 1) * 96 + o] + Y[r * 96 + 32 + o] +
                            Y[(r + 1) * 96 + 64 + o];
            a = gelu_erf(h);
        }
        Y[r * 96 + 32 + o] = a;
    }
    __syncthreads();

    // output layer + sigmoid for tokens t0 .. t0+123 (local rows 2 .. 125)
    if (tid < kScoreTile) {
        const int t = t0 + tid;
        if (t >= tlo && t <= thi) {
            float z = b2g;
            const float* a = Y + 32;
            const int r = tid + 2;
#pragma unroll 8
            for (int o = 0; o < kHidden; ++o) {
                z += w2s[o * 3 + 0] * a[(r - 1) * 96 + o] + w2s[o * 3 + 1] * a[r * 96 + o] +
                     w2s[o * 3 + 2] * a[(r + 1) * 96 + o];
            }
            store(t, 1.0f / (1.0f + expf(-z)));
        }
    }
    __syncthreads();
}

// One wave scores tokens [t0, t0+28) clipped to [tlo, thi] (the decode
// path's deferred batches, split across the waves of a step).  Same
// arithmetic per token as score_chunk: layer 1 on v_mfma_f32_32x32x16_bf16
// over the 32 rows t0-2 .. t0+29, with W1's bf16 operands built from the fp32
// weights; a token's score does not depend on how tokens are grouped.
//   Ya       LDS of kWaveScoreBytesA: layer-1 taps 0 and 1 [32 rows][64], wave-private
//   Yb       LDS of kWaveScoreBytesB: layer-1 tap 2 [32 rows][32], wave-private
//   w1g      fp32 W1 of this head [hidden][2D][3]; w2g [hidden][3]
constexpr int kWaveScoreTile = 28;
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
