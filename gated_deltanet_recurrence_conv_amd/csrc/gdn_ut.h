// gdn_ut.h -- fp32 MFMA helpers shared by the chunked-prefill kernels: 16x16
// block products of LDS-resident fp32 matrices on v_mfma_f32_16x16x4f32, and
// the inverse of the unit lower-triangular 64 x 64 matrix I + A of the WY/UT
// form ("Parallelizing Linear Transformers with the Delta Rule over Sequence
// Length", Yang et al., NeurIPS 2024; Joffrain et al., "Accumulating
// Householder transformations, revisited", ACM TOMS 2006).  Not part of the
// ABI.
//
// Fragment layout of the 16x16x4 fp32 MFMA (wave64): A (16 x 4): lane l holds
// A[l%16][l/16]; B (4 x 16): lane l holds B[l/16][l%16]; C (16 x 16): lane l
// holds column l%16, rows 4*(l/16)..+4.
#pragma once

#include "gdn_internal.h"

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16x16 block product on fp32 MFMA, operands in LDS with row pitches XP, YP
// (floats): acc += X[xr.., xc..] * Y[yr.., yc..] (one 16-wide k block).
template <int XP, int YP>
__device__ __forceinline__ f32x4 blk_mul(const float* X, int xr, int xc, const float* Y, int yr, int yc,
                                         f32x4 acc, int fr, int gq)
{
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        acc = mfma32(X[(xr + fr) * XP + xc + 4 * kk + gq], Y[(yr + 4 * kk + gq) * YP + yc + fr], acc);
    return acc;
}

// Stores a C tile scaled by sgn at (r0, c0) of a matrix with row pitch MP.
template <int MP>
__device__ __forceinline__ void blk_store(float* M, int r0, int c0, const f32x4& v, float sgn, int fr, int gq)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) M[(r0 + 4 * gq + j) * MP + c0 + fr] = sgn * v[j];
}

// T = (I + A)^-1 for a strictly lower-triangular 64 x 64 fp32 matrix A in LDS
// (row pitch FP), run by the four waves of a workgroup (w = wave index).
// Only the blocks on and below the diagonal of Tf are written; the caller
// keeps the six blocks above it zero.  Scr is per-wave scratch.
//  - diagonal 16x16 block w: (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8),
//    exact because N is strictly lower triangular (N^16 = 0);
//  - the subdiagonal blocks of the two 32 x 32 halves: T10 = -D1 A10 D0,
//    T32 = -D3 A32 D2;
//  - the lower-left 32 x 32 quadrant: X = A[32:64, 0:32] T[0:32, 0:32], then
//    T[32:64, 0:32] = -T[32:64, 32:64] X.
// Every stage ends with a workgroup barrier over LDS.
template <int FP>
__device__ __forceinline__ void ut_inverse64(const float* Af, float* Tf, float (*Scr)[2][16][17], int w, int fr,
                                             int gq)
{
    constexpr int SP = 17;
    {
        float* S0 = &Scr[w][0][0][0];
        float* S1 = &Scr[w][1][0][0];
        const int o = 16 * w;
        f32x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = ((4 * gq + j) == fr ? 1.f : 0.f) - Af[(o + 4 * gq + j) * FP + o + fr];
        blk_store<FP>(Tf, o, o, x, 1.f, fr, gq);
        f32x4 pw = blk_mul<FP, FP>(Af, o, o, Af, o, o, f32x4{0.f, 0.f, 0.f, 0.f}, fr, gq);   // N^2
        blk_store<SP>(S0, 0, 0, pw, 1.f, fr, gq);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int step = 0; step < 3; ++step) {
            float* Pcur = (step & 1) ? S1 : S0;
            float* Pnext = (step & 1) ? S0 : S1;
            x = blk_mul<FP, SP>(Tf, o, o, Pcur, 0, 0, x, fr, gq);   // X += X P
            if (step < 2) pw = blk_mul<SP, SP>(Pcur, 0, 0, Pcur, 0, 0, f32x4{0.f, 0.f, 0.f, 0.f}, fr, gq);
            __builtin_amdgcn_wave_barrier();
            blk_store<FP>(Tf, o, o, x, 1.f, fr, gq);
            if (step < 2) blk_store<SP>(Pnext, 0, 0, pw, 1.f, fr, gq);
            __builtin_amdgcn_wave_barrier();
        }
    }
    lds_barrier();
    if (w == 1 || w == 3) {
        const int b = 16 * (w - 1);   // column block of the pair
        float* S0 = &Scr[w][0][0][0];
        const f32x4 xa = blk_mul<FP, FP>(Af, b + 16, b, Tf, b, b, f32x4{0.f, 0.f, 0.f, 0.f}, fr, gq);
        blk_store<SP>(S0, 0, 0, xa, 1.f, fr, gq);
        __builtin_amdgcn_wave_barrier();
        const f32x4 t = blk_mul<FP, SP>(Tf, b + 16, b + 16, S0, 0, 0, f32x4{0.f, 0.f, 0.f, 0.f}, fr, gq);
        blk_store<FP>(Tf, b + 16, b, t, -1.f, fr, gq);
    }
    lds_barrier();
    {
        const int pr = w >> 1, pc = w & 1;   // this wave's 16x16 block of X
        f32x4 xa = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kb = pc; kb < 2; ++kb)   // T[0:32,0:32] is block lower triangular
            xa = blk_mul<FP, FP>(Af, 32 + 16 * pr, 16 * kb, Tf, 16 * kb, 16 * pc, xa, fr, gq);
        blk_store<SP>(&Scr[pr][pc][0][0], 0, 0, xa, 1.f, fr, gq);
    }
    lds_barrier();
    {
        const int pr = w >> 1, pc = w & 1;
        f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb <= pr; ++kb)   // T[32:64, 32:64] is block lower triangular
            t = blk_mul<FP, SP>(Tf, 32 + 16 * pr, 32 + 16 * kb, &Scr[kb][pc][0][0], 0, 0, t, fr, gq);
        blk_store<FP>(Tf, 32 + 16 * pr, 16 * pc, t, -1.f, fr, gq);
    }
    lds_barrier();
}

}  // namespace gdn
