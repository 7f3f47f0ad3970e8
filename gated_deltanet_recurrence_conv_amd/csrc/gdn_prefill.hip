// gdn_prefill.hip -- chunked prompt prefill of the gated delta rule in the
// WY/UT form, on bf16 MFMA (v_mfma_f32_16x16x32_bf16) with fp32 accumulation.
//
// "perf(qwen): full-context MTP draft prefill and replay-free rewind" (Whallm
// PR #14), Measurements: prompts are prefilled layer-major in 1,024-token
// calls; "MTP inference: review and commit structure" (eole docs),
// Verification and limits: the chunk recurrence equals the sequential one up
// to rounding.  The chunked form is that of "Parallelizing Linear
// Transformers with the Delta Rule over Sequence Length" (Yang et al.,
// NeurIPS 2024) applied to the gated rule.  With G_r = sum_{i<=r} g_i,
// gamma_r = exp(G_r), E_ri = exp(G_r - G_i), q^ = q/|q|, k^ = k/|k|, a chunk
// of n <= 64 tokens starting from the state H (d_k x d_v, h = S^T) gives
//   A  = strictly_lower(diag(beta) E o K^K^T),  T = (I + A)^-1
//   U~ = T diag(beta) V,  W~ = T diag(beta gamma) K^,  U = U~ - W~ H
//   O  = scale (diag(gamma) Q^ H + (lower_incl o E o Q^K^T) U)
//   H' = gamma_n H + (diag(exp(G_n - G)) K^)^T U.
// Every row scaling (1/|q|, 1/|k|, beta, gamma, E, scale) is folded into an
// fp32 operand, so the bf16 inputs Q, K, V enter the MFMA exactly.  fp32
// operands that meet bf16 MFMA are split into hi + lo bf16 parts where the
// error budget needs it: T diag(beta), P = scale lower_incl(E o Q^K^T), U,
// diag(s) U, and H in Q H; W~ and H in W~ H take one bf16 rounding each.  A
// float64 emulation of exactly this plan at d = 128 over 1,024 tokens gives
// ~5e-5 normwise output error against the sequential rule (the bound is 2e-3).
//
// Two kernels:
//  prep (grid chunks x value heads x rows): everything that does not depend
//       on the carried state -- norms, G, K K^T, Q K^T, the UT inverse, U~,
//       W~ -- written as one record per (row, head, chunk) in MFMA fragment
//       order, so the scan reads it with 16-byte coalesced loads.
//  scan (grid d_v/16 x value heads x rows): the sequential part.  Each
//       workgroup owns 16 columns of one head's state (the d_v columns are
//       independent recurrences) in VGPRs and walks the chunks: U, then O and
//       H', prefetching the next chunk's fragments while it computes.
//
// MFMA fragment layout (16x16x32 bf16, wave64): A (16 x 32): lane l holds row
// l%16, k = 8*(l/16)..+8; B (32 x 16): lane l holds column l%16, k =
// 8*(l/16)..+8; C (16 x 16): lane l holds column l%16, rows 4*(l/16)..+4.
#include "gdn_internal.h"

namespace gdn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;      // chunk length
constexpr int NTHR = 256;   // 4 waves
constexpr int TP = CH + 8;  // padded row of a [.][64] bf16 LDS tile

__device__ __forceinline__ f32x4 mfma(const uint4& a, const uint4& b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint2 pack4(uint16_t a, uint16_t b, uint16_t c, uint16_t d)
{
    return make_uint2(static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16),
                      static_cast<uint32_t>(c) | (static_cast<uint32_t>(d) << 16));
}

// hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo)
{
    hi = f32_to_bf16_bits(x);
    lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

// Byte layout of one (layer, row, value head, chunk) record in the workspace.
template <int DK, int DV>
struct Rec {
    static constexpr int KS = DK / 32;                           // k-steps over d_k
    static constexpr size_t WT = 0;                              // W~ A-frags [4][KS][64] x 16 B
    static constexpr size_t UT = WT + 4 * KS * 64 * 16;          // U~ C-frags [4][DV/16][64] x 16 B
    static constexpr size_t PH = UT + 4 * (DV / 16) * 64 * 16;   // P hi A-frags [4][2][64] x 16 B
    static constexpr size_t PL = PH + 4 * 2 * 64 * 16;           // P lo
    static constexpr size_t KT = PL + 4 * 2 * 64 * 16;           // K^T A-frags [DK/16][2][64] x 16 B
    static constexpr size_t VEC = KT + (DK / 16) * 2 * 64 * 16;  // qs[64], ks[64], gC
    static constexpr size_t BYTES = VEC + 3 * 64 * 4;
};

// LDS plan of the prep kernel (bytes).  Region X is reused phase by phase:
//  phase 1: Ks, Qs rows                       [X, X + 2*64*KP*2)
//  phase 2: Af (A), Xs (scratch), Tf (T), Pst (P staging)
//  phase 3: T1h, T1l, T2 over Pst and beyond; Wst (W~ staging) over Af/Xs
template <int DK, int DV>
struct PrepLds {
    static constexpr int KP = DK + 8;
    static constexpr size_t KST = 0;                                 // K^T [DK][TP] bf16
    static constexpr size_t VST = KST + static_cast<size_t>(DK) * TP * 2;   // V^T [DV][TP] bf16
    static constexpr size_t VECS = VST + static_cast<size_t>(DV) * TP * 2;  // G, beta, 1/|q|, 1/|k|
    static constexpr size_t X = VECS + 4 * CH * 4;
    // phase 1
    static constexpr size_t KS_ = X;
    static constexpr size_t QS_ = X + static_cast<size_t>(CH) * KP * 2;
    static constexpr size_t P1_END = QS_ + static_cast<size_t>(CH) * KP * 2;
    // phase 2
    static constexpr size_t AF = X;                                  // float [64][65]
    static constexpr size_t XS = AF + CH * (CH + 1) * 4;             // float [3][16][17]
    static constexpr size_t TF = XS + 3 * 16 * 17 * 4;               // float [64][65]
    static constexpr size_t PST = TF + CH * (CH + 1) * 4;            // bf16 [2][64][TP]
    static constexpr size_t P2_END = PST + 2 * CH * TP * 2;
    // phase 3
    static constexpr size_t T1H = PST;                               // bf16 [64][TP]
    static constexpr size_t T1L = T1H + CH * TP * 2;
    static constexpr size_t T2 = T1L + CH * TP * 2;
    static constexpr size_t P3_END = T2 + CH * TP * 2;
    static constexpr size_t WST = X;                                 // bf16 [64][KP]
    static_assert(WST + static_cast<size_t>(CH) * KP * 2 <= TF, "W~ staging overlaps T");
    static constexpr size_t END1 = P1_END > P2_END ? P1_END : P2_END;
    static constexpr size_t BYTES = END1 > P3_END ? END1 : P3_END;
};

// ---------------------------------------------------------------------------
// prep kernel: one workgroup per (chunk, value head, layer*row).
template <int DK, int DV>
__global__ __launch_bounds__(NTHR) void prefill_prep_kernel(PrefillParams p)
{
    using R = Rec<DK, DV>;
    using S = PrepLds<DK, DV>;
    constexpr int KP = S::KP;
    __shared__ __align__(16) char smem[S::BYTES];
    auto KsT = reinterpret_cast<uint16_t(*)[TP]>(smem + S::KST);
    auto VsT = reinterpret_cast<uint16_t(*)[TP]>(smem + S::VST);
    float* Gs = reinterpret_cast<float*>(smem + S::VECS);
    float* Bs = Gs + CH;
    float* Inq = Bs + CH;
    float* Ink = Inq + CH;
    auto Ks = reinterpret_cast<uint16_t(*)[KP]>(smem + S::KS_);
    auto Qs = reinterpret_cast<uint16_t(*)[KP]>(smem + S::QS_);
    auto Af = reinterpret_cast<float(*)[CH + 1]>(smem + S::AF);
    auto Xs = reinterpret_cast<float(*)[16][17]>(smem + S::XS);
    auto Tf = reinterpret_cast<float(*)[CH + 1]>(smem + S::TF);
    auto Pst = reinterpret_cast<uint16_t(*)[CH][TP]>(smem + S::PST);
    auto T1h = reinterpret_cast<uint16_t(*)[TP]>(smem + S::T1H);
    auto T1l = reinterpret_cast<uint16_t(*)[TP]>(smem + S::T1L);
    auto T2 = reinterpret_cast<uint16_t(*)[TP]>(smem + S::T2);
    auto Wst = reinterpret_cast<uint16_t(*)[KP]>(smem + S::WST);

    const int c = blockIdx.x;
    const int hv = blockIdx.y;
    const int lb = blockIdx.z;
    const int NC = (p.T + CH - 1) / CH;
    const int t0 = c * CH;
    const int n = min(CH, p.T - t0);
    const int m = hv / (p.HV / p.HK);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int fr = lane & 15;         // fragment row / column
    const int fk = (lane >> 4) * 8;   // fragment k offset (A, B)
    const int fq = (lane >> 4) * 4;   // fragment row offset (C)
    const size_t C = p.C;
    const bool l2 = (p.flags & FLAG_L2) != 0;
    const uint16_t* y = static_cast<const uint16_t*>(p.y);

    // ---- phase 1: load q, k (qk head m) and v (value head hv) rows ----
    {
        const int r = tid >> 2;   // 4 threads per token row
        const int sub = tid & 3;
        const bool real = r < n;
        const size_t row = (static_cast<size_t>(lb) * p.T + t0 + (real ? r : 0)) * C;
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int v = sub; v < DK / 8; v += 4) {
            uint4 qv = make_uint4(0, 0, 0, 0), kv = make_uint4(0, 0, 0, 0);
            if (real) {
                qv = *reinterpret_cast<const uint4*>(y + row + static_cast<size_t>(m) * DK + v * 8);
                kv = *reinterpret_cast<const uint4*>(y + row + static_cast<size_t>(p.HK + m) * DK + v * 8);
            }
            *reinterpret_cast<uint4*>(&Qs[r][v * 8]) = qv;
            *reinterpret_cast<uint4*>(&Ks[r][v * 8]) = kv;
            const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
            const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float k0 = __uint_as_float(kw[e] << 16), k1 = __uint_as_float(kw[e] & 0xffff0000u);
                const float q0 = __uint_as_float(qw[e] << 16), q1 = __uint_as_float(qw[e] & 0xffff0000u);
                sk = fmaf(k0, k0, sk);
                sk = fmaf(k1, k1, sk);
                sq = fmaf(q0, q0, sq);
                sq = fmaf(q1, q1, sq);
                KsT[v * 8 + 2 * e][r] = static_cast<uint16_t>(kw[e] & 0xffffu);
                KsT[v * 8 + 2 * e + 1][r] = static_cast<uint16_t>(kw[e] >> 16);
            }
        }
#pragma unroll
        for (int v = sub; v < DV / 8; v += 4) {
            uint4 vv = make_uint4(0, 0, 0, 0);
            if (real)
                vv = *reinterpret_cast<const uint4*>(y + row + static_cast<size_t>(2 * p.HK) * DK +
                                                     static_cast<size_t>(hv) * DV + v * 8);
            const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                VsT[v * 8 + 2 * e][r] = static_cast<uint16_t>(vw[e] & 0xffffu);
                VsT[v * 8 + 2 * e + 1][r] = static_cast<uint16_t>(vw[e] >> 16);
            }
        }
        // the 4 threads of one row are consecutive lanes (fixed order)
        sq += __shfl_xor(sq, 1, 64);
        sq += __shfl_xor(sq, 2, 64);
        sk += __shfl_xor(sk, 1, 64);
        sk += __shfl_xor(sk, 2, 64);
        if (sub == 0) {
            Inq[r] = (real && l2) ? 1.0f / sqrtf(sq + p.l2_eps) : 1.0f;
            Ink[r] = (real && l2) ? 1.0f / sqrtf(sk + p.l2_eps) : 1.0f;
        }
    }
    // gates and the within-chunk cumulative log decay (wave 0, fixed order)
    if (w == 0) {
        const size_t gi = (static_cast<size_t>(lb) * p.T + t0 + min(lane, n - 1)) * p.HV + hv;
        float gv = load_act<ACT_BF16>(p.g, gi);
        float bv = load_act<ACT_BF16>(p.beta, gi);
        if (lane >= n) {
            gv = 0.f;
            bv = 0.f;
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_up(gv, off, 64);
            if (lane >= off) gv += o;
        }
        Gs[lane] = gv;
        Bs[lane] = bv;
    }
    __syncthreads();

    // ---- K K^T and Q K^T (64 x 64, K = d_k): wave w owns row tile w ----
    f32x4 kk[4], qk[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        kk[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        qk[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        const uint4 ak = *reinterpret_cast<const uint4*>(&Ks[16 * w + fr][32 * ks + fk]);
        const uint4 aq = *reinterpret_cast<const uint4*>(&Qs[16 * w + fr][32 * ks + fk]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const uint4 bk = *reinterpret_cast<const uint4*>(&Ks[16 * nt + fr][32 * ks + fk]);
            kk[nt] = mfma(ak, bk, kk[nt]);
            qk[nt] = mfma(aq, bk, qk[nt]);
        }
    }
    __syncthreads();   // Ks/Qs are overwritten by phase 2

    // ---- phase 2: A (fp32) and P (split bf16) ----
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * w + fq + j;
            const int i = 16 * nt + fr;
            const float e = (i <= r) ? expf(Gs[r] - Gs[i]) : 0.f;
            Af[r][i] = (i < r) ? Bs[r] * e * kk[nt][j] * Ink[r] * Ink[i] : 0.f;
            const float pv = (i <= r) ? p.scale * e * qk[nt][j] * Inq[r] * Ink[i] : 0.f;
            uint16_t hi, lo;
            split_bf16(pv, hi, lo);
            Pst[0][r][i] = hi;
            Pst[1][r][i] = lo;
        }
    }
    // upper blocks of T are zero
    for (int e = tid; e < CH * CH; e += NTHR) {
        const int r = e / CH, i = e % CH;
        if ((i >> 4) > (r >> 4)) Tf[r][i] = 0.f;
    }
    __syncthreads();

    char* rec = static_cast<char*>(p.ws) +
                ((static_cast<size_t>(lb) * p.HV + hv) * NC + c) * R::BYTES;
    // P fragments: [mt][ks][lane] x 8 bf16 along k, hi and lo planes.
    for (int f = tid; f < 2 * 4 * 2 * 64; f += NTHR) {
        const int ln = f & 63, ks = (f >> 6) & 1, mt = (f >> 7) & 3, pl = f >> 9;
        const uint4 v = *reinterpret_cast<const uint4*>(&Pst[pl][16 * mt + (ln & 15)][32 * ks + (ln >> 4) * 8]);
        *reinterpret_cast<uint4*>(rec + (pl ? R::PL : R::PH) + ((mt * 2 + ks) * 64 + ln) * 16) = v;
    }
    // T = (I + A)^-1: diagonal 16x16 blocks, one thread per (block, column)
    if (tid < 64) {
        const int bb = tid >> 4, j = tid & 15, o = 16 * bb;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i < r && i >= j) s = fmaf(-Af[o + r][o + i], x[i], s);
            x[r] = (r < j) ? 0.f : s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Tf[o + r][o + j] = x[r];
    }
    __syncthreads();
    // off-diagonal blocks by distance d: T_ij = -T_ii * sum_{k=j..i-1} A_ik T_kj
    for (int d = 1; d < 4; ++d) {
        const int nblk = 4 - d;
        for (int e = tid; e < nblk * 256; e += NTHR) {
            const int bj = e >> 8, bi = bj + d, r = (e >> 4) & 15, cc = e & 15;
            float s = 0.f;
            for (int bk = bj; bk < bi; ++bk)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    s = fmaf(Af[16 * bi + r][16 * bk + i], Tf[16 * bk + i][16 * bj + cc], s);
            Xs[bj][r][cc] = s;
        }
        __syncthreads();
        for (int e = tid; e < nblk * 256; e += NTHR) {
            const int bj = e >> 8, bi = bj + d, r = (e >> 4) & 15, cc = e & 15;
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) s = fmaf(Tf[16 * bi + r][16 * bi + i], Xs[bj][i][cc], s);
            Tf[16 * bi + r][16 * bj + cc] = -s;
        }
        __syncthreads();
    }

    // ---- phase 3: T1 = T diag(beta) (split), T2 = T diag(beta gamma / |k|) ----
    for (int e = tid; e < CH * CH; e += NTHR) {
        const int r = e / CH, i = e % CH;
        const float t = Tf[r][i];
        uint16_t hi, lo;
        split_bf16(t * Bs[i], hi, lo);
        T1h[r][i] = hi;
        T1l[r][i] = lo;
        T2[r][i] = f32_to_bf16_bits(t * Bs[i] * expf(Gs[i]) * Ink[i]);
    }
    __syncthreads();

    // U~ = T1 V (64 x DV): wave w owns row tile w; written as C-fragments.
    {
        f32x4 acc[DV / 16];
#pragma unroll
        for (int nt = 0; nt < DV / 16; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint4 ah = *reinterpret_cast<const uint4*>(&T1h[16 * w + fr][32 * ks + fk]);
            const uint4 al = *reinterpret_cast<const uint4*>(&T1l[16 * w + fr][32 * ks + fk]);
#pragma unroll
            for (int nt = 0; nt < DV / 16; ++nt) {
                const uint4 bv = *reinterpret_cast<const uint4*>(&VsT[16 * nt + fr][32 * ks + fk]);
                acc[nt] = mfma(ah, bv, acc[nt]);
                acc[nt] = mfma(al, bv, acc[nt]);
            }
        }
#pragma unroll
        for (int nt = 0; nt < DV / 16; ++nt)
            *reinterpret_cast<f32x4*>(rec + R::UT + ((w * (DV / 16) + nt) * 64 + lane) * 16) = acc[nt];
    }
    // W~ = T2 K (64 x DK), staged row-major in bf16, then written as A-fragments.
    {
        f32x4 acc[DK / 16];
#pragma unroll
        for (int nt = 0; nt < DK / 16; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint4 a2 = *reinterpret_cast<const uint4*>(&T2[16 * w + fr][32 * ks + fk]);
#pragma unroll
            for (int nt = 0; nt < DK / 16; ++nt) {
                const uint4 bk = *reinterpret_cast<const uint4*>(&KsT[16 * nt + fr][32 * ks + fk]);
                acc[nt] = mfma(a2, bk, acc[nt]);
            }
        }
#pragma unroll
        for (int nt = 0; nt < DK / 16; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) Wst[16 * w + fq + j][16 * nt + fr] = f32_to_bf16_bits(acc[nt][j]);
    }
    __syncthreads();
    for (int f = tid; f < 4 * R::KS * 64; f += NTHR) {
        const int ln = f & 63, ks = (f >> 6) % R::KS, mt = (f >> 6) / R::KS;
        const uint4 v = *reinterpret_cast<const uint4*>(&Wst[16 * mt + (ln & 15)][32 * ks + (ln >> 4) * 8]);
        *reinterpret_cast<uint4*>(rec + R::WT + ((mt * R::KS + ks) * 64 + ln) * 16) = v;
    }
    // K^T A-fragments (row = d_k index, k = token) for the state update.
    for (int f = tid; f < (DK / 16) * 2 * 64; f += NTHR) {
        const int ln = f & 63, ks = (f >> 6) & 1, mt = f >> 7;
        const uint4 v = *reinterpret_cast<const uint4*>(&KsT[16 * mt + (ln & 15)][32 * ks + (ln >> 4) * 8]);
        *reinterpret_cast<uint4*>(rec + R::KT + ((mt * 2 + ks) * 64 + ln) * 16) = v;
    }
    // per-token vectors
    if (tid < CH) {
        const int r = tid;
        const float gl = Gs[n - 1];
        float* vec = reinterpret_cast<float*>(rec + R::VEC);
        vec[r] = (r < n) ? p.scale * expf(Gs[r]) * Inq[r] : 0.f;
        vec[CH + r] = (r < n) ? expf(gl - Gs[r]) * Ink[r] : 0.f;
        vec[2 * CH + r] = expf(gl);
    }
}

// ---------------------------------------------------------------------------
// scan kernel: one workgroup per (16-column slice, value head, layer*row).
template <int DK, int DV>
struct ScanFrags {
    static constexpr int KS = DK / 32;
    static constexpr int MQ = (DK / 16 + 3) / 4;   // H' row tiles per wave
    uint4 wt[KS];      // W~ rows of this wave's token tile
    uint4 q[KS];       // raw Q rows of this wave's token tile
    uint4 ph[2], pl[2];
    uint4 kt[MQ][2];   // K^T rows of this wave's state tiles
    f32x4 ut;          // U~ tile
    f32x4 qs, ks;      // per-row output / update scalings
    float gC;
};

template <int DK, int DV>
__device__ __forceinline__ void scan_load(ScanFrags<DK, DV>& f, const char* rec, const uint16_t* yq,
                                          int w, int lane, int cs)
{
    using R = Rec<DK, DV>;
#pragma unroll
    for (int ks = 0; ks < R::KS; ++ks) {
        f.wt[ks] = *reinterpret_cast<const uint4*>(rec + R::WT + ((w * R::KS + ks) * 64 + lane) * 16);
        f.q[ks] = *reinterpret_cast<const uint4*>(yq + 32 * ks);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        f.ph[ks] = *reinterpret_cast<const uint4*>(rec + R::PH + ((w * 2 + ks) * 64 + lane) * 16);
        f.pl[ks] = *reinterpret_cast<const uint4*>(rec + R::PL + ((w * 2 + ks) * 64 + lane) * 16);
    }
#pragma unroll
    for (int qq = 0; qq < ScanFrags<DK, DV>::MQ; ++qq) {
        const int mt = w + 4 * qq;
        if (mt < DK / 16) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                f.kt[qq][ks] = *reinterpret_cast<const uint4*>(rec + R::KT + ((mt * 2 + ks) * 64 + lane) * 16);
        }
    }
    f.ut = *reinterpret_cast<const f32x4*>(rec + R::UT + ((w * (DV / 16) + cs) * 64 + lane) * 16);
    const float* vec = reinterpret_cast<const float*>(rec + R::VEC);
    const int fq = (lane >> 4) * 4;
    f.qs = *reinterpret_cast<const f32x4*>(vec + 16 * w + fq);
    f.ks = *reinterpret_cast<const f32x4*>(vec + CH + 16 * w + fq);
    f.gC = vec[2 * CH];
}

template <int DK, int DV>
__global__ __launch_bounds__(NTHR) void prefill_scan_kernel(PrefillParams p)
{
    using R = Rec<DK, DV>;
    using F = ScanFrags<DK, DV>;
    constexpr int HP = DK + 8;
    __shared__ __align__(16) uint16_t HTh[2][16][HP];   // H^T hi, ping-pong
    __shared__ __align__(16) uint16_t HTl[2][16][HP];   // H^T lo
    __shared__ __align__(16) uint16_t UTh[16][TP];      // U^T hi / lo
    __shared__ __align__(16) uint16_t UTl[16][TP];
    __shared__ __align__(16) uint16_t STh[16][TP];      // (diag(s) U)^T hi / lo
    __shared__ __align__(16) uint16_t STl[16][TP];

    const int cs = blockIdx.x;
    const int hv = blockIdx.y;
    const int lb = blockIdx.z;
    const int NC = (p.T + CH - 1) / CH;
    const int m = hv / (p.HV / p.HK);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int fr = lane & 15;
    const int fk = (lane >> 4) * 8;
    const int fq = (lane >> 4) * 4;

    const int slot = p.cur ? p.cur[lb] : 0;
    if (slot < 0 || slot >= p.S) {
        if (tid == 0 && cs == 0 && p.err) atomicOr(p.err, ERR_SLOT);
        return;
    }
    float* st = p.state + ((static_cast<size_t>(lb) * p.S + slot) * p.HV + hv) * DK * DV;
    const int col = 16 * cs + fr;

    // the state slice: wave w owns row tiles w, w+4, ... in C layout
    f32x4 h[F::MQ];
#pragma unroll
    for (int qq = 0; qq < F::MQ; ++qq) {
        const int mt = w + 4 * qq;
        if (mt < DK / 16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) h[qq][j] = st[(16 * mt + fq + j) * DV + col];
            uint16_t hi[4], lo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split_bf16(h[qq][j], hi[j], lo[j]);
            *reinterpret_cast<uint2*>(&HTh[0][fr][16 * mt + fq]) = pack4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint2*>(&HTl[0][fr][16 * mt + fq]) = pack4(lo[0], lo[1], lo[2], lo[3]);
        }
    }
    __syncthreads();

    const char* recs = static_cast<const char*>(p.ws) + (static_cast<size_t>(lb) * p.HV + hv) * NC * R::BYTES;
    const uint16_t* y = static_cast<const uint16_t*>(p.y);
    auto qrow = [&](int c) {
        const int t = min(c * CH + 16 * w + fr, p.T - 1);
        return y + (static_cast<size_t>(lb) * p.T + t) * p.C + static_cast<size_t>(m) * DK + fk;
    };

    F cur;
    scan_load<DK, DV>(cur, recs, qrow(0), w, lane, cs);
    for (int c = 0; c < NC; ++c) {
        const int pb = c & 1;
        F nxt;
        if (c + 1 < NC) scan_load<DK, DV>(nxt, recs + static_cast<size_t>(c + 1) * R::BYTES, qrow(c + 1), w, lane, cs);

        // U = U~ - W~ H (this wave's 16 tokens x 16 columns)
        f32x4 wh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < R::KS; ++ks) {
            const uint4 hb = *reinterpret_cast<const uint4*>(&HTh[pb][fr][32 * ks + fk]);
            wh = mfma(cur.wt[ks], hb, wh);
        }
        f32x4 u;
        uint16_t uh[4], ul[4], sh[4], sl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u[j] = cur.ut[j] - wh[j];
            split_bf16(u[j], uh[j], ul[j]);
            split_bf16(cur.ks[j] * u[j], sh[j], sl[j]);
        }
        *reinterpret_cast<uint2*>(&UTh[fr][16 * w + fq]) = pack4(uh[0], uh[1], uh[2], uh[3]);
        *reinterpret_cast<uint2*>(&UTl[fr][16 * w + fq]) = pack4(ul[0], ul[1], ul[2], ul[3]);
        *reinterpret_cast<uint2*>(&STh[fr][16 * w + fq]) = pack4(sh[0], sh[1], sh[2], sh[3]);
        *reinterpret_cast<uint2*>(&STl[fr][16 * w + fq]) = pack4(sl[0], sl[1], sl[2], sl[3]);
        __syncthreads();

        // O = diag(qs) Q H + P U
        f32x4 qh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < R::KS; ++ks) {
            const uint4 hb = *reinterpret_cast<const uint4*>(&HTh[pb][fr][32 * ks + fk]);
            const uint4 lb_ = *reinterpret_cast<const uint4*>(&HTl[pb][fr][32 * ks + fk]);
            qh = mfma(cur.q[ks], hb, qh);
            qh = mfma(cur.q[ks], lb_, qh);
        }
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = cur.qs[j] * qh[j];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint4 bh = *reinterpret_cast<const uint4*>(&UTh[fr][32 * ks + fk]);
            const uint4 bl = *reinterpret_cast<const uint4*>(&UTl[fr][32 * ks + fk]);
            o = mfma(cur.ph[ks], bh, o);
            o = mfma(cur.ph[ks], bl, o);
            o = mfma(cur.pl[ks], bh, o);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = c * CH + 16 * w + fq + j;
            if (t < p.T) {
                const size_t oi = ((static_cast<size_t>(lb) * p.T + t) * p.HV + hv) * DV + col;
                if (p.out == ACT_BF16) static_cast<uint16_t*>(p.o)[oi] = f32_to_bf16_bits(o[j]);
                else static_cast<float*>(p.o)[oi] = o[j];
            }
        }

        // H' = gC H + K^T (diag(s) U) for this wave's state tiles
#pragma unroll
        for (int qq = 0; qq < F::MQ; ++qq) {
            const int mt = w + 4 * qq;
            if (mt < DK / 16) {
                f32x4 acc;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = cur.gC * h[qq][j];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const uint4 bh = *reinterpret_cast<const uint4*>(&STh[fr][32 * ks + fk]);
                    const uint4 bl = *reinterpret_cast<const uint4*>(&STl[fr][32 * ks + fk]);
                    acc = mfma(cur.kt[qq][ks], bh, acc);
                    acc = mfma(cur.kt[qq][ks], bl, acc);
                }
                h[qq] = acc;
                uint16_t hi[4], lo[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) split_bf16(acc[j], hi[j], lo[j]);
                *reinterpret_cast<uint2*>(&HTh[pb ^ 1][fr][16 * mt + fq]) = pack4(hi[0], hi[1], hi[2], hi[3]);
                *reinterpret_cast<uint2*>(&HTl[pb ^ 1][fr][16 * mt + fq]) = pack4(lo[0], lo[1], lo[2], lo[3]);
            }
        }
        __syncthreads();
        if (c + 1 < NC) cur = nxt;
    }
#pragma unroll
    for (int qq = 0; qq < F::MQ; ++qq) {
        const int mt = w + 4 * qq;
        if (mt < DK / 16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) st[(16 * mt + fq + j) * DV + col] = h[qq][j];
        }
    }
}

template <int DK, int DV>
hipError_t launch_pf(const PrefillParams& p, hipStream_t s)
{
    const int NC = (p.T + CH - 1) / CH;
    const long long rows = static_cast<long long>(p.L) * p.B;
    if (NC > 0x7fffffff || p.HV > 65535 || rows > 65535) return hipErrorInvalidConfiguration;
    clear_stale_error();
    hipLaunchKernelGGL((prefill_prep_kernel<DK, DV>), dim3(NC, p.HV, static_cast<unsigned>(rows)),
                       dim3(NTHR), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_scan_kernel<DK, DV>), dim3(DV / 16, p.HV, static_cast<unsigned>(rows)),
                       dim3(NTHR), 0, s, p);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_pf_dv(const PrefillParams& p, int DV, hipStream_t s)
{
    switch (DV) {
    case 16: return launch_pf<DK, 16>(p, s);
    case 32: return launch_pf<DK, 32>(p, s);
    case 64: return launch_pf<DK, 64>(p, s);
    case 128: return launch_pf<DK, 128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

template <int DK>
size_t rec_bytes_dv(int DV)
{
    switch (DV) {
    case 16: return Rec<DK, 16>::BYTES;
    case 32: return Rec<DK, 32>::BYTES;
    case 64: return Rec<DK, 64>::BYTES;
    case 128: return Rec<DK, 128>::BYTES;
    default: return 0;
    }
}

}  // namespace

bool prefill_supported(int DK, int DV, int act)
{
    return act == ACT_BF16 && (DK == 32 || DK == 64 || DK == 128) &&
           (DV == 16 || DV == 32 || DV == 64 || DV == 128);
}

size_t prefill_workspace_bytes(int L, int B, int T, int HV, int DK, int DV, int chunk)
{
    if (chunk != CH) return 0;
    size_t rec = 0;
    switch (DK) {
    case 32: rec = rec_bytes_dv<32>(DV); break;
    case 64: rec = rec_bytes_dv<64>(DV); break;
    case 128: rec = rec_bytes_dv<128>(DV); break;
    default: return 0;
    }
    const size_t NC = (static_cast<size_t>(T) + CH - 1) / CH;
    return static_cast<size_t>(L) * B * HV * NC * rec;
}

hipError_t launch_prefill(const PrefillParams& p, int DK, int DV, hipStream_t s)
{
    switch (DK) {
    case 32: return launch_pf_dv<32>(p, DV, s);
    case 64: return launch_pf_dv<64>(p, DV, s);
    case 128: return launch_pf_dv<128>(p, DV, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
