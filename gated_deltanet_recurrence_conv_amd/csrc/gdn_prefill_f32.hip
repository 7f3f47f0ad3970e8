// gdn_prefill_f32.hip -- the chunked prompt prefill in fp32: fp32 activations
// (the tiny fp32 workload and any fp32 caller) and head shapes the bf16 MFMA
// kernels do not tile (d_k = 16).  Same WY/UT chunk form as the bf16 path
// ("Parallelizing Linear Transformers with the Delta Rule over Sequence
// Length", Yang et al., NeurIPS 2024, applied to the gated rule), with every
// dense product on fp32 MFMA (v_mfma_f32_16x16x4f32) over LDS-resident fp32
// operands, so the result is the sequential recurrence up to fp32 rounding
// ("MTP inference: review and commit structure" (eole docs), Verification and
// limits: chunk and sequential recurrences differ only in rounding;
// "perf(qwen): full-context MTP draft prefill and replay-free rewind",
// Measurements: layer-major prefill calls).
//
// One 256-thread workgroup per (layer*row, value head, 16-column slice of
// d_v) walks the row's chunks in order; its slice of the state stays in LDS.
// For a chunk of n <= 64 tokens with raw rows K, Q (qk head), V (the slice),
// norms 1/|k|, 1/|q| (or 1 without the L2 flag), G = cumsum(g) (kept in fp64
// so that decays within a chunk keep full fp32 accuracy), D_ri = e^{G_r-G_i}:
//   A  = strictly_lower(diag(beta / |k|) D o K K^T diag(1/|k|)),  T = (I + A)^-1
//   X  = diag(1/|k|) K H,   R = diag(beta) (V - diag(e^G) X),   U = T R
//   O  = scale (diag(e^G / |q|) Q H + (lower_incl D o diag(1/|q|) Q K^T diag(1/|k|)) U)
//   H' = e^{G_n} H + K^T diag(e^{G_n - G} / |k|) U
// which is the chunk form W~ H = T diag(beta e^G) K^ H rewritten so that no
// W~ or U~ is stored.  Wave w owns token tile w (rows 16w..16w+15) of every
// chunk-sized product and d_k tiles w, w+4, ... of H'.
#include <atomic>

#include "gdn_internal.h"
#include "gdn_ut.h"

namespace gdn {

namespace {

constexpr int FC = 64;     // chunk length
constexpr int FT = 256;    // threads (4 waves)
constexpr int FSW = 16;    // state columns per workgroup

// LDS layout in floats (dynamic shared memory).
template <int DK>
struct FLds {
    static constexpr int KP = DK + 4;   // row pitch of K and Q rows
    static constexpr int SP = FSW + 4;  // row pitch of 16-column matrices
    static constexpr int MP = FC + 4;   // row pitch of 64 x 64 matrices
    static constexpr int KR = 0;                      // K rows [FC][KP]
    static constexpr int QR = KR + FC * KP;           // Q rows [FC][KP]
    static constexpr int HS = QR + FC * KP;           // H slice [DK][SP]
    static constexpr int VS = HS + DK * SP;           // V, then R [FC][SP]
    static constexpr int US = VS + FC * SP;           // U [FC][SP]
    static constexpr int AM = US + FC * SP;           // A, then P [FC][MP]
    static constexpr int TM = AM + FC * MP;           // T [FC][MP]
    static constexpr int SC = TM + FC * MP;           // inverse scratch [4][2][16][17]
    static constexpr int GD = SC + 4 * 2 * 16 * 17;   // G as fp64 [FC] (2 floats each)
    static constexpr int BV = GD + 2 * FC;            // beta
    static constexpr int NK = BV + FC;                // 1/|k|
    static constexpr int NQ = NK + FC;                // 1/|q|
    static constexpr int GA = NQ + FC;                // e^{G_r}
    static constexpr int DN = GA + FC;                // e^{G_n - G_r} (0 past the chunk)
    static constexpr int FLOATS = DN + FC;
    static constexpr size_t BYTES = static_cast<size_t>(FLOATS) * 4;
    static_assert(GD % 2 == 0, "fp64 alignment");
};

// C tile (rows r0.., columns c0..) += sum over k in [k0, k1) of
// opA(r, k) opB(k, c), opA(r, k) = AT ? A[k lda + r] : A[r lda + k],
// opB(k, c) = BT ? B[c ldb + k] : B[k ldb + c]; k1 - k0 a multiple of 4.
template <bool AT, bool BT>
__device__ __forceinline__ f32x4 mm16(const float* A, int lda, const float* B, int ldb, int r0, int c0, int k0,
                                      int k1, f32x4 acc, int fr, int gq)
{
    for (int k = k0; k < k1; k += 4) {
        const float a = AT ? A[(k + gq) * lda + r0 + fr] : A[(r0 + fr) * lda + k + gq];
        const float b = BT ? B[(c0 + fr) * ldb + k + gq] : B[(k + gq) * ldb + c0 + fr];
        acc = mfma32(a, b, acc);
    }
    return acc;
}

__device__ __forceinline__ float decay(const double* Gd, int r, int i)
{
    return static_cast<float>(exp(Gd[r] - Gd[i]));
}

template <int DK, int ACT, int OUT>
__global__ __launch_bounds__(FT) void prefill_f32_kernel(PrefillParams p, int DV)
{
    using F = FLds<DK>;
    extern __shared__ __align__(16) float lds[];
    float* Kr = lds + F::KR;
    float* Qr = lds + F::QR;
    float* Hs = lds + F::HS;
    float* Vs = lds + F::VS;
    float* Us = lds + F::US;
    float* Am = lds + F::AM;
    float* Tm = lds + F::TM;
    auto Scr = reinterpret_cast<float(*)[2][16][17]>(lds + F::SC);
    double* Gd = reinterpret_cast<double*>(lds + F::GD);
    float* Bv = lds + F::BV;
    float* Nk = lds + F::NK;
    float* Nq = lds + F::NQ;
    float* Ga = lds + F::GA;
    float* Dn = lds + F::DN;
    constexpr int KP = F::KP, SP = F::SP, MP = F::MP;

    const int cs = blockIdx.x;
    const int hv = blockIdx.y;
    const int lb = blockIdx.z;
    const int m = hv / (p.HV / p.HK);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int fr = lane & 15, gq = lane >> 4;

    const int slot = p.cur ? p.cur[lb] : 0;
    const int len = p.lengths ? p.lengths[lb % p.B] : p.T;
    {
        const int e = (slot < 0 || slot >= p.S ? ERR_SLOT : 0) | (len < 0 || len > p.T ? ERR_LENGTH : 0);
        if (e) {
            if (tid == 0 && cs == 0 && hv == 0 && p.err) atomicOr(p.err, e);
            return;
        }
    }
    if (len == 0) return;

    float* st = p.state + ((static_cast<size_t>(lb) * p.S + slot) * p.HV + hv) * DK * DV + cs * FSW;
    for (int e = tid; e < DK * FSW; e += FT) Hs[(e / FSW) * SP + e % FSW] = st[(e / FSW) * DV + e % FSW];
    // the blocks of T above the diagonal are zero (the inverse writes only
    // those on and below it)
    for (int e = tid; e < FC * FC; e += FT)
        if (((e % FC) >> 4) > ((e / FC) >> 4)) Tm[(e / FC) * MP + e % FC] = 0.f;

    const bool l2 = (p.flags & FLAG_L2) != 0;
    const size_t C = p.C;
    const int NC = (len + FC - 1) / FC;
    for (int c = 0; c < NC; ++c) {
        const int t0 = c * FC;
        const int n = min(FC, len - t0);
        const size_t row0 = static_cast<size_t>(lb) * p.T + t0;

        // ---- K, Q rows of qk head m, the V slice, g, beta; rows past n are zero ----
        for (int e = tid; e < FC * DK; e += FT) {
            const int r = e / DK, i = e % DK;
            float kv = 0.f, qv = 0.f;
            if (r < n) {
                const size_t base = (row0 + r) * C;
                kv = load_act<ACT>(p.y, base + static_cast<size_t>(p.HK + m) * DK + i);
                qv = load_act<ACT>(p.y, base + static_cast<size_t>(m) * DK + i);
            }
            Kr[r * KP + i] = kv;
            Qr[r * KP + i] = qv;
        }
        for (int e = tid; e < FC * FSW; e += FT) {
            const int r = e / FSW, j = e % FSW;
            Vs[r * SP + j] = r < n ? load_act<ACT>(p.y, (row0 + r) * C + static_cast<size_t>(2 * p.HK) * DK +
                                                        static_cast<size_t>(hv) * DV + cs * FSW + j)
                                   : 0.f;
        }
        float graw = 0.f;
        if (w == 2) {
            const size_t gi = (row0 + lane) * p.HV + hv;
            graw = lane < n ? load_act<ACT>(p.g, gi) : 0.f;
            Bv[lane] = lane < n ? load_act<ACT>(p.beta, gi) : 0.f;
        }
        lds_barrier();

        // ---- norms (wave 0: keys, wave 1: queries), G = cumsum(g) in fp64 (wave 2) ----
        if (w < 2) {
            const float* row = (w == 0 ? Kr : Qr) + lane * KP;
            float s2 = 0.f;
            for (int i = 0; i < DK; ++i) s2 = fmaf(row[i], row[i], s2);
            (w == 0 ? Nk : Nq)[lane] = (l2 && lane < n) ? 1.0f / sqrtf(s2 + p.l2_eps) : 1.0f;
        } else if (w == 2) {
            double gv = graw;
            for (int off = 1; off < 64; off <<= 1) {   // inclusive scan, fixed order
                const double o = __shfl_up(gv, off, 64);
                if (lane >= off) gv += o;
            }
            Gd[lane] = gv;
            const double gl = __shfl(gv, n - 1, 64);
            Ga[lane] = static_cast<float>(exp(gv));
            Dn[lane] = lane < n ? static_cast<float>(exp(gl - gv)) : 0.f;
        }
        lds_barrier();

        // ---- wave w: A row tile w; X = K^ H and R in place of V; Q^ H in registers ----
        const int r0 = 16 * w;
        for (int ct = 0; ct <= w; ++ct) {
            const f32x4 kk = mm16<false, true>(Kr, KP, Kr, KP, r0, 16 * ct, 0, DK, f32x4{0.f, 0.f, 0.f, 0.f}, fr, gq);
            const int i = 16 * ct + fr;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = r0 + 4 * gq + j;
                Am[r * MP + i] = i < r ? Bv[r] * Nk[r] * Nk[i] * decay(Gd, r, i) * kk[j] : 0.f;
            }
        }
        f32x4 qh;
        {
            const f32x4 x = mm16<false, false>(Kr, KP, Hs, SP, r0, 0, 0, DK, f32x4{0.f, 0.f, 0.f, 0.f}, fr, gq);
            qh = mm16<false, false>(Qr, KP, Hs, SP, r0, 0, 0, DK, f32x4{0.f, 0.f, 0.f, 0.f}, fr, gq);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = r0 + 4 * gq + j;
                float* v = &Vs[r * SP + fr];
                *v = Bv[r] * (*v - Ga[r] * (Nk[r] * x[j]));
                qh[j] *= Nq[r];
            }
        }

        // ---- T = (I + A)^-1; ends with a workgroup barrier ----
        ut_inverse64<MP>(Am, Tm, Scr, w, fr, gq);

        // ---- U = T R (row tile w); P = lower_incl(D o Q^ K^T) scaled, in place of A ----
        {
            f32x4 u = f32x4{0.f, 0.f, 0.f, 0.f};
            u = mm16<false, false>(Tm, MP, Vs, SP, r0, 0, 0, r0 + 16, u, fr, gq);
#pragma unroll
            for (int j = 0; j < 4; ++j) Us[(r0 + 4 * gq + j) * SP + fr] = u[j];
        }
        for (int ct = 0; ct < 4; ++ct) {
            f32x4 qk = f32x4{0.f, 0.f, 0.f, 0.f};
            if (ct <= w) qk = mm16<false, true>(Qr, KP, Kr, KP, r0, 16 * ct, 0, DK, qk, fr, gq);
            const int i = 16 * ct + fr;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = r0 + 4 * gq + j;
                Am[r * MP + i] = i <= r ? p.scale * Nq[r] * Nk[i] * decay(Gd, r, i) * qk[j] : 0.f;
            }
        }
        lds_barrier();

        // ---- O (row tile w) and H' (d_k tiles w, w + 4, ...) ----
        {
            f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
            o = mm16<false, false>(Am, MP, Us, SP, r0, 0, 0, r0 + 16, o, fr, gq);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = r0 + 4 * gq + j;
                if (r < n) {
                    const float v = p.scale * Ga[r] * qh[j] + o[j];
                    const size_t oi = ((row0 + r) * p.HV + hv) * DV + cs * FSW + fr;
                    if constexpr (OUT == ACT_BF16) static_cast<uint16_t*>(p.o)[oi] = f32_to_bf16_bits(v);
                    else static_cast<float*>(p.o)[oi] = v;
                }
            }
        }
        const float gn = Ga[n - 1];
        for (int a = w; a < DK / 16; a += 4) {
            f32x4 h;
#pragma unroll
            for (int j = 0; j < 4; ++j) h[j] = gn * Hs[(16 * a + 4 * gq + j) * SP + fr];
            for (int k = 0; k < FC; k += 4) {
                const int r = k + gq;
                h = mfma32(Kr[r * KP + 16 * a + fr], Nk[r] * Dn[r] * Us[r * SP + fr], h);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) Hs[(16 * a + 4 * gq + j) * SP + fr] = h[j];
        }
        lds_barrier();
    }
    for (int e = tid; e < DK * FSW; e += FT) st[(e / FSW) * DV + e % FSW] = Hs[(e / FSW) * SP + e % FSW];
}

template <int DK, int ACT, int OUT>
hipError_t launch_f32_one(const PrefillParams& p, int DV, hipStream_t s)
{
    constexpr size_t bytes = FLds<DK>::BYTES;
    static std::atomic<int> attr_set{0};
    if (!attr_set.load(std::memory_order_acquire)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_f32_kernel<DK, ACT, OUT>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
        if (e != hipSuccess) return e;
        attr_set.store(1, std::memory_order_release);
    }
    const dim3 grid(DV / FSW, p.HV, static_cast<unsigned>(static_cast<long long>(p.L) * p.B));
    hipLaunchKernelGGL((prefill_f32_kernel<DK, ACT, OUT>), grid, dim3(FT), bytes, s, p, DV);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_f32_dk(const PrefillParams& p, int DV, hipStream_t s)
{
    if (p.act == ACT_BF16)
        return p.out == ACT_BF16 ? launch_f32_one<DK, ACT_BF16, ACT_BF16>(p, DV, s)
                                 : launch_f32_one<DK, ACT_BF16, ACT_F32>(p, DV, s);
    return p.out == ACT_BF16 ? launch_f32_one<DK, ACT_F32, ACT_BF16>(p, DV, s)
                             : launch_f32_one<DK, ACT_F32, ACT_F32>(p, DV, s);
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams& p, int DK, int DV, hipStream_t s)
{
    if (p.HV > 65535 || static_cast<long long>(p.L) * p.B > 65535 || DV % FSW != 0)
        return hipErrorInvalidConfiguration;
    clear_stale_error();
    switch (DK) {
    case 16: return launch_f32_dk<16>(p, DV, s);
    case 32: return launch_f32_dk<32>(p, DV, s);
    case 64: return launch_f32_dk<64>(p, DV, s);
    case 128: return launch_f32_dk<128>(p, DV, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
