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
//  scan (one workgroup per 16 columns of a head and row): the sequential part.  Each
//       workgroup owns 16 columns of one head's state (the d_v columns are
//       independent recurrences): one wave runs the recurrence with the state
//       in VGPRs, two more compute the outputs; all prefetch the next chunk's
//       fragments while they compute.
//
// MFMA fragment layout (16x16x32 bf16, wave64): A (16 x 32): lane l holds row
// l%16, k = 8*(l/16)..+8; B (32 x 16): lane l holds column l%16, k =
// 8*(l/16)..+8; C (16 x 16): lane l holds column l%16, rows 4*(l/16)..+4.
// 16x16x4 fp32: A: lane l holds A[l%16][l/16]; B: B[l/16][l%16]; C as above.
//
// Fragments whose contraction index is a token index or whose row/column
// roles get swapped use a permuted k order inside each 32-wide block: element
// e of lane group q = l/16 stands for k = 4q + e (e < 4) or 16 + 4q + (e - 4),
// i.e. the rows of two stacked C tiles.  A fixed permutation of the
// contraction index does not change a product, and it lets a C-layout result
// be used as an operand with no data exchange.  Operands that need the
// transposed orientation (K^T, and V as a B operand over tokens) are made by
// multiplying the row-major tile by a 0/1 selection matrix on the MFMA, which
// is exact and lands the data in C layout, instead of 2-byte LDS transposes.
#include "gdn_internal.h"
#include "gdn_ut.h"

namespace gdn {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int CH = 64;      // chunk length
constexpr int NTHR = 256;   // 4 waves

__device__ __forceinline__ f32x4 mfma(const uint4& a, const uint4& b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// hi = bf16(a), lo = bf16(a - hi), two values at a time (packed bf16x2)
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo)
{
    hi = f32x2_to_bf16x2(a, b);
    lo = f32x2_to_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// 8 floats -> one bf16x8 fragment
__device__ __forceinline__ uint4 cvt8(const float* v)
{
    return make_uint4(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]),
                      f32x2_to_bf16x2(v[4], v[5]), f32x2_to_bf16x2(v[6], v[7]));
}

// 8 floats -> hi and lo bf16x8 fragments
__device__ __forceinline__ void split8(const float* v, uint4& hi, uint4& lo)
{
    split2(v[0], v[1], hi.x, lo.x);
    split2(v[2], v[3], hi.y, lo.y);
    split2(v[4], v[5], hi.z, lo.z);
    split2(v[6], v[7], hi.w, lo.w);
}

// Byte layout of one (layer, row, value head, chunk) record in the workspace.
template <int DK, int DV>
struct Rec {
    static constexpr int KS = DK / 32;                           // k-steps over d_k
    static constexpr size_t WT = 0;                              // W~ A-frags [4][KS][64] x 16 B (permuted d_k)
    static constexpr size_t UT = WT + 4 * KS * 64 * 16;          // U~ C-frags [4][DV/16][64] x 16 B
    static constexpr size_t PH = UT + 4 * (DV / 16) * 64 * 16;   // P hi A-frags [4][2][64] x 16 B (permuted tokens)
    static constexpr size_t PL = PH + 4 * 2 * 64 * 16;           // P lo
    static constexpr size_t KT = PL + 4 * 2 * 64 * 16;           // K^T A-frags [DK/16][2][64] x 16 B (permuted tokens)
    static constexpr size_t QA = KT + (DK / 16) * 2 * 64 * 16;   // Q A-frags [4][KS][64] x 16 B (standard d_k order)
    static constexpr size_t VEC = QA + 4 * KS * 64 * 16;         // qs[64], ks[64], gC
    static constexpr size_t BYTES = VEC + 3 * 64 * 4;
};

// 0/1 selection fragment (B operand, 32 x 16): B[k][n] = (k == n + 16 half).
__device__ __forceinline__ uint4 select_frag(int lane, int half)
{
    const int fr = lane & 15, gq = lane >> 4;
    uint32_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (8 * gq + e == fr + 16 * half) ? 0x3f80u : 0u;   // bf16 1.0
    return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
}

// Two C tiles (rows 0..15 and 16..31 of a 32-row block, one column per lane)
// -> one fragment over the permuted 32-wide k order.
__device__ __forceinline__ uint4 frag_from_c(const f32x4& lo, const f32x4& hi)
{
    const float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return cvt8(v);
}

// Raw buffer resources: the prep kernel's record stores and every load and
// store of the scan kernel go through them.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_WORD3 = 0x00020000;   // raw (stride 0) buffer, 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), RSRC_WORD3);
}
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Cache policy of the prep kernel's record stores: device scope (the SC1 bit
// of a gfx950 buffer store).  The records are written through the XCD's L2 as
// they are issued instead of sitting dirty in it until the kernel ends, when
// the whole 40 MB of a 1,024-token call (32 heads, d = 128) would be written
// back before the scan, on other XCDs, may start; the scan still finds them
// in the MALL.  Measured on that call: prep 17.9 -> 15.7 us, scan unchanged
// (20.8 - 21.1 us).  Non-temporal stores end the prep sooner still but leave
// the records in HBM only, and the scan then takes 24.5 us.
constexpr int kRecordStorePolicy = 16;

// ---------------------------------------------------------------------------
// prep kernel: one workgroup per (chunk, value head, layer*row).  Wave w owns
// token tile w (tokens 16w..16w+15 of the chunk): the columns of its K K^T
// and K Q^T products and the rows of P, U~ and W~.
template <int DK, int DV, bool CONV>
__global__ __launch_bounds__(NTHR, 2) void prefill_prep_kernel(PrefillParams p)
{
    using R = Rec<DK, DV>;
    constexpr int KS = DK / 32;
    constexpr int KP = DK + 8;   // bf16 row pitch of K rows
    constexpr int VP = DV + 8;   // bf16 row pitch of V rows
    constexpr int FP = CH + 4;   // fp32 row pitch of A and T (16-byte rows)
    // region 1: K and V rows (bf16) while loading; A and T (fp32) afterwards
    constexpr size_t R1A = static_cast<size_t>(CH) * KP * 2 + static_cast<size_t>(CH) * VP * 2;
    constexpr size_t R1B = 2 * static_cast<size_t>(CH) * FP * 4;
    __shared__ __align__(16) char r1[R1A > R1B ? R1A : R1B];
    __shared__ __align__(16) uint4 KTf[DK / 16][2][64];   // K^T A-frags (permuted tokens)
    __shared__ __align__(16) uint4 Vf[DV / 16][2][64];    // V B-frags (permuted tokens)
    constexpr int SP = 17;       // fp32 row pitch of the inverse scratch
    __shared__ float Scr[4][2][16][SP];                   // per-wave scratch for the inverse
    __shared__ __align__(16) float Gs[CH];      // cumulative decay, log2 units
    __shared__ __align__(16) float Bs[CH];
    __shared__ __align__(16) float Ink[CH];
    auto Ks = reinterpret_cast<uint16_t(*)[KP]>(r1);
    auto Vs = reinterpret_cast<uint16_t(*)[VP]>(r1 + static_cast<size_t>(CH) * KP * 2);
    float* Af = reinterpret_cast<float*>(r1);
    float* Tf = reinterpret_cast<float*>(r1) + CH * FP;

    const int c = blockIdx.x;
    const int hv = blockIdx.y;
    const int lb = blockIdx.z;
    const int NC = (p.T + CH - 1) / CH;   // record layout: the padded length
    const int t0 = c * CH;
    const int len = p.lengths ? p.lengths[lb % p.B] : p.T;
    if (len < 0 || len > p.T) return;     // reported by the scan kernel
    const int n = min(CH, len - t0);
    if (n <= 0) return;                   // past this row's prompt
    const int m = hv / (p.HV / p.HK);
    // the raw K and Q fragments are the same for every value head of qk head
    // m: only its first value head stores them
    const bool kq_owner = hv % (p.HV / p.HK) == 0;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int fr = lane & 15;          // fragment row / column
    const int gq = lane >> 4;          // lane group
    const int fk = gq * 8;             // standard k offset of A/B fragments
    const int fq = gq * 4;             // row offset of C fragments
    const size_t C = p.C;
    const bool l2 = (p.flags & FLAG_L2) != 0;
    const uint16_t* y = static_cast<const uint16_t*>(p.y);
    const size_t ybase = static_cast<size_t>(lb) * p.T + t0;   // token row of chunk start

    // ---- every global load first; rows past the chunk re-read its last row ----
    const int lr = tid >> 2;     // token row of this thread's K / V vectors
    const int sub = tid & 3;
    constexpr int NKV = DK / 32;                     // 16-byte K vectors per thread
    constexpr int NVV = (DV / 8 + 3) / 4;            // 16-byte V vectors per thread
    uint4 kv[NKV], vv[NVV], qf[KS];
    if constexpr (CONV) {
        // ---- y is the short conv (+ SiLU) of the window [conv_state ; x],
        // rounded to bf16 as the conv step writes it (conv8_token: the same
        // arithmetic).  K and V rows go straight to LDS: thread -> one group
        // of 8 channels x TRC consecutive tokens, its TRC + 3 window rows
        // loaded once.  Rows past the chunk are clamped onto its last token
        // and their results are zero. ----
        constexpr int GK = DK / 8, G = GK + DV / 8;
        constexpr int NB = NTHR / G, TRC = (CH + NB - 1) / NB;
        const bool silu = (p.flags & FLAG_SILU) != 0;
        const uint16_t* xs = static_cast<const uint16_t*>(p.x);
        const uint16_t* cst = static_cast<const uint16_t*>(p.conv_state);
        const size_t lc = static_cast<size_t>(lb / p.B) * C;   // layer's first conv channel
        // window row q of this (layer, row): conv cache row q (q < 3) or x row q - 3
        auto wrow = [&](int q, size_t ch) -> uint4 {
            return q < 3 ? *reinterpret_cast<const uint4*>(cst + (static_cast<size_t>(lb) * 3 + q) * C + ch)
                         : *reinterpret_cast<const uint4*>(xs + (static_cast<size_t>(lb) * p.T + (q - 3)) * C + ch);
        };
        auto pack8 = [](const float (&v)[8]) {
            return make_uint4(f32_to_bf16_bits(v[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[1])) << 16),
                              f32_to_bf16_bits(v[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[3])) << 16),
                              f32_to_bf16_bits(v[4]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[5])) << 16),
                              f32_to_bf16_bits(v[6]) | (static_cast<uint32_t>(f32_to_bf16_bits(v[7])) << 16));
        };
        const int g = tid % G, j0 = (tid / G) * TRC;
        if (tid < NB * G) {
            const size_t ch = g < GK ? static_cast<size_t>(p.HK + m) * DK + 8 * g
                                     : static_cast<size_t>(2 * p.HK) * DK + static_cast<size_t>(hv) * DV + 8 * (g - GK);
            uint4 raw[TRC + 3];
#pragma unroll
            for (int r = 0; r < TRC + 3; ++r) raw[r] = wrow(t0 + min(j0 + r, n + 2), ch);
            float wt4[4][8], bias[8], win[4][8];
            conv_taps8<ACT_BF16>(p.conv_w, p.conv_b, lc + ch, wt4, bias);
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const uint4 rr[1] = {raw[r]};
                to_f32x8<ACT_BF16>(rr, win[r]);
            }
#pragma unroll
            for (int k = 0; k < TRC; ++k) {
                const int i = j0 + k;
                const uint4 rr[1] = {raw[k + 3]};
                to_f32x8<ACT_BF16>(rr, win[3]);
                float yv[8];
                conv8_token(wt4, win, bias, silu, yv);
                const uint4 yb = i < n ? pack8(yv) : make_uint4(0, 0, 0, 0);
                if (i < CH) {
                    if (g < GK) *reinterpret_cast<uint4*>(&Ks[i][8 * g]) = yb;
                    else *reinterpret_cast<uint4*>(&Vs[i][8 * (g - GK)]) = yb;
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    win[0][c] = win[1][c];
                    win[1][c] = win[2][c];
                    win[2][c] = win[3][c];
                }
            }
        }
        // Q fragments of token 16 w + fr, each from its own 4 window rows
        const int tq = min(16 * w + fr, n - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const size_t ch = static_cast<size_t>(m) * DK + 32 * ks + fk;
            float wt4[4][8], bias[8], win[4][8], yv[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 rr[1] = {wrow(t0 + tq + j, ch)};
                to_f32x8<ACT_BF16>(rr, win[j]);
            }
            conv_taps8<ACT_BF16>(p.conv_w, p.conv_b, lc + ch, wt4, bias);
            conv8_token(wt4, win, bias, silu, yv);
            qf[ks] = pack8(yv);
        }
    } else {
        const size_t row = (ybase + min(lr, n - 1)) * C;
#pragma unroll
        for (int q = 0; q < NKV; ++q)
            kv[q] = *reinterpret_cast<const uint4*>(y + row + static_cast<size_t>(p.HK + m) * DK + 8 * (sub + 4 * q));
#pragma unroll
        for (int q = 0; q < NVV; ++q)
            vv[q] = *reinterpret_cast<const uint4*>(y + row + static_cast<size_t>(2 * p.HK) * DK +
                                                    static_cast<size_t>(hv) * DV + 8 * min(sub + 4 * q, DV / 8 - 1));
        const size_t qrow = (ybase + min(16 * w + fr, n - 1)) * C + static_cast<size_t>(m) * DK;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const uint4*>(y + qrow + 32 * ks + fk);
    }
    const size_t gi = (ybase + min(lane, n - 1)) * p.HV + hv;
    const float graw = load_act<ACT_BF16>(p.g, gi);
    const float braw = load_act<ACT_BF16>(p.beta, gi);

    // ---- rows into LDS, norms, gates ----
    const bool lreal = lr < n;
    float sk = 0.f;
    if constexpr (CONV) {
        lds_barrier();   // the conv wrote the K and V rows; read this thread's K vectors back
#pragma unroll
        for (int q = 0; q < NKV; ++q) kv[q] = *reinterpret_cast<const uint4*>(&Ks[lr][8 * (sub + 4 * q)]);
    }
#pragma unroll
    for (int q = 0; q < NKV; ++q) {
        if (!lreal) kv[q] = make_uint4(0, 0, 0, 0);
        if constexpr (!CONV) *reinterpret_cast<uint4*>(&Ks[lr][8 * (sub + 4 * q)]) = kv[q];
        const uint32_t kw[4] = {kv[q].x, kv[q].y, kv[q].z, kv[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a0 = __uint_as_float(kw[e] << 16), a1 = __uint_as_float(kw[e] & 0xffff0000u);
            sk = fmaf(a0, a0, sk);
            sk = fmaf(a1, a1, sk);
        }
    }
#pragma unroll
    for (int q = 0; q < NVV; ++q) {
        if constexpr (!CONV) {
            if (!lreal) vv[q] = make_uint4(0, 0, 0, 0);
            if (sub + 4 * q < DV / 8) *reinterpret_cast<uint4*>(&Vs[lr][8 * (sub + 4 * q)]) = vv[q];
        }
    }
    sk += __shfl_xor(sk, 1, 64);   // the 4 threads of a token row are consecutive lanes
    sk += __shfl_xor(sk, 2, 64);
    if (sub == 0) Ink[lr] = (l2 && lreal) ? 1.0f / sqrtf(sk + p.l2_eps) : 1.0f;
    const int r_me = 16 * w + fr;   // this lane's column token
    if (r_me >= n)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = make_uint4(0, 0, 0, 0);
    char* rec = static_cast<char*>(p.ws) + ((static_cast<size_t>(lb) * p.HV + hv) * NC + c) * R::BYTES;
    const rsrc_t rrec = make_rsrc(rec, static_cast<uint32_t>(R::BYTES));
    auto rst = [&](size_t off, const uint4& v) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rrec, static_cast<int>(off), 0, kRecordStorePolicy);
    };
    auto rstf = [&](size_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rrec, static_cast<int>(off), 0, kRecordStorePolicy);
    };
    // raw Q rows of token tile w: the A operand of the output products
    if (kq_owner)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            rst(R::QA + ((w * KS + ks) * 64 + lane) * 16, qf[ks]);
    float sq = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint32_t qw[4] = {qf[ks].x, qf[ks].y, qf[ks].z, qf[ks].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a0 = __uint_as_float(qw[e] << 16), a1 = __uint_as_float(qw[e] & 0xffff0000u);
            sq = fmaf(a0, a0, sq);
            sq = fmaf(a1, a1, sq);
        }
    }
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    const float inq_me = (l2 && r_me < n) ? 1.0f / sqrtf(sq + p.l2_eps) : 1.0f;
    if (w == 0) {
        float gv = lane < n ? graw : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {   // inclusive scan, fixed order
            const float o = __shfl_up(gv, off, 64);
            if (lane >= off) gv += o;
        }
        Gs[lane] = gv * 1.4426950408889634f;   // log2(e): decays below are exp2 of differences
        Bs[lane] = lane < n ? braw : 0.f;
    }
    lds_barrier();

    // ---- K K^T and K Q^T: rows i (all tiles), columns r (tile w) ----
    f32x4 kk[4], kq[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        kk[a] = f32x4{0.f, 0.f, 0.f, 0.f};
        kq[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint4 bk = *reinterpret_cast<const uint4*>(&Ks[16 * w + fr][32 * ks + fk]);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const uint4 ak = *reinterpret_cast<const uint4*>(&Ks[16 * a + fr][32 * ks + fk]);
            kk[a] = mfma(ak, bk, kk[a]);
            kq[a] = mfma(ak, qf[ks], kq[a]);
        }
    }
    // ---- K^T and V in token-permuted fragment order via 0/1 selection products ----
    {
        const uint4 sel0 = select_frag(lane, 0), sel1 = select_frag(lane, 1);
        for (int db = w; db < DK / 16; db += 4) {
            f32x4 d4[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const uint4 a = *reinterpret_cast<const uint4*>(&Ks[16 * tb + fr][32 * (db >> 1) + fk]);
                d4[tb] = mfma(a, (db & 1) ? sel1 : sel0, f32x4{0.f, 0.f, 0.f, 0.f});
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint4 f = frag_from_c(d4[2 * ks], d4[2 * ks + 1]);
                KTf[db][ks][lane] = f;
                if (kq_owner) rst(R::KT + ((db * 2 + ks) * 64 + lane) * 16, f);
            }
        }
        for (int nt = w; nt < DV / 16; nt += 4) {
            f32x4 d4[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                // with d_v = 16 the upper half of the 32-wide k block is the row
                // pad (never written): feed zeros, not 0 x garbage
                const uint4 a = (32 * (nt >> 1) + fk < DV)
                                    ? *reinterpret_cast<const uint4*>(&Vs[16 * tb + fr][32 * (nt >> 1) + fk])
                                    : make_uint4(0, 0, 0, 0);
                d4[tb] = mfma(a, (nt & 1) ? sel1 : sel0, f32x4{0.f, 0.f, 0.f, 0.f});
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) Vf[nt][ks][lane] = frag_from_c(d4[2 * ks], d4[2 * ks + 1]);
        }
    }
    lds_barrier();   // K and V rows are dead from here on (region 1 becomes A and T)

    // ---- A (fp32, LDS), P = scale lower_incl(E o Q^K^T) (split A-frags), per-token vectors ----
    {
        const float g_me = Gs[r_me], b_me = Bs[r_me], ink_me = Ink[r_me];
        const float sa = b_me * ink_me, sp = p.scale * inq_me;
        float pv[2][8];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            // this lane's 4 columns i = 16 a + fq + j: one vector read per table
            const f32x4 gi = *reinterpret_cast<const f32x4*>(&Gs[16 * a + fq]);
            const f32x4 ki = *reinterpret_cast<const f32x4*>(&Ink[16 * a + fq]);
            f32x4 arow;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 16 * a + fq + j;
                // exp2 of G_r - G_i <= 0 on and below the diagonal; the value
                // above it is discarded by the selects
                const float e = (i <= r_me) ? __builtin_amdgcn_exp2f(g_me - gi[j]) : 0.f;
                arow[j] = (i < r_me) ? sa * e * kk[a][j] * ki[j] : 0.f;
                pv[a >> 1][4 * (a & 1) + j] = sp * e * kq[a][j] * ki[j];
            }
            *reinterpret_cast<f32x4*>(&Af[r_me * FP + 16 * a + fq]) = arow;
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            uint4 h, l;
            split8(pv[ks], h, l);
            if (w >= 2 || ks == 0) {   // tiles 0 and 1 see only the first 32 tokens
                rst(R::PH + ((w * 2 + ks) * 64 + lane) * 16, h);
                rst(R::PL + ((w * 2 + ks) * 64 + lane) * 16, l);
            }
        }
        if (gq == 0) rstf(R::VEC + 4 * r_me, (r_me < n) ? p.scale * exp2f(g_me) * inq_me : 0.f);
        if (w == 0) {
            const float gl = Gs[n - 1];
            rstf(R::VEC + 4 * (CH + lane), (lane < n) ? exp2f(gl - Gs[lane]) * Ink[lane] : 0.f);
            rstf(R::VEC + 4 * (2 * CH + lane), exp2f(gl));
        }
        // upper blocks of T are zero: thread -> row tid / 4, columns 16 (tid % 4) ..
        {
            const int rr = tid >> 2, qb = tid & 3;
            if (qb > (rr >> 4))
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *reinterpret_cast<f32x4*>(&Tf[rr * FP + 16 * qb + 4 * e]) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    lds_barrier();   // A complete

    // ---- T = (I + A)^-1 on fp32 MFMA (diagonal blocks by the product formula,
    // then block substitution); ends with a workgroup barrier ----
    ut_inverse64<FP>(Af, Tf, Scr, w, fr, gq);

    // ---- U~ = T diag(beta) V (split T) and W~^T = K^T (T diag(beta gamma / |k|))^T ----
    // Both read row r_me of T over the permuted token order.
    uint4 t1h[2], t1l[2], t2[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(&Tf[r_me * FP + 32 * ks + fq]);
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(&Tf[r_me * FP + 32 * ks + 16 + fq]);
        const f32x4 bl = *reinterpret_cast<const f32x4*>(&Bs[32 * ks + fq]);
        const f32x4 bh = *reinterpret_cast<const f32x4*>(&Bs[32 * ks + 16 + fq]);
        const f32x4 gl = *reinterpret_cast<const f32x4*>(&Gs[32 * ks + fq]);
        const f32x4 gh = *reinterpret_cast<const f32x4*>(&Gs[32 * ks + 16 + fq]);
        const f32x4 il = *reinterpret_cast<const f32x4*>(&Ink[32 * ks + fq]);
        const f32x4 ih = *reinterpret_cast<const f32x4*>(&Ink[32 * ks + 16 + fq]);
        float v1[8], v2[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {   // tokens 32 ks + fq + e and 32 ks + 16 + fq + e
            v1[e] = a4[e] * bl[e];
            v1[4 + e] = b4[e] * bh[e];
            v2[e] = v1[e] * __builtin_amdgcn_exp2f(gl[e]) * il[e];
            v2[4 + e] = v1[4 + e] * __builtin_amdgcn_exp2f(gh[e]) * ih[e];
        }
        split8(v1, t1h[ks], t1l[ks]);
        t2[ks] = cvt8(v2);
    }
#pragma unroll
    for (int nt = 0; nt < DV / 16; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint4 bvv = Vf[nt][ks][lane];
            acc = mfma(t1h[ks], bvv, acc);
            acc = mfma(t1l[ks], bvv, acc);
        }
        rst(R::UT + ((w * (DV / 16) + nt) * 64 + lane) * 16, __builtin_bit_cast(uint4, acc));
    }
    f32x4 wt[DK / 16];
#pragma unroll
    for (int a = 0; a < DK / 16; ++a) {
        wt[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) wt[a] = mfma(KTf[a][ks][lane], t2[ks], wt[a]);
    }
    // wt[a][j] = W~[r_me][d_k = 16a + fq + j]: the permuted-d_k fragment of block a/2
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        rst(R::WT + ((w * KS + ks) * 64 + lane) * 16, frag_from_c(wt[2 * ks], wt[2 * ks + 1]));
}

// ---------------------------------------------------------------------------
// scan kernel: one workgroup of three waves per (16-column slice, value head,
// layer*row).
//  wave 0 (state wave) carries the slice of H (d_k x 16, fp32, C layout) in
//    VGPRs and runs the recurrence: U = U~ - W~ H, S = diag(s) U,
//    H' = gC H + K^T S.  Because W~, K^T and the S operand use the permuted
//    k order, every operand it needs is built from its own C-layout
//    registers: no LDS and no barrier on the recurrence chain.
//  waves 1 and 2 (output waves) compute O = diag(qs) Q H + P U for two of
//    the four 16-token tiles each, tiles {0, 3} and {1, 2}: P is lower
//    triangular, so tiles 0 and 1 need only the first 32 tokens of U and
//    the two pairs carry equal work.  They take the fp32 H and U the state
//    wave publishes in a two-slot LDS ring and split them into bf16 hi/lo
//    operands themselves.
// One barrier per chunk hands a ring slot from the state wave to the output
// waves; they finish reading slot c%2 before they reach the next barrier,
// after which the state wave may overwrite it.  The barrier orders LDS only,
// so the prefetches issued just before it stay in flight across it.
//
// Every load and store goes through a buffer resource whose base moves with
// the chunk, so a per-access address is a lane-constant VGPR plus constants
// (no 64-bit address arithmetic per load).  All operands come from the chunk
// record in fragment order (1 KB contiguous per wave load).  For the output
// the row index sits in the VGPR offset and the resource's byte range ends
// inside the last valid token row, so in the tail chunk the stores of rows
// past the prompt are dropped by the range check.

__device__ __forceinline__ uint4 bload16(rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ f32x4 as_f4(const uint4& v)
{
    return __builtin_bit_cast(f32x4, v);
}

// W~ is single-buffered: it is consumed by the first products of a chunk and
// reloaded for the next chunk right after them.  K^T, U~ and the scalings are
// double-buffered (K^T is consumed at the end of the chunk).
template <int DK>
struct WFrags {
    uint4 wt[4][DK / 32];   // W~ rows (4 token tiles, permuted d_k)
};
template <int DK, int DV>
struct KFrags {
    uint4 kt[DK / 16][2];   // K^T rows (d_k tiles, permuted tokens)
    uint4 ut[4];            // U~ tiles of this column slice (fp32 C layout)
    uint4 ks[4];            // update scalings of the token rows (fp32)
    float gC;               // chunk decay
};

template <int DK, int DV>
__device__ __forceinline__ void w_load(WFrags<DK>& f, rsrc_t r, int lane16)
{
    using R = Rec<DK, DV>;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int ks = 0; ks < R::KS; ++ks) f.wt[tb][ks] = bload16(r, lane16, R::WT + (tb * R::KS + ks) * 1024);
}

template <int DK, int DV>
__device__ __forceinline__ void k_load(KFrags<DK, DV>& f, rsrc_t r, rsrc_t rk, int lane16, int vq16, int cs)
{
    using R = Rec<DK, DV>;
    // in the order the chunk uses them (the compiler starts the chunk with
    // the decay's multiply of H, and loads complete in order): the decay, U~,
    // the scalings, then K^T (1,024-token call: 37.6 -> 36.6 us on one box)
    f.gC = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 0, R::VEC + 2 * CH * 4, 0));
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) f.ut[tb] = bload16(r, lane16, R::UT + (tb * (DV / 16) + cs) * 1024);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) f.ks[tb] = bload16(r, vq16, R::VEC + (CH + 16 * tb) * 4);
#pragma unroll
    for (int a = 0; a < DK / 16; ++a)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) f.kt[a][ks] = bload16(rk, lane16, R::KT + (a * 2 + ks) * 1024);
}

template <int DK>
struct Ring {
    f32x4 h[2][DK / 16][64];   // H at the start of the chunk (C tiles), two slots
    f32x4 u[2][4][64];         // U of the chunk (C tiles)
};

template <int DK, int DV>
__device__ __forceinline__ void state_chunk(WFrags<DK>& wf, const KFrags<DK, DV>& f, rsrc_t rnext,
                                            f32x4 (&h)[DK / 16], Ring<DK>& ring, int c, int lane)
{
    constexpr int KS = DK / 32, NA = DK / 16;
    const int slot = c & 1;
    // publish H; its bf16 rounding is the B operand of W~ H
    uint4 hh[KS];
#pragma unroll
    for (int a = 0; a < NA; ++a) ring.h[slot][a][lane] = h[a];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) hh[ks] = frag_from_c(h[2 * ks], h[2 * ks + 1]);
    // P = W~ H
    f32x4 acc[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc[tb] = mfma(wf.wt[tb][ks], hh[ks], acc[tb]);
    }
    w_load<DK, DV>(wf, rnext, lane * 16);   // W~ of the next chunk
    // U = U~ - W~ H, published; S = diag(s) U split into hi + lo
    f32x4 sv[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const f32x4 u = as_f4(f.ut[tb]) - acc[tb];
        ring.u[slot][tb][lane] = u;
        sv[tb] = as_f4(f.ks[tb]) * u;
    }
    uint4 sh[2], sl[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const float v[8] = {sv[2 * ks][0], sv[2 * ks][1], sv[2 * ks][2], sv[2 * ks][3],
                            sv[2 * ks + 1][0], sv[2 * ks + 1][1], sv[2 * ks + 1][2], sv[2 * ks + 1][3]};
        split8(v, sh[ks], sl[ks]);
    }
    // H' = gC H + K^T S
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        f32x4 acc2 = f.gC * h[a];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            acc2 = mfma(f.kt[a][ks], sh[ks], acc2);
            acc2 = mfma(f.kt[a][ks], sl[ks], acc2);
        }
        h[a] = acc2;
    }
}

// the k-steps of P U that can be nonzero for token tile tb (P is lower triangular)
constexpr int pu_steps(int tb) { return tb >= 2 ? 2 : 1; }

template <int DK, int DV>
struct OutFrags {
    static constexpr int KS = DK / 32;
    uint4 q[2][KS];             // raw Q rows of the two tiles (standard d_k order)
    uint4 ph[2][2], pl[2][2];   // P rows (permuted tokens), hi and lo
    uint4 qs[2];                // output scalings of the token rows (fp32)
};

template <int DK, int DV, int TA, int TB>
__device__ __forceinline__ void out_load(OutFrags<DK, DV>& f, rsrc_t rrec, rsrc_t rq, int lane16, int vq16)
{
    using R = Rec<DK, DV>;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tb = i ? TB : TA;
#pragma unroll
        for (int ks = 0; ks < R::KS; ++ks) f.q[i][ks] = bload16(rq, lane16, R::QA + (tb * R::KS + ks) * 1024);
#pragma unroll
        for (int ks = 0; ks < pu_steps(tb); ++ks) {
            f.ph[i][ks] = bload16(rrec, lane16, R::PH + (tb * 2 + ks) * 1024);
            f.pl[i][ks] = bload16(rrec, lane16, R::PL + (tb * 2 + ks) * 1024);
        }
        f.qs[i] = bload16(rrec, vq16, R::VEC + 16 * tb * 4);
    }
}

template <int DK, int DV, int OUT, int TA, int TB>
__device__ __forceinline__ void out_chunk(const OutFrags<DK, DV>& f, const Ring<DK>& ring, int c, rsrc_t ro,
                                          const int (&vo)[2][4], int coff, int lane)
{
    constexpr int KS = DK / 32;
    const int slot = c & 1;
    uint4 hh[KS], hl[KS], uh[2], ul[2];
    // H rows 32 ks + 8 gq + (0..7) of column fr, the standard k order of Q's
    // A fragments: rows 4 of C tile 2 ks + gq / 2 held by two lanes of the ring
    const int gq = lane >> 4, fr = lane & 15;
    const int l0 = 32 * (gq & 1) + fr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const f32x4 a = ring.h[slot][2 * ks + (gq >> 1)][l0], b = ring.h[slot][2 * ks + (gq >> 1)][l0 + 16];
        const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        split8(v, hh[ks], hl[ks]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const f32x4 a = ring.u[slot][2 * ks][lane], b = ring.u[slot][2 * ks + 1][lane];
        const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        split8(v, uh[ks], ul[ks]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tb = i ? TB : TA;
        f32x4 qa = {0.f, 0.f, 0.f, 0.f}, qb = {0.f, 0.f, 0.f, 0.f}, pu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qa = mfma(f.q[i][ks], hh[ks], qa);
            qb = mfma(f.q[i][ks], hl[ks], qb);
        }
#pragma unroll
        for (int ks = 0; ks < pu_steps(tb); ++ks) {
            pu = mfma(f.ph[i][ks], uh[ks], pu);
            pu = mfma(f.ph[i][ks], ul[ks], pu);
            pu = mfma(f.pl[i][ks], uh[ks], pu);
        }
        const f32x4 o = as_f4(f.qs[i]) * (qa + qb) + pu;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (OUT == ACT_BF16)
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(o[j]), ro, vo[i][j] + coff, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[j]), ro, vo[i][j] + coff, 0, 0);
        }
    }
}

// resources of chunk c: its workspace record and its output rows
struct ChunkRes {
    rsrc_t rec, kq, o;   // own record, the qk head's K/Q fragments, output rows
};

template <int DK, int DV, int OUT>
__device__ __forceinline__ ChunkRes chunk_res(const PrefillParams& p, const char* recs, const char* recs_kq, int c,
                                              int len, int lb, int hv)
{
    using R = Rec<DK, DV>;
    constexpr int OSZ = OUT == ACT_BF16 ? 2 : 4;
    const int t0 = c * CH;
    const int n = min(CH, len - t0);   // >= 1: c is a chunk of this row's prompt
    ChunkRes r;
    r.rec = make_rsrc(recs + static_cast<size_t>(c) * R::BYTES, static_cast<uint32_t>(R::BYTES));
    r.kq = make_rsrc(recs_kq + static_cast<size_t>(c) * R::BYTES, static_cast<uint32_t>(R::BYTES));
    const size_t row0 = static_cast<size_t>(lb) * p.T + t0;
    r.o = make_rsrc(static_cast<const char*>(p.o) + ((row0 * p.HV + hv) * DV) * OSZ,
                    static_cast<uint32_t>(((n - 1) * p.HV + 1) * DV * OSZ));
    return r;
}

// Output wave of a workgroup carrying SL column slices (16 SL columns from
// column 16 SL cs): the Q, P and scaling operands are the same for every
// slice of the head, so they are loaded once and used SL times.
template <int DK, int DV, int OUT, int TA, int TB, int SL>
__device__ __forceinline__ void out_wave(const PrefillParams& p, Ring<DK> (&ring)[SL], const char* recs,
                                         const char* recs_kq, int NC, int len, int lb, int hv, int cs, int lane)
{
    constexpr int OSZ = OUT == ACT_BF16 ? 2 : 4;
    const int fr = lane & 15, gq = lane >> 4;
    const int lane16 = lane * 16, vq16 = gq * 16;
    int vo[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tb = i ? TB : TA;
#pragma unroll
        for (int j = 0; j < 4; ++j) vo[i][j] = ((16 * tb + 4 * gq + j) * p.HV * DV + 16 * SL * cs + fr) * OSZ;
    }
    auto chunk_out = [&](const OutFrags<DK, DV>& f, int cc, rsrc_t ro) {
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) out_chunk<DK, DV, OUT, TA, TB>(f, ring[sl], cc, ro, vo, 16 * sl * OSZ, lane);
    };
    OutFrags<DK, DV> fa, fb;
    ChunkRes ra = chunk_res<DK, DV, OUT>(p, recs, recs_kq, 0, len, lb, hv), rb;
    out_load<DK, DV, TA, TB>(fa, ra.rec, ra.kq, lane16, vq16);
    int c = 0;
    for (; c + 2 <= NC; c += 2) {
        rb = chunk_res<DK, DV, OUT>(p, recs, recs_kq, c + 1, len, lb, hv);
        out_load<DK, DV, TA, TB>(fb, rb.rec, rb.kq, lane16, vq16);
        lds_barrier();
        chunk_out(fa, c, ra.o);
        const int c2 = min(c + 2, NC - 1);
        ra = chunk_res<DK, DV, OUT>(p, recs, recs_kq, c2, len, lb, hv);
        out_load<DK, DV, TA, TB>(fa, ra.rec, ra.kq, lane16, vq16);
        lds_barrier();
        chunk_out(fb, c + 1, rb.o);
    }
    if (c < NC) {
        lds_barrier();
        chunk_out(fa, c, ra.o);
    }
}

// Fused conv: the conv cache of row lb becomes window rows T .. T+2 of
// [conv_state ; x], as the conv step commits it.  The prep kernel, which read
// the old cache, has finished before this kernel starts.  This workgroup's
// share: the v channels of its column slices of value head hv and, in the
// workgroups of the qk head's first value head, a strided part of the q and k
// channels of qk head m; thread i of the two output waves takes every 128th
// channel of that share, reading its three source rows before writing them
// (for T < 3 some sources are cache rows further down).
template <int DK, int DV, int SL>
__device__ __forceinline__ void conv_commit(const PrefillParams& p, int lb, int m, int hv, int gsz, int cs, int i)
{
    constexpr int NSW = DV / 16 / SL;    // workgroups per value head
    constexpr int NQK = (2 * DK + NSW - 1) / NSW;   // q/k channels per workgroup (at most)
    const size_t C = p.C;
    uint16_t* cst = static_cast<uint16_t*>(p.conv_state);
    const uint16_t* xs = static_cast<const uint16_t*>(p.x);
    const bool first = hv == m * gsz;
    const int nv = 16 * SL, nt = nv + (first ? NQK : 0);
    for (int e = i; e < nt; e += 128) {
        size_t ch;
        if (e < nv) {
            ch = 2 * static_cast<size_t>(p.HK) * DK + static_cast<size_t>(hv) * DV + 16 * SL * cs + e;
        } else {
            const int k = cs + NSW * (e - nv);   // q (k < DK) or k (DK <= k < 2 DK) channel of head m
            if (k >= 2 * DK) continue;
            ch = k < DK ? static_cast<size_t>(m) * DK + k : static_cast<size_t>(p.HK) * DK + m * DK + (k - DK);
        }
        uint16_t v[3];
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int q = p.T + r;   // window row that becomes cache row r
            v[r] = q < 3 ? cst[(static_cast<size_t>(lb) * 3 + q) * C + ch]
                         : xs[(static_cast<size_t>(lb) * p.T + (q - 3)) * C + ch];
        }
#pragma unroll
        for (int r = 0; r < 3; ++r) cst[(static_cast<size_t>(lb) * 3 + r) * C + ch] = v[r];
    }
}

template <int DK, int DV, int OUT, int SL, bool CONV>
__global__ __launch_bounds__(64 * (SL + 2)) void prefill_scan_kernel(PrefillParams p)
{
    using R = Rec<DK, DV>;
    static_assert(SL >= 1 && (DV / 16) % SL == 0, "a workgroup's slices must divide d_v");
    __shared__ __align__(16) Ring<DK> ring[SL];

    // ---- block -> (layer*row, qk head, value head, column slice), XCD-aware:
    // workgroups go round-robin over the 8 XCDs, so the index is remapped to
    // put every slice of the value heads of one qk head on one XCD, where
    // they share the chunk records and q rows through its L2.
    constexpr int NS = DV / 16 / SL;   // workgroups per value head
    const int gsz = p.HV / p.HK;
    const int per_group = gsz * NS;
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int sg = bid >> 3;
    const int r_in = sg % per_group;
    const int grp = (sg / per_group) * 8 + xcd;
    if (grp >= p.L * p.B * p.HK) return;
    const int m = grp % p.HK;
    const int lb = grp / p.HK;
    const int hv = m * gsz + r_in / NS;
    const int cs = r_in % NS;
    const int NC = (p.T + CH - 1) / CH;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform role

    const int slot = p.cur ? p.cur[lb] : 0;
    const int len = p.lengths ? p.lengths[lb % p.B] : p.T;
    {
        const int e = (slot < 0 || slot >= p.S ? ERR_SLOT : 0) | (len < 0 || len > p.T ? ERR_LENGTH : 0);
        if (e) {
            if (threadIdx.x == 0 && cs == 0 && hv == m * gsz && p.err) atomicOr(p.err, e);
            return;
        }
    }
    if (len == 0) return;
    const char* recs = static_cast<const char*>(p.ws) + (static_cast<size_t>(lb) * p.HV + hv) * NC * R::BYTES;
    // K^T and Q fragments live in the records of the qk head's first value head
    const char* recs_kq = static_cast<const char*>(p.ws) + (static_cast<size_t>(lb) * p.HV + m * gsz) * NC * R::BYTES;
    const int NCr = (len + CH - 1) / CH;   // chunks of this row's prompt

    if (w < SL) {
        // ---- state wave of column slice SL cs + w ----
        const int sc = SL * cs + w;
        const int fr = lane & 15, fq = (lane >> 4) * 4;
        const int lane16 = lane * 16, vq16 = (lane >> 4) * 16;
        const int col = 16 * sc + fr;
        float* st = p.state + ((static_cast<size_t>(lb) * p.S + slot) * p.HV + hv) * DK * DV;
        f32x4 h[DK / 16];
#pragma unroll
        for (int a = 0; a < DK / 16; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j) h[a][j] = st[(16 * a + fq + j) * DV + col];
        auto rec_rsrc = [&](int cc) {
            return make_rsrc(recs + static_cast<size_t>(min(cc, NCr - 1)) * R::BYTES, static_cast<uint32_t>(R::BYTES));
        };
        auto kq_rsrc = [&](int cc) {
            return make_rsrc(recs_kq + static_cast<size_t>(min(cc, NCr - 1)) * R::BYTES,
                             static_cast<uint32_t>(R::BYTES));
        };
        WFrags<DK> wf;
        KFrags<DK, DV> fa, fb;
        w_load<DK, DV>(wf, rec_rsrc(0), lane16);
        k_load<DK, DV>(fa, rec_rsrc(0), kq_rsrc(0), lane16, vq16, sc);
        int c = 0;
        for (; c + 2 <= NCr; c += 2) {
            k_load<DK, DV>(fb, rec_rsrc(c + 1), kq_rsrc(c + 1), lane16, vq16, sc);
            state_chunk<DK, DV>(wf, fa, rec_rsrc(c + 1), h, ring[w], c, lane);
            lds_barrier();
            k_load<DK, DV>(fa, rec_rsrc(c + 2), kq_rsrc(c + 2), lane16, vq16, sc);
            state_chunk<DK, DV>(wf, fb, rec_rsrc(c + 2), h, ring[w], c + 1, lane);
            lds_barrier();
        }
        if (c < NCr) {
            state_chunk<DK, DV>(wf, fa, rec_rsrc(c), h, ring[w], c, lane);
            lds_barrier();
        }
#pragma unroll
        for (int a = 0; a < DK / 16; ++a)
#pragma unroll
            for (int j = 0; j < 4; ++j) st[(16 * a + fq + j) * DV + col] = h[a][j];
    } else {
        if constexpr (CONV) conv_commit<DK, DV, SL>(p, lb, m, hv, gsz, cs, (w - SL) * 64 + lane);
        if (w == SL) out_wave<DK, DV, OUT, 0, 3, SL>(p, ring, recs, recs_kq, NCr, len, lb, hv, cs, lane);
        else out_wave<DK, DV, OUT, 1, 2, SL>(p, ring, recs, recs_kq, NCr, len, lb, hv, cs, lane);
    }
}

// The scan instantiations: output dtype x slices per workgroup x fused conv
// (whose cache commit is compiled only where it is used).
template <int DK, int DV, bool CONV>
void launch_scan(const PrefillParams& p, dim3 grid, bool two, hipStream_t s)
{
    if constexpr (DV >= 32) {
        if (two) {
            if (p.out == ACT_BF16)
                hipLaunchKernelGGL((prefill_scan_kernel<DK, DV, ACT_BF16, 2, CONV>), grid, dim3(256), 0, s, p);
            else
                hipLaunchKernelGGL((prefill_scan_kernel<DK, DV, ACT_F32, 2, CONV>), grid, dim3(256), 0, s, p);
            return;
        }
    }
    if (p.out == ACT_BF16) hipLaunchKernelGGL((prefill_scan_kernel<DK, DV, ACT_BF16, 1, CONV>), grid, dim3(192), 0, s, p);
    else hipLaunchKernelGGL((prefill_scan_kernel<DK, DV, ACT_F32, 1, CONV>), grid, dim3(192), 0, s, p);
}

template <int DK, int DV>
hipError_t launch_pf(const PrefillParams& p, hipStream_t s)
{
    const int NC = (p.T + CH - 1) / CH;
    const long long rows = static_cast<long long>(p.L) * p.B;
    if (NC > 0x7fffffff || p.HV > 65535 || rows > 65535) return hipErrorInvalidConfiguration;
    clear_stale_error();
    if (p.x)
        hipLaunchKernelGGL((prefill_prep_kernel<DK, DV, true>), dim3(NC, p.HV, static_cast<unsigned>(rows)),
                           dim3(NTHR), 0, s, p);
    else
        hipLaunchKernelGGL((prefill_prep_kernel<DK, DV, false>), dim3(NC, p.HV, static_cast<unsigned>(rows)),
                           dim3(NTHR), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // One 16-column slice per workgroup, or two slices of a head per
    // workgroup whose output waves serve both.  A scan workgroup uses 412
    // VGPRs per lane in its state wave, so a CU holds one at a time and a grid
    // runs in rounds of CU-count workgroups.  A two-slice round costs about
    // 1.4-1.75 one-slice rounds (1,024-token calls at 32 heads, d = 128: B = 2
    // 63.8 against 67.8 us, B = 3 101-103 against 96.4 us, B = 4 120 against
    // 129 us, B = 8 257-262 against 305 us, two against one slice), so two
    // slices are taken when 5 r2 < 3 r1 for r1, r2 the rounds of the two grids.
    const long long groups = rows * p.HK;
    const long long blocks1 = (groups + 7) / 8 * 8 * (p.HV / p.HK) * (DV / 16);
    const int cus = device_cus();
    const long long r1 = cus > 0 ? (blocks1 + cus - 1) / cus : 0;
    const long long r2 = cus > 0 ? (blocks1 / 2 + cus - 1) / cus : 0;
    const bool two = DV >= 32 && cus > 0 && 5 * r2 < 3 * r1;
    const long long blocks = two ? blocks1 / 2 : blocks1;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (p.x) launch_scan<DK, DV, true>(p, grid, two, s);
    else launch_scan<DK, DV, false>(p, grid, two, s);
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

// The bf16 MFMA kernels serve bf16 activations with d_k >= 32; fp32
// activations and d_k = 16 take the fp32 kernel (gdn_prefill_f32.hip).
static bool bf16_path(int DK, int act) { return act == ACT_BF16 && DK >= 32; }

bool prefill_supported(int DK, int DV, int act)
{
    return (act == ACT_BF16 || act == ACT_F32) && (DK == 16 || DK == 32 || DK == 64 || DK == 128) &&
           (DV == 16 || DV == 32 || DV == 64 || DV == 128);
}

// The fused conv runs inside the bf16 prep kernel only.
bool prefill_conv_supported(int DK, int DV, int act)
{
    return prefill_supported(DK, DV, act) && bf16_path(DK, act);
}

size_t prefill_workspace_bytes(int L, int B, int T, int HV, int DK, int DV, int act, int chunk)
{
    if (chunk != CH) return 0;
    if (!bf16_path(DK, act)) return 0;   // the fp32 kernel keeps everything in LDS
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
    if (!bf16_path(DK, p.act)) return p.x ? hipErrorInvalidValue : launch_prefill_f32(p, DK, DV, s);
    switch (DK) {
    case 32: return launch_pf_dv<32>(p, DV, s);
    case 64: return launch_pf_dv<64>(p, DV, s);
    case 128: return launch_pf_dv<128>(p, DV, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
