// gdn_recurrent.hip -- verify and rewind: fused short conv + SiLU + q/k L2
// norm + T (<= 4) steps of the gated delta rule, one 64-lane wavefront per
// (layer, row, value head, 32-column slice of the d_v axis).
//
// Method: "perf(qwen): full-context MTP draft prefill and replay-free rewind"
// (Whallm PR #14), Summary item 4 -- rerun only the Gated DeltaNet mixer on
// the captured verification inputs from the pre-verification state;
// "Add request-owned eight-way MTP serving for Qwen 35B" (MTPLX PR #245),
// What was broken items 2, 4, 6 -- B8/T2 verification, keep in {0,1,2},
// keep=0 keeps the snapshot, rows are separable.  Update rule: gated delta
// rule, S_t = a S_{t-1}(I - b k k^T) + b v k^T, o_t = S_t q_t, stored as
// h = S^T (h[i][j], i over d_k, j over d_v contiguous).
//
// Why this shape on CDNA4: each (row, head) state is 64 KiB of fp32 that is
// touched for only 3 * 2 * 128 * 128 flops per token, so the kernel is
// bound by HBM.  The d_v columns of the state are independent recurrences
// (column j only needs column j of h and v_j; k, q, a, b are shared), so a
// head is cut into column slices with no communication between waves.
// Inside a wave, lane (ig, j4) holds a float4 of 4 consecutive columns for
// rows i = ig + IG*r: one load instruction covers IG rows x 128 contiguous
// bytes, the whole slice is loaded once and kept in VGPRs across the T steps,
// and the d_k reductions are in-lane sums plus a log2(IG)-level xor-shuffle
// butterfly (every lane ends with bit-identical sums).  The two reductions
// of a step (h^T k and h^T q) are taken together on the pre-update state and
// the output uses o = scale*(a*(h^T q) + u*(k.q)), which equals
// scale*h_t^T q algebraically.  The reduction tree does not depend on B, T,
// the mode or the slot, so B8 == 8 x B1, prefix windows and rewind ==
// candidate hold bit for bit.
//
// Workgroups are dispatched round-robin over the 8 XCDs; the block index is
// remapped so that all waves of one (layer, row, qk head) -- which read the
// same q/k conv channels -- land on the same XCD and share its L2.
#include <atomic>

#include "gdn_internal.h"

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));

template <int IG, int JL>
__device__ __forceinline__ float sum_over_rows(float v)
{
#pragma unroll
    for (int off = JL; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// One of four values chosen by a wave-uniform index (clamped to 0..3), so
// that register arrays are never indexed dynamically.
__device__ __forceinline__ float pick4(const float (&v)[4], int i)
{
    return i <= 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

// LAZY: the fused commit-then-verify of one decode cycle ("MTP inference:
// review and commit structure" (eole docs), Functional commits item 2 and
// Verification and limits: commits replay only the accepted prefix).  The
// wave replays the previous window's keep tokens from the snapshot, writes
// the committed state in place, and runs the new window on from there,
// writing outputs but no candidates.  Its token sequence is
// Z = [conv cache ; previous x[0..keep) ; new x[0..T)], so the committed conv
// cache (rows keep..keep+2 of the previous window) is simply rows keep..keep+2
// of Z and one conv pass covers both windows.
//
// NORM: the gated RMSNorm that follows the mixer ("MTP inference: review and
// commit structure" (eole docs), Functional commits item 4) is applied to
// every output before it is stored, y[j] = o[j] / sqrt(mean_j(o^2) + eps) *
// w[l][j] * SiLU(z[j]), so the raw o never goes to memory.  The mean runs over
// all d_v columns of a head, so one workgroup holds the NS column-slice waves
// of a head (wave w = slice w) and adds their partial sums of squares through
// LDS, one barrier per output token.
template <int DV>
constexpr int waves_per_head()
{
    return DV / (DV < 32 ? DV : 32);
}

template <int DK, int DV, int ACT, bool LAZY, bool NORM>
__global__ __launch_bounds__(NORM ? 64 * waves_per_head<DV>() : 64) void recurrent_kernel(RecParams p)
{
    constexpr int SW = DV < 32 ? DV : 32;  // columns per wave
    constexpr int NS = DV / SW;            // column slices per head
    constexpr int JL = SW / 4;             // lanes across one row segment
    constexpr int IG = 64 / JL;            // row groups per wave
    constexpr int RPL = DK / IG;           // rows held per lane
    constexpr int MAXT = LAZY ? 8 : 4;     // tokens one wave runs
    constexpr int NW = NORM ? NS : 1;      // waves per workgroup
    // conv channels of the workgroup: q and k of the qk head, then the v
    // channels of its one slice, or (NORM) of all NS slices, whose waves share
    // the q and k conv
    constexpr int NCH = 2 * DK + (NORM ? DV : SW);
    static_assert(RPL >= 1 && DK % IG == 0, "tile shape");

    __shared__ float ys[MAXT][NCH];
    __shared__ float ssq[NORM ? MAXT : 1][NW];   // per-slice sums of o^2 (NORM)
    __shared__ float gzw[NW][NORM ? 4 : 1][NORM ? SW : 1];   // w[j] * SiLU(z[t][j]) (NORM)

    // ---- block -> (layer, row, qk head, value head, slice), XCD-aware ----
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int sgrp = bid >> 3;
    const int r_in = sgrp % p.per_group;
    const int grp = (sgrp / p.per_group) * 8 + xcd;
    if (grp >= p.groups) return;
    const int m = grp % p.HK;
    const int lb = grp / p.HK;  // l * B + b
    const int b = lb % p.B;
    const int gsz = p.HV / p.HK;
    const int wid = NORM ? static_cast<int>(threadIdx.x >> 6) : 0;
    const int slice = NORM ? wid : r_in % NS;
    const int hv = NORM ? m * gsz + r_in : m * gsz + r_in / NS;

    const int lane = NORM ? static_cast<int>(threadIdx.x & 63) : static_cast<int>(threadIdx.x);
    const int j4 = lane % JL;
    const int ig = lane / JL;
    const int col0 = slice * SW + j4 * 4;

    // ---- row status ----
    int slot0 = 0, is_active = 1, kp = 0;
    if (p.cur) slot0 = p.cur[lb];
    if (p.active) is_active = p.active[b];
    if (p.keep) kp = p.keep[b];
    int nsteps = p.T;
    if constexpr (LAZY) {
        int e = 0;
        if (kp < 0 || kp > p.T) e |= ERR_KEEP;
        if (slot0 < 0 || slot0 >= p.S) e |= ERR_SLOT;
        if (e) {
            if (lane == 0 && p.err) atomicOr(p.err, e);
            return;
        }
        if (is_active == 0 && kp == 0) return;
        nsteps = kp + (is_active ? p.T : 0);
    } else if (p.mode == REC_VERIFY) {
        if (is_active == 0) return;
        if (slot0 < 0 || slot0 >= p.S) {
            if (lane == 0 && p.err) atomicOr(p.err, ERR_SLOT);
            return;
        }
    } else {
        int e = 0;
        if (kp < 0 || kp > p.T) e |= ERR_KEEP;
        if (slot0 < 0 || slot0 >= p.S) e |= ERR_SLOT;
        if (e) {
            if (lane == 0 && p.err) atomicOr(p.err, e);
            return;
        }
        if (kp == 0) return;
        nsteps = kp;
    }

    // ---- conv inputs: q and k channels of qk head m, v channels of the slice.
    // Every load is unconditional (lanes past the last channel re-read it,
    // rows past the window re-read its last row, a missing bias reads a
    // weight and discards it) so that they are all in flight together.
    const int C = p.C;
    const int l = lb / p.B;
    const size_t xrow = static_cast<size_t>(lb) * p.T;        // x row of token 0
    const size_t srow = static_cast<size_t>(lb) * 3;          // conv_state row 0
    const bool has_bias = p.conv_b != nullptr;
    const void* bptr = has_bias ? p.conv_b : p.conv_w;
    constexpr int NG = (NCH + 64 * NW - 1) / (64 * NW);   // channel groups per wave
    // channel of group n in this lane: lane + 64 * (wid + NW * n)
    const int vcol = NORM ? 0 : slice * SW;   // first v column of the channel set
    constexpr int NROW = MAXT + 3;   // window rows per channel
    float wv[NG][4];
    float win[NG][NROW];
    float bias[NG];
#pragma unroll
    for (int n = 0; n < NG; ++n) {
        const int ch = min(lane + 64 * (wid + NW * n), NCH - 1);
        const int c = ch < DK ? m * DK + ch
                    : (ch < 2 * DK ? p.HK * DK + m * DK + (ch - DK)
                                   : 2 * p.HK * DK + hv * DV + vcol + (ch - 2 * DK));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            wv[n][j] = load_act<ACT>(p.conv_w, (static_cast<size_t>(l) * C + c) * 4 + j);
#pragma unroll
        for (int r = 0; r < 3; ++r)
            win[n][r] = load_act<ACT>(p.conv_state, (srow + r) * C + c);
        if constexpr (LAZY) {
            float xp[4], xn[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                xp[t] = load_act<ACT>(p.x_prev, (xrow + min(t, p.T - 1)) * C + c);
                xn[t] = load_act<ACT>(p.x, (xrow + min(t, p.T - 1)) * C + c);
            }
#pragma unroll
            for (int j = 0; j < MAXT; ++j) win[n][3 + j] = j < kp ? xp[j < 4 ? j : 3] : pick4(xn, j - kp);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                win[n][3 + t] = load_act<ACT>(p.x, (xrow + min(t, p.T - 1)) * C + c);
        }
        const float bv = load_act<ACT>(bptr, has_bias ? static_cast<size_t>(l) * C + c : 0);
        bias[n] = has_bias ? bv : 0.0f;
    }
    // Gates of every window token (rows past the window re-read the last one).
    const size_t ghead = xrow * p.HV + hv;  // g/beta index of token 0
    float gate_a[MAXT], gate_b[MAXT];
    if constexpr (LAZY) {
        float gp[4], bp[4], gn[4], bn[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const size_t gi = ghead + static_cast<size_t>(min(t, p.T - 1)) * p.HV;
            gp[t] = load_act<ACT>(p.g_prev, gi);
            bp[t] = load_act<ACT>(p.beta_prev, gi);
            gn[t] = load_act<ACT>(p.g, gi);
            bn[t] = load_act<ACT>(p.beta, gi);
        }
#pragma unroll
        for (int j = 0; j < MAXT; ++j) {
            gate_a[j] = j < kp ? gp[j < 4 ? j : 3] : pick4(gn, j - kp);
            gate_b[j] = j < kp ? bp[j < 4 ? j : 3] : pick4(bn, j - kp);
        }
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const size_t gi = ghead + static_cast<size_t>(min(t, p.T - 1)) * p.HV;
            gate_a[t] = load_act<ACT>(p.g, gi);
            gate_b[t] = load_act<ACT>(p.beta, gi);
        }
    }

    // ---- gated-norm operands of this lane's 4 columns (NORM); they are folded
    // into w * SiLU(z) in LDS with the conv, so no register holds them
    // through the recurrence ----
    float zv[4][4], nw[4];
    if constexpr (NORM) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                zv[t][c] = load_act<ACT>(p.z, ((xrow + min(t, p.T - 1)) * p.HV + hv) * DV + col0 + c);
#pragma unroll
        for (int c = 0; c < 4; ++c) nw[c] = load_act<ACT>(p.norm_w, static_cast<size_t>(l) * DV + col0 + c);
    }

    // ---- the state slice: every load issued before any use ----
    const size_t tile = static_cast<size_t>(DK) * DV;
    float* st_lb = p.state + static_cast<size_t>(lb) * p.S * p.HV * tile;
    const float* src = st_lb + (static_cast<size_t>(slot0) * p.HV + hv) * tile + col0;
    f4 h[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r)
        h[r] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(src + (ig + IG * r) * DV));

    // ---- conv + SiLU for every window token, into LDS ----
    const bool use_silu = (p.flags & FLAG_SILU) != 0;
#pragma unroll
    for (int n = 0; n < NG; ++n) {
        const int ch = lane + 64 * (wid + NW * n);
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            float acc = wv[n][0] * win[n][t];
            acc = fmaf(wv[n][1], win[n][t + 1], acc);
            acc = fmaf(wv[n][2], win[n][t + 2], acc);
            acc = fmaf(wv[n][3], win[n][t + 3], acc);
            acc += bias[n];
            const float sv = silu(acc);
            if (ch < NCH && t < nsteps) ys[t][ch] = use_silu ? sv : acc;
        }
    }
    if constexpr (NORM) {
        if (ig == 0)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int c = 0; c < 4; ++c) gzw[wid][t][j4 * 4 + c] = nw[c] * silu(zv[t][c]);
    }
    lds_barrier();

    const bool l2 = (p.flags & FLAG_L2) != 0;
    for (int t = 0; t < nsteps; ++t) {
        float kr[RPL], qr[RPL];
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            qr[r] = ys[t][ig + IG * r];
            kr[r] = ys[t][DK + ig + IG * r];
        }
        float pp[4] = {0.f, 0.f, 0.f, 0.f}, rr[4] = {0.f, 0.f, 0.f, 0.f};
        float sq = 0.f, sk = 0.f, kq = 0.f;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pp[c] = fmaf(h[r][c], kr[r], pp[c]);
                rr[c] = fmaf(h[r][c], qr[r], rr[c]);
            }
            sq = fmaf(qr[r], qr[r], sq);
            sk = fmaf(kr[r], kr[r], sk);
            kq = fmaf(kr[r], qr[r], kq);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pp[c] = sum_over_rows<IG, JL>(pp[c]);
            rr[c] = sum_over_rows<IG, JL>(rr[c]);
        }
        sq = sum_over_rows<IG, JL>(sq);
        sk = sum_over_rows<IG, JL>(sk);
        kq = sum_over_rows<IG, JL>(kq);

        const float inv_nq = l2 ? 1.0f / sqrtf(sq + p.l2_eps) : 1.0f;
        const float inv_nk = l2 ? 1.0f / sqrtf(sk + p.l2_eps) : 1.0f;
        const float kqn = kq * inv_nk * inv_nq;
        // t is uniform: select the token's gates without dynamic indexing.
        float gt, bt;
        if constexpr (LAZY) {
            gt = gate_a[MAXT - 1];
            bt = gate_b[MAXT - 1];
#pragma unroll
            for (int j = MAXT - 2; j >= 0; --j) {
                gt = t == j ? gate_a[j] : gt;
                bt = t == j ? gate_b[j] : bt;
            }
        } else {
            gt = t == 0 ? gate_a[0] : t == 1 ? gate_a[1] : t == 2 ? gate_a[2] : gate_a[3];
            bt = t == 0 ? gate_b[0] : t == 1 ? gate_b[1] : t == 2 ? gate_b[2] : gate_b[3];
        }
        const float a = expf(gt);

        float u[4], oo[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float vj = ys[t][2 * DK + (NORM ? slice * SW : 0) + j4 * 4 + c];
            u[c] = bt * (vj - a * (pp[c] * inv_nk));
            oo[c] = p.scale * (a * (rr[c] * inv_nq) + u[c] * kqn);
        }
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const float kn = kr[r] * inv_nk;
#pragma unroll
            for (int c = 0; c < 4; ++c) h[r][c] = fmaf(a, h[r][c], kn * u[c]);
        }

        const int tout = LAZY ? t - kp : t;   // token of the window o belongs to
        if constexpr (NORM) {
            if (tout >= 0) {   // uniform over the workgroup: kp is the row's
                // every lane holds its row group's copy of the 4 columns; the
                // JL lanes of a row group cover the wave's SW columns
                float ss = oo[0] * oo[0];
#pragma unroll
                for (int c = 1; c < 4; ++c) ss = fmaf(oo[c], oo[c], ss);
#pragma unroll
                for (int off = 1; off < JL; off <<= 1) ss += __shfl_xor(ss, off, 64);
                if (lane == 0) ssq[t][wid] = ss;
                lds_barrier();
                float tot = ssq[t][0];
#pragma unroll
                for (int w = 1; w < NW; ++w) tot += ssq[t][w];
                const float rn = 1.0f / sqrtf(tot / static_cast<float>(DV) + p.norm_eps);
                const int tz = tout < 4 ? tout : 3;
#pragma unroll
                for (int c = 0; c < 4; ++c) oo[c] = oo[c] * rn * gzw[wid][tz][j4 * 4 + c];
            }
        }
        if (LAZY && t + 1 == kp) {
            // committed state of the previous window, in place
            float* dst = st_lb + (static_cast<size_t>(slot0) * p.HV + hv) * tile + col0;
#pragma unroll
            for (int r = 0; r < RPL; ++r)
                __builtin_nontemporal_store(h[r], reinterpret_cast<f4*>(dst + (ig + IG * r) * DV));
        }
        if (p.o && ig == 0 && tout >= 0) {
            const size_t oi = ((xrow + tout) * p.HV + hv) * DV + col0;
            if (p.out == ACT_BF16) {
                uint2 pk;
                pk.x = f32_to_bf16_bits(oo[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(oo[1])) << 16);
                pk.y = f32_to_bf16_bits(oo[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(oo[3])) << 16);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + oi) = pk;
            } else {
                f4 ov = {oo[0], oo[1], oo[2], oo[3]};
                __builtin_nontemporal_store(ov, reinterpret_cast<f4*>(static_cast<float*>(p.o) + oi));
            }
        }
        if (!LAZY && p.mode == REC_VERIFY) {
            const int slot = (slot0 + t + 1) % p.S;
            float* dst = st_lb + (static_cast<size_t>(slot) * p.HV + hv) * tile + col0;
#pragma unroll
            for (int r = 0; r < RPL; ++r)
                __builtin_nontemporal_store(h[r], reinterpret_cast<f4*>(dst + (ig + IG * r) * DV));
        }
    }
    if (!LAZY && p.mode == REC_REWIND) {
        float* dst = st_lb + (static_cast<size_t>(slot0) * p.HV + hv) * tile + col0;
#pragma unroll
        for (int r = 0; r < RPL; ++r)
            __builtin_nontemporal_store(h[r], reinterpret_cast<f4*>(dst + (ig + IG * r) * DV));
    }
}

// Occupancy cap for verify.  A verify wave streams its state slice in and its
// candidates out with little arithmetic between; more than one such wave
// resident per SIMD only adds concurrent DRAM streams and costs bandwidth
// (measured at the B8/T2 cohort over 30 layers: one wave per SIMD 5.86 TB/s,
// two 5.56, three 5.30).  The cap is set by reserving dynamic LDS so that
// exactly wg_per_cu one-wave workgroups fit in a CU's LDS.  Rewind computes
// up to T steps between its single read and single write of the slice and
// needs the other waves to cover that, so it runs uncapped.
constexpr int kVerifyWgPerCU = 4;   // one wave per SIMD
// A verify grid many rounds deep (the 30-layer B8/T2 cohort: 30,720
// workgroups, 30 rounds at four per CU) runs faster at five per CU once it is
// streaming: in the decode loop (verify + commit replayed from a HIP graph)
// 215-220 us per step against 227-236 us at four and 216-217 us at six, and
// 203-205 us against 206-208 us for back-to-back verify launches (three
// interleaved runs of each on one MI355X).  Short grids keep four: the solo
// B1/T3 launch over 30 layers (3,840 workgroups) takes 56.9 us at four
// against 58.7 us at five and 58.9 us at six.
constexpr int kVerifyWgPerCULong = 5;
constexpr int kVerifyLongRounds = 8;   // rounds at four per CU beyond which the long cap applies
// Verify with the fused norm runs the NS waves of a head as one workgroup
// with a barrier per token, so a wave stalls for its siblings; two such
// workgroups per CU (two waves per SIMD) cover that (B8/T2 cohort, 30
// layers: one per CU 253 us, two 204 us, three 203 us, uncapped 204 us,
// against 216-224 us for verify plus the separate norm launch).
constexpr int kVerifyNormWgPerCU = 2;
constexpr int kRewindWgPerCU = 0;   // no cap
constexpr int kLazyWgPerCU = 0;     // no cap (replay steps between read and write)

static size_t occupancy_lds_bytes(size_t static_bytes, int wg_per_cu)
{
    if (wg_per_cu <= 0) return 0;
    static std::atomic<int> cached[64];   // LDS bytes per CU, per device; 0 = not queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int lds = cached[dev].load(std::memory_order_relaxed);
    if (lds == 0) {
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
            lds <= 0)
            return 0;
        cached[dev].store(lds, std::memory_order_relaxed);
    }
    // a per-workgroup allocation in (lds / (wg_per_cu + 1), lds / wg_per_cu]
    const size_t total = static_cast<size_t>(lds) / wg_per_cu - 1024;
    return total > static_bytes ? total - static_bytes : 0;
}

// Static LDS of one kernel instantiation, queried once per process (the
// cache is a static of this function template, so each instantiation has its
// own).
template <int DK, int DV, int ACT, bool LAZY, bool NORM>
static size_t static_lds()
{
    static std::atomic<long long> cached{-1};
    long long v = cached.load(std::memory_order_relaxed);
    if (v < 0) {
        hipFuncAttributes a{};
        if (hipFuncGetAttributes(&a, reinterpret_cast<const void*>(recurrent_kernel<DK, DV, ACT, LAZY, NORM>)) !=
            hipSuccess) {
            clear_stale_error();
            return 0;   // no cap can be derived; the launch then runs uncapped
        }
        v = static_cast<long long>(a.sharedSizeBytes);
        cached.store(v, std::memory_order_relaxed);
    }
    return static_cast<size_t>(v);
}

template <int DK, int DV, int ACT, bool LAZY, bool NORM>
static void launch_one(const RecParams& p, dim3 grid, int threads, int cap, hipStream_t s)
{
    const size_t st = cap > 0 ? static_lds<DK, DV, ACT, LAZY, NORM>() : 0;
    const size_t dyn = cap > 0 && st > 0 ? occupancy_lds_bytes(st, cap) : 0;
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, ACT, LAZY, NORM>), grid, dim3(threads), dyn, s, p);
}

template <int DK, int DV, bool LAZY, bool NORM>
static void launch_rec_act(const RecParams& p, dim3 grid, int threads, int cap, hipStream_t s)
{
    if (p.act == ACT_BF16) launch_one<DK, DV, ACT_BF16, LAZY, NORM>(p, grid, threads, cap, s);
    else launch_one<DK, DV, ACT_F32, LAZY, NORM>(p, grid, threads, cap, s);
}

template <int DK, int DV>
static hipError_t launch_rec(RecParams p, hipStream_t s)
{
    constexpr int SW = DV < 32 ? DV : 32;
    constexpr int NS = DV / SW;
    const bool lazy = p.mode == REC_LAZY;
    const bool norm = p.norm_w != nullptr;
    const int nw = norm ? NS : 1;   // waves per workgroup
    p.groups = p.L * p.B * p.HK;
    p.per_group = (p.HV / p.HK) * (norm ? 1 : NS);
    const long long blocks = static_cast<long long>((p.groups + 7) / 8) * 8 * p.per_group;
    if (blocks <= 0 || blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    int cap = p.mode == REC_VERIFY ? kVerifyWgPerCU : p.mode == REC_LAZY ? kLazyWgPerCU : kRewindWgPerCU;
    if (norm && nw > 1 && p.mode == REC_VERIFY) cap = kVerifyNormWgPerCU;
    if (p.mode == REC_VERIFY && !norm) {
        const int cus = device_cus();
        if (cus > 0 && blocks > static_cast<long long>(kVerifyLongRounds) * kVerifyWgPerCU * cus)
            cap = kVerifyWgPerCULong;
    }
    const dim3 grid(static_cast<unsigned>(blocks));
    clear_stale_error();
    if (lazy) {
        if (norm) launch_rec_act<DK, DV, true, true>(p, grid, 64 * nw, cap, s);
        else launch_rec_act<DK, DV, true, false>(p, grid, 64, cap, s);
    } else {
        if (norm) launch_rec_act<DK, DV, false, true>(p, grid, 64 * nw, cap, s);
        else launch_rec_act<DK, DV, false, false>(p, grid, 64, cap, s);
    }
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_rec_dv(const RecParams& p, int DV, hipStream_t s)
{
    switch (DV) {
    case 16: return launch_rec<DK, 16>(p, s);
    case 32: return launch_rec<DK, 32>(p, s);
    case 64: return launch_rec<DK, 64>(p, s);
    case 128: return launch_rec<DK, 128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_recurrent(const RecParams& p, int DK, int DV, hipStream_t s)
{
    switch (DK) {
    case 16: return launch_rec_dv<16>(p, DV, s);
    case 32: return launch_rec_dv<32>(p, DV, s);
    case 64: return launch_rec_dv<64>(p, DV, s);
    case 128: return launch_rec_dv<128>(p, DV, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
