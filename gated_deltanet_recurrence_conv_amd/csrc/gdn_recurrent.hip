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

// Sum over the IG row groups of a wave (lanes JL apart); every lane ends
// with the same bits.
template <int IG, int JL>
__device__ __forceinline__ float sum_over_rows(float v)
{
    if constexpr (JL <= 4) v = xor_add<4>(v);
    if constexpr (JL <= 8) v = xor_add<8>(v);
    if constexpr (JL <= 16) v = xor_add<16>(v);
    return xor_add<32>(v);
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

#ifndef GDN_KSPLIT
#define GDN_KSPLIT 1
#endif
// d_k parts of a (row, head, column slice): each part is one wave holding
// DK / KS rows of the slice, and the partial d_k sums of a step are added
// across the parts through LDS.  More waves per slice shortens each wave's
// chain (loads, conv share, step arithmetic), which sets the time of a launch
// that fits the GPU in one round (one layer of the B8/T2 cohort: 768 waves).
// The split depends only on the head shape, so every mode and every batch
// uses the same reduction tree.
template <int DK, int DV>
constexpr int ksplit()
{
    constexpr int SW = DV < 32 ? DV : 32;
    constexpr int IG = 64 / (SW / 4);
    return GDN_KSPLIT < DK / IG ? GDN_KSPLIT : DK / IG;
}

// GRP: one workgroup per (layer, row, qk head) holding the column-slice waves
// of all its value heads (lazy and rewind).  Every conv channel of a row is
// then read by exactly one lane of the launch, so that lane can write the
// shifted conv cache itself, and the q/k conv is computed once per qk head
// instead of once per wave.  At most kGroupMaxWaves waves per workgroup
// (more than 8 would cap registers at 128 per lane and spill).
constexpr int kGroupMaxWaves = 8;
constexpr int kGroupGridWavesPerCU = 8;   // deepest grid that takes the GRP layout

template <int DK, int DV, bool NORM, bool GRP>
constexpr int waves_per_wg()
{
    return GRP ? kGroupMaxWaves : (NORM ? waves_per_head<DV>() : 1) * ksplit<DK, DV>();
}

// LZ: 0 for verify and rewind; for the fused form (LAZY) the most tokens a
// wave runs, a replayed prefix of at most T tokens plus a window of T: 4 when
// T <= 2, 8 when T <= 4.  The conv outputs in LDS and the window and gate
// registers are sized by it, and the T <= 2 instantiation's halved LDS lets
// more waves share a CU (30-layer B8/T2 cohort: fused cycle 152-156 against
// 141-144 us; one-layer launches 456 against 440 us per 30-layer cycle).
template <int DK, int DV, int ACT, int LZ, bool NORM, bool GRP>
__global__ __launch_bounds__((64 * waves_per_wg<DK, DV, NORM, GRP>())) void recurrent_kernel(RecParams p)
{
    constexpr bool LAZY = LZ > 0;
    constexpr int SW = DV < 32 ? DV : 32;  // columns per wave
    constexpr int NS = DV / SW;            // column slices per head
    constexpr int JL = SW / 4;             // lanes across one row segment
    constexpr int IG = 64 / JL;            // row groups per wave
    constexpr int KS = ksplit<DK, DV>();   // d_k parts (waves) per slice
    constexpr int KR = DK / KS;            // rows of one part
    constexpr int RPL = KR / IG;           // rows held per lane
    constexpr int MAXT = LAZY ? LZ : 4;    // tokens one wave runs
    constexpr int NW = NORM ? NS : 1;      // column slices per workgroup (NORM)
    constexpr int NWG = NW * KS;           // waves per workgroup (not GRP)
    // conv channels of the workgroup: q and k of the qk head, then the v
    // channels of its one slice, or (NORM) of all NS slices, or (GRP) of all
    // slices of up to kGroupMaxWaves / NS value heads; its waves share the q
    // and k conv (NCH is the LDS allocation, nch below the channels in use)
    constexpr int NCH = 2 * DK + (GRP ? (kGroupMaxWaves / NS) * DV : NORM ? DV : SW);
    static_assert(RPL >= 1 && KR % IG == 0, "tile shape");
    static_assert(!GRP || (KS == 1 && !NORM), "GRP workgroups hold whole slices, no norm");

    __shared__ float ys[MAXT][NCH];
    __shared__ float ssq[NORM ? MAXT : 1][NW];   // per-slice sums of o^2 (NORM)
    __shared__ float gzw[NW][NORM ? 4 : 1][NORM ? SW : 1];   // w[j] * SiLU(z[t][j]) (NORM)
    // partial d_k sums of a step (8 column sums, |q|^2, |k|^2, k.q) per part,
    // double-buffered by step parity
    __shared__ __align__(16) float xch[KS > 1 ? 2 : 1][NW][KS][JL][12];

    // ---- block -> (layer, row, qk head, value head, slice), XCD-aware ----
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int sgrp = bid >> 3;
    const int r_in = GRP ? 0 : sgrp % p.per_group;
    const int grp = GRP ? bid : (sgrp / p.per_group) * 8 + xcd;
    if (grp >= p.groups) return;
    const int m = grp % p.HK;
    const int lb = grp / p.HK;  // l * B + b
    const int b = lb % p.B;
    const int gsz = p.HV / p.HK;
    const int wid = static_cast<int>(threadIdx.x >> 6);
    const int kpart = wid % KS;            // d_k part of this wave
    const int sw = wid / KS;               // slice wave index (NORM)
    const int slice = NORM ? sw : GRP ? wid % NS : r_in % NS;
    const int hv = NORM ? m * gsz + r_in : GRP ? m * gsz + wid / NS : m * gsz + r_in / NS;
    // waves and conv channels of the workgroup
    const int nwg = GRP ? static_cast<int>(blockDim.x >> 6) : NWG;
    const int nch = GRP ? 2 * DK + gsz * DV : NCH;
    const int row0 = kpart * KR;           // first state row of this wave's part

    const int lane = static_cast<int>(threadIdx.x & 63);
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
    // channel groups per wave (GRP: the most over 1 <= gsz, reached at gsz = 1)
    constexpr int NG = GRP ? (2 * DK + DV + 64 * NS - 1) / (64 * NS) : (NCH + 64 * NWG - 1) / (64 * NWG);
    // channel of group n in this lane: lane + 64 * (wid + nwg * n)
    const int vch0 = GRP ? 2 * p.HK * DK + m * gsz * DV                    // all value heads of m
                         : 2 * p.HK * DK + hv * DV + (NORM ? 0 : slice * SW);   // first v channel of the set
    constexpr int NROW = MAXT + 3;   // window rows per channel
    float wv[NG][4];
    float win[NG][NROW];
    float bias[NG];
#pragma unroll
    for (int n = 0; n < NG; ++n) {
        const int ch = min(lane + 64 * (wid + nwg * n), nch - 1);
        const int c = ch < DK ? m * DK + ch : (ch < 2 * DK ? p.HK * DK + m * DK + (ch - DK) : vch0 + (ch - 2 * DK));
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
        h[r] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(src + (row0 + ig + IG * r) * DV));

    // ---- conv + SiLU for every window token, into LDS (a rewind without o
    // needs no q channels, nor do the replayed tokens of the 4-token fused
    // form, whose steps skip the q work) ----
    const bool use_silu = (p.flags & FLAG_SILU) != 0;
    const int qskip = LAZY ? (LZ == 4 ? kp : 0) : (p.mode == REC_REWIND && !p.o ? nsteps : 0);
#pragma unroll
    for (int n = 0; n < NG; ++n) {
        const int ch = lane + 64 * (wid + nwg * n);
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
            if (t < nsteps && !(ch < DK && t < qskip)) {
                float acc = wv[n][0] * win[n][t];
                acc = fmaf(wv[n][1], win[n][t + 1], acc);
                acc = fmaf(wv[n][2], win[n][t + 2], acc);
                acc = fmaf(wv[n][3], win[n][t + 3], acc);
                acc += bias[n];
                if (ch < nch) ys[t][ch] = use_silu ? silu_hw(acc) : acc;
            }
        }
    }
    if constexpr (GRP) {
        // A committing row's conv cache becomes window rows kp .. kp+2 of
        // [conv cache ; tokens] (the replayed window's, in the fused form).
        // This lane is the only reader of its channels in the whole launch,
        // and it has read them: it can overwrite them now.  Lanes past the
        // last channel re-read it and write nothing.
        if (p.conv_out && kp > 0) {
#pragma unroll
            for (int n = 0; n < NG; ++n) {
                const int ch = lane + 64 * (wid + nwg * n);
                if (ch < nch) {
                    const int c = ch < DK ? m * DK + ch
                                : (ch < 2 * DK ? p.HK * DK + m * DK + (ch - DK) : vch0 + (ch - 2 * DK));
#pragma unroll
                    for (int r = 0; r < 3; ++r) {
                        float v = win[n][1];   // kp + r is in 1 .. T + 2
#pragma unroll
                        for (int j = 2; j < NROW && j <= 6; ++j) v = kp + r == j ? win[n][j] : v;
                        store_act<ACT>(p.conv_out, (srow + r) * C + c, v);
                    }
                }
            }
        }
    }
    if constexpr (NORM) {
        if (ig == 0 && kpart == 0)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int c = 0; c < 4; ++c) gzw[sw][t][j4 * 4 + c] = nw[c] * silu_hw(zv[t][c]);
    }
    lds_barrier();

    const bool l2 = (p.flags & FLAG_L2) != 0;
    for (int t = 0; t < nsteps; ++t) {
        const int tout = LAZY ? t - kp : t;   // token of the window o belongs to
        // A step without an output (a rewind without o, a replayed token of
        // the fused form) needs neither h^T q nor |q| and k.q (a uniform
        // branch; u and h are computed the same way in both, so the fused form
        // stays bit-equal to rewind + verify).  With the 4-token window the
        // fused form's replayed steps take the short body (B8/T2 cohort: one
        // layer per launch 419 -> 395 us per 30-layer cycle, 30 layers in one
        // launch 140-146 -> 138-139 us); with the 8-token window the two bodies
        // measured slower (171 against 148-152 us), so every step there is full.
        const bool want_out = p.o != nullptr && tout >= 0;
        const bool full_step = want_out || LZ == 8;
        float kr[RPL], qr[RPL];
#pragma unroll
        for (int r = 0; r < RPL; ++r) kr[r] = ys[t][DK + row0 + ig + IG * r];
        float pp[4] = {0.f, 0.f, 0.f, 0.f}, rr[4] = {0.f, 0.f, 0.f, 0.f};
        float sq = 0.f, sk = 0.f, kq = 0.f;
        if (full_step) {
#pragma unroll
            for (int r = 0; r < RPL; ++r) qr[r] = ys[t][row0 + ig + IG * r];
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
        } else {
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
#pragma unroll
                for (int c = 0; c < 4; ++c) pp[c] = fmaf(h[r][c], kr[r], pp[c]);
                sk = fmaf(kr[r], kr[r], sk);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) pp[c] = sum_over_rows<IG, JL>(pp[c]);
            sk = sum_over_rows<IG, JL>(sk);
        }
        if constexpr (KS > 1) {
            // add the parts' sums in part order, the same in every wave
            float(*xs)[JL][12] = xch[t & 1][sw];
            if (ig == 0) {
                float* xp = xs[kpart][j4];
                *reinterpret_cast<f4*>(xp) = f4{pp[0], pp[1], pp[2], pp[3]};
                *reinterpret_cast<f4*>(xp + 4) = f4{rr[0], rr[1], rr[2], rr[3]};
                *reinterpret_cast<f4*>(xp + 8) = f4{sq, sk, kq, 0.f};
            }
            lds_barrier();
            f4 a0 = *reinterpret_cast<const f4*>(xs[0][j4]);
            f4 a1 = *reinterpret_cast<const f4*>(xs[0][j4] + 4);
            f4 a2 = *reinterpret_cast<const f4*>(xs[0][j4] + 8);
#pragma unroll
            for (int k = 1; k < KS; ++k) {
                a0 += *reinterpret_cast<const f4*>(xs[k][j4]);
                a1 += *reinterpret_cast<const f4*>(xs[k][j4] + 4);
                a2 += *reinterpret_cast<const f4*>(xs[k][j4] + 8);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pp[c] = a0[c];
                rr[c] = a1[c];
            }
            sq = a2[0];
            sk = a2[1];
            kq = a2[2];
        }

        const float inv_nk = l2 ? __builtin_amdgcn_rsqf(sk + p.l2_eps) : 1.0f;
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

        // u and o are written with explicit fmaf so that no instantiation is
        // left to contract them its own way: every mode and workgroup layout
        // computes the same bits.
        float u[4], oo[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float vj = ys[t][2 * DK + (NORM ? slice * SW : GRP ? (wid / NS) * DV + slice * SW : 0) + j4 * 4 + c];
            u[c] = bt * fmaf(-a, pp[c] * inv_nk, vj);
        }
        if (want_out) {
            const float inv_nq = l2 ? __builtin_amdgcn_rsqf(sq + p.l2_eps) : 1.0f;
            const float kqn = kq * inv_nk * inv_nq;
#pragma unroll
            for (int c = 0; c < 4; ++c) oo[c] = p.scale * fmaf(a, rr[c] * inv_nq, u[c] * kqn);
        }
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const float kn = kr[r] * inv_nk;
#pragma unroll
            for (int c = 0; c < 4; ++c) h[r][c] = fmaf(a, h[r][c], kn * u[c]);
        }

        if constexpr (NORM) {
            if (want_out) {   // uniform over the workgroup: kp is the row's
                // every lane holds its row group's copy of the 4 columns; the
                // JL lanes of a row group cover the wave's SW columns
                float ss = oo[0] * oo[0];
#pragma unroll
                for (int c = 1; c < 4; ++c) ss = fmaf(oo[c], oo[c], ss);
#pragma unroll
                for (int off = 1; off < JL; off <<= 1) ss += __shfl_xor(ss, off, 64);
                if (lane == 0 && kpart == 0) ssq[t][sw] = ss;
                lds_barrier();
                float tot = ssq[t][0];
#pragma unroll
                for (int w = 1; w < NW; ++w) tot += ssq[t][w];
                const float rn = 1.0f / sqrtf(tot / static_cast<float>(DV) + p.norm_eps);
                const int tz = tout < 4 ? tout : 3;
#pragma unroll
                for (int c = 0; c < 4; ++c) oo[c] = oo[c] * rn * gzw[sw][tz][j4 * 4 + c];
            }
        }
        if (LAZY && t + 1 == kp) {
            // committed state of the previous window, in place
            float* dst = st_lb + (static_cast<size_t>(slot0) * p.HV + hv) * tile + col0;
#pragma unroll
            for (int r = 0; r < RPL; ++r)
                __builtin_nontemporal_store(h[r], reinterpret_cast<f4*>(dst + (row0 + ig + IG * r) * DV));
        }
        if (want_out && ig == 0 && kpart == 0) {
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
                __builtin_nontemporal_store(h[r], reinterpret_cast<f4*>(dst + (row0 + ig + IG * r) * DV));
        }
    }
    if (!LAZY && p.mode == REC_REWIND) {
        float* dst = st_lb + (static_cast<size_t>(slot0) * p.HV + hv) * tile + col0;
#pragma unroll
        for (int r = 0; r < RPL; ++r)
            __builtin_nontemporal_store(h[r], reinterpret_cast<f4*>(dst + (row0 + ig + IG * r) * DV));
    }
}

// Occupancy caps, in waves per CU (a launch reserves dynamic LDS so that
// cap / waves-per-workgroup workgroups fit in a CU's LDS).  A verify wave
// streams its state slice in and its candidates out with little arithmetic
// between; more than about one such wave resident per SIMD only adds
// concurrent DRAM streams and costs bandwidth (measured with one-wave
// workgroups at the B8/T2 cohort over 30 layers: one wave per SIMD 5.86 TB/s,
// two 5.56, three 5.30).  A verify grid many rounds deep (the 30-layer
// cohort) ran best at five waves per CU once streaming, shorter grids at
// four.  Verify with the fused norm runs the waves of a head as one
// workgroup with a barrier per token, so two waves per SIMD cover the
// stalls.  Rewind and the fused commit + verify compute several steps
// between their single read and write of the slice and need other waves to
// cover that: they run uncapped (0).
#ifndef GDN_VW_SHORT
#define GDN_VW_SHORT 4
#endif
#ifndef GDN_VW_LONG
#define GDN_VW_LONG 5
#endif
#ifndef GDN_VW_NORM
#define GDN_VW_NORM 8
#endif
#ifndef GDN_VW_LAZY
#define GDN_VW_LAZY 0
#endif
#ifndef GDN_VW_REWIND
#define GDN_VW_REWIND 0
#endif
constexpr int kVerifyWavesPerCU = GDN_VW_SHORT;
constexpr int kVerifyWavesPerCULong = GDN_VW_LONG;
constexpr int kVerifyLongRounds = 8;   // rounds at the short cap beyond which the long cap applies
constexpr int kVerifyNormWavesPerCU = GDN_VW_NORM;
constexpr int kLazyWavesPerCU = GDN_VW_LAZY;
constexpr int kRewindWavesPerCU = GDN_VW_REWIND;

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
template <int DK, int DV, int ACT, int LZ, bool NORM, bool GRP>
static size_t static_lds()
{
    static std::atomic<long long> cached{-1};
    long long v = cached.load(std::memory_order_relaxed);
    if (v < 0) {
        hipFuncAttributes a{};
        if (hipFuncGetAttributes(&a, reinterpret_cast<const void*>(recurrent_kernel<DK, DV, ACT, LZ, NORM, GRP>)) !=
            hipSuccess) {
            clear_stale_error();
            return 0;   // no cap can be derived; the launch then runs uncapped
        }
        v = static_cast<long long>(a.sharedSizeBytes);
        cached.store(v, std::memory_order_relaxed);
    }
    return static_cast<size_t>(v);
}

template <int DK, int DV, int ACT, int LZ, bool NORM, bool GRP>
static void launch_one(const RecParams& p, dim3 grid, int threads, int cap, hipStream_t s)
{
    const size_t st = cap > 0 ? static_lds<DK, DV, ACT, LZ, NORM, GRP>() : 0;
    const size_t dyn = cap > 0 && st > 0 ? occupancy_lds_bytes(st, cap) : 0;
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, ACT, LZ, NORM, GRP>), grid, dim3(threads), dyn, s, p);
}

template <int DK, int DV, int LZ, bool NORM, bool GRP = false>
static void launch_rec_act(const RecParams& p, dim3 grid, int threads, int cap, hipStream_t s)
{
    if (p.act == ACT_BF16) launch_one<DK, DV, ACT_BF16, LZ, NORM, GRP>(p, grid, threads, cap, s);
    else launch_one<DK, DV, ACT_F32, LZ, NORM, GRP>(p, grid, threads, cap, s);
}

// The fused form's instantiation by its token capacity (T <= 4 is checked
// by the caller).
template <int DK, int DV, bool NORM, bool GRP = false>
static void launch_lazy_act(const RecParams& p, dim3 grid, int threads, int cap, hipStream_t s)
{
    if (p.T <= 2) launch_rec_act<DK, DV, 4, NORM, GRP>(p, grid, threads, cap, s);
    else launch_rec_act<DK, DV, 8, NORM, GRP>(p, grid, threads, cap, s);
}

template <int DK, int DV>
static hipError_t launch_rec(RecParams p, hipStream_t s, bool* conv_shifted)
{
    constexpr int SW = DV < 32 ? DV : 32;
    constexpr int NS = DV / SW;
    constexpr int KS = ksplit<DK, DV>();
    const bool lazy = p.mode == REC_LAZY;
    const bool norm = p.norm_w != nullptr;
    // Lazy and rewind without the norm, on a grid the GPU holds at once (two
    // waves per SIMD, e.g. one layer of the B8 cohort): one workgroup per qk
    // head, which also shifts the conv cache, so no second launch follows.
    // Deeper grids (all 30 layers in one launch) keep one-wave workgroups and
    // the separate shift: there the 8-wave workgroups run one per CU and
    // stream worse (30-layer cohort: fused cycle 162 against 151 us, rewind
    // 166 against 156 us; one layer: 15.3 against 19.7 us per layer-cycle).
    const int cus = device_cus();
    const long long grp_waves = static_cast<long long>(p.L) * p.B * p.HV * NS;
    const bool grp = (lazy || p.mode == REC_REWIND) && !norm && KS == 1 && p.conv_out != nullptr &&
                     p.HK > 0 && (p.HV / p.HK) * NS <= kGroupMaxWaves && cus > 0 &&
                     grp_waves <= static_cast<long long>(kGroupGridWavesPerCU) * cus;
    if (conv_shifted) *conv_shifted = grp;
    if (grp) {
        const int wpw = (p.HV / p.HK) * NS;
        p.groups = p.L * p.B * p.HK;
        p.per_group = 1;
        const long long blocks = static_cast<long long>(p.groups);
        if (blocks <= 0 || blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const int waves = lazy ? kLazyWavesPerCU : kRewindWavesPerCU;
        const int cap = waves > 0 ? (waves / wpw > 0 ? waves / wpw : 1) : 0;
        clear_stale_error();
        if (lazy) launch_lazy_act<DK, DV, false, true>(p, dim3(static_cast<unsigned>(blocks)), 64 * wpw, cap, s);
        else launch_rec_act<DK, DV, 0, false, true>(p, dim3(static_cast<unsigned>(blocks)), 64 * wpw, cap, s);
        return hipGetLastError();
    }
    p.conv_out = nullptr;
    const int wpw = (norm ? NS : 1) * KS;   // waves per workgroup
    p.groups = p.L * p.B * p.HK;
    p.per_group = (p.HV / p.HK) * (norm ? 1 : NS);
    const long long blocks = static_cast<long long>((p.groups + 7) / 8) * 8 * p.per_group;
    if (blocks <= 0 || blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    int waves = p.mode == REC_VERIFY ? kVerifyWavesPerCU : p.mode == REC_LAZY ? kLazyWavesPerCU : kRewindWavesPerCU;
    if (norm && p.mode == REC_VERIFY) waves = kVerifyNormWavesPerCU;
    if (p.mode == REC_VERIFY && !norm) {
        const int cus = device_cus();
        if (cus > 0 && blocks * wpw > static_cast<long long>(kVerifyLongRounds) * kVerifyWavesPerCU * cus)
            waves = kVerifyWavesPerCULong;
    }
    const int cap = waves > 0 ? (waves / wpw > 0 ? waves / wpw : 1) : 0;   // workgroups per CU
    const dim3 grid(static_cast<unsigned>(blocks));
    clear_stale_error();
    if (lazy) {
        if (norm) launch_lazy_act<DK, DV, true>(p, grid, 64 * wpw, cap, s);
        else launch_lazy_act<DK, DV, false>(p, grid, 64 * wpw, cap, s);
    } else {
        if (norm) launch_rec_act<DK, DV, 0, true>(p, grid, 64 * wpw, cap, s);
        else launch_rec_act<DK, DV, 0, false>(p, grid, 64 * wpw, cap, s);
    }
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_rec_dv(const RecParams& p, int DV, hipStream_t s, bool* cs)
{
    switch (DV) {
    case 16: return launch_rec<DK, 16>(p, s, cs);
    case 32: return launch_rec<DK, 32>(p, s, cs);
    case 64: return launch_rec<DK, 64>(p, s, cs);
    case 128: return launch_rec<DK, 128>(p, s, cs);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_recurrent(const RecParams& p, int DK, int DV, hipStream_t s, bool* conv_shifted)
{
    if (conv_shifted) *conv_shifted = false;
    switch (DK) {
    case 16: return launch_rec_dv<16>(p, DV, s, conv_shifted);
    case 32: return launch_rec_dv<32>(p, DV, s, conv_shifted);
    case 64: return launch_rec_dv<64>(p, DV, s, conv_shifted);
    case 128: return launch_rec_dv<128>(p, DV, s, conv_shifted);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
