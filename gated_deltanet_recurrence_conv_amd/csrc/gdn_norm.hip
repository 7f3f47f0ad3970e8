// gdn_norm.hip -- gated RMSNorm epilogue of the mixer output.
//
// "MTP inference: review and commit structure" (eole docs), Functional
// commits item 4: the gated RMSNorm that follows the Gated DeltaNet mixer.
// For every (layer, row, token, value head):
//     y[j] = o[j] / sqrt(mean_j(o^2) + eps) * w[l][j] * SiLU(z[j]).
//
// Streaming work (o and z read once, y written once): one 64-lane wave per
// (layer, row, token, head), lanes over the d_v columns so every access is a
// contiguous run, the mean square reduced across the wave.  y may alias o:
// each lane reads its columns before the reduction and writes them after.
#include "gdn_internal.h"

namespace gdn {

template <int ACT, int OUT>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(NormParams p)
{
    constexpr int MAXV = 2;   // columns per lane (d_v <= 128)
    const long long wave = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const long long total = static_cast<long long>(p.L) * p.B * p.T * p.HV;
    if (wave >= total) return;
    const int b = static_cast<int>((wave / (static_cast<long long>(p.T) * p.HV)) % p.B);
    const int l = static_cast<int>(wave / (static_cast<long long>(p.B) * p.T * p.HV));
    if (p.active && p.active[b] == 0) return;
    const int DV = p.DV;
    const size_t base = static_cast<size_t>(wave) * DV;

    float ov[MAXV], zv[MAXV], wv[MAXV];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int j = lane + 64 * i;
        const bool in = j < DV;
        const int jj = in ? j : 0;
        ov[i] = in ? load_act<OUT>(p.o, base + jj) : 0.f;
        zv[i] = load_act<ACT>(p.z, base + jj);
        wv[i] = load_act<ACT>(p.w, static_cast<size_t>(l) * DV + jj);
        ss = fmaf(ov[i], ov[i], ss);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off, 64);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(DV) + p.eps);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int j = lane + 64 * i;
        if (j >= DV) continue;
        const float yv = ov[i] * r * wv[i] * silu(zv[i]);
        if constexpr (OUT == ACT_BF16) static_cast<uint16_t*>(p.y)[base + j] = f32_to_bf16_bits(yv);
        else static_cast<float*>(p.y)[base + j] = yv;
    }
}

hipError_t launch_gated_rmsnorm(const NormParams& p, hipStream_t s)
{
    const long long total = static_cast<long long>(p.L) * p.B * p.T * p.HV;
    const long long blocks = (total + 3) / 4;
    if (total <= 0 || blocks > 0x7fffffffLL || p.DV > 128) return hipErrorInvalidConfiguration;
    clear_stale_error();
    const dim3 grid(static_cast<unsigned>(blocks));
    if (p.act == ACT_BF16) {
        if (p.out == ACT_BF16) hipLaunchKernelGGL((gated_rmsnorm_kernel<ACT_BF16, ACT_BF16>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((gated_rmsnorm_kernel<ACT_BF16, ACT_F32>), grid, dim3(256), 0, s, p);
    } else {
        if (p.out == ACT_BF16) hipLaunchKernelGGL((gated_rmsnorm_kernel<ACT_F32, ACT_BF16>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((gated_rmsnorm_kernel<ACT_F32, ACT_F32>), grid, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace gdn
