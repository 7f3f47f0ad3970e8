// gdn_accept.hip -- greedy acceptance of a verification window on the device.
//
// "Add request-owned eight-way MTP serving for Qwen 35B" (MTPLX PR #245),
// Follow-up: the greedy cohort route keeps draft IDs on the device and moves
// only token-ID arrays; What was broken item 2: a row commits two tokens, one
// token, or none.  Window token 0 is the pending (already sampled) token and
// tokens 1..T-1 are drafts; target[b][j] is the target's greedy token after
// window position j.  keep[b] = 1 + the number of leading drafts equal to the
// target token one position earlier (0 for an inactive row), and next[b] =
// target[b][keep-1], the next pending token.  keep feeds gdn_commit /
// gdn_verify_lazy directly, so a decode cycle needs no host round trip.
//
// One thread per row: B is a cohort (8) and T <= 4, so this is a single tiny
// launch whose cost is its launch.
#include "gdn_internal.h"

namespace gdn {

__global__ __launch_bounds__(256) void accept_kernel(AcceptParams p)
{
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= p.B) return;
    if (p.active && p.active[b] == 0) {
        p.keep[b] = 0;
        return;
    }
    const int T = p.T;
    const int32_t* tg = p.target + static_cast<size_t>(b) * T;
    const int32_t* dr = p.draft ? p.draft + static_cast<size_t>(b) * (T - 1) : nullptr;
    int k = 1;
    while (k < T && dr[k - 1] == tg[k - 1]) ++k;
    p.keep[b] = k;
    if (p.next) p.next[b] = tg[k - 1];
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t s)
{
    if (p.B <= 0) return hipErrorInvalidConfiguration;
    clear_stale_error();
    hipLaunchKernelGGL(accept_kernel, dim3((p.B + 255) / 256), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace gdn
