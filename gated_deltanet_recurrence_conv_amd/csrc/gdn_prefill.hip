// gdn_prefill.hip -- chunked prompt prefill (WY/UT form on MFMA).
#include "gdn_internal.h"

namespace gdn {

size_t prefill_workspace_bytes(int L, int B, int T, int HV, int DK, int DV, int chunk)
{
    (void)L; (void)B; (void)T; (void)HV; (void)DK; (void)DV; (void)chunk;
    return 0;
}

hipError_t launch_prefill(const PrefillParams& p, int DK, int DV, hipStream_t s)
{
    (void)p; (void)DK; (void)DV; (void)s;
    return hipErrorNotSupported;
}

}  // namespace gdn
