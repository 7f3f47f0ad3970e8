// gdn_api.hip -- the C ABI of libgdn.so: host-side validation, launch
// geometry and status codes.  Every argument is validated before any launch,
// and a call that fails validation launches nothing ("MTP inference: review
// and commit structure", Review fixes; "Add request-owned eight-way MTP
// serving for Qwen 35B", Clean-install verification).  There is exactly one
// code path per call and no host fallback.
#include "gdn.h"
#include "gdn_internal.h"

#include <stdint.h>

#include <mutex>

// Device scratch of gdn_prefill_chunked_noalloc: the chunk records of the
// prefill, in a static array of the library's code object instead of a
// caller's workspace.  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never passes this name to a kernel (on the
// host it is only a stand-in for the device symbol); it uses the device
// address from hipGetSymbolAddress, kept per device.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

using gdn::RecParams;
using gdn::WinParams;
using gdn::ConvParams;

bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

long long channels64(const gdn_dims* d)
{
    return 2LL * d->HK * d->DK + static_cast<long long>(d->HV) * d->DV;
}

// Conv channels; fits int32 once check_dims has passed (C * T <= 2^31).
int channels(const gdn_dims* d) { return static_cast<int>(channels64(d)); }

// Checks shared by every call.
gdn_status check_dims(const gdn_dims* d)
{
    if (!d) return GDN_E_NULL;
    if (d->act != GDN_F32 && d->act != GDN_BF16) return GDN_E_DTYPE;
    if (d->out != GDN_F32 && d->out != GDN_BF16) return GDN_E_DTYPE;
    if (d->L < 1 || d->B < 1 || d->T < 1 || d->HV < 1 || d->HK < 1 || d->S < 1)
        return GDN_E_SHAPE;
    if (d->HV % d->HK != 0) return GDN_E_SHAPE;
    if (!head_dim_ok(d->DK) || !head_dim_ok(d->DV)) return GDN_E_SHAPE;
    if (d->KCONV != 4) return GDN_E_SHAPE;
    // Keep every element index of every array inside int64 and the grids
    // inside their limits.
    const long long C = channels64(d);
    if (static_cast<long long>(d->L) * d->B > 65535) return GDN_E_SHAPE;
    if (static_cast<long long>(d->L) * d->B * d->HV > (1LL << 30)) return GDN_E_SHAPE;   // 32-bit tile counts
    if (static_cast<long long>(d->HV) * d->DK * d->DV * d->S * d->B * d->L > (1LL << 40))
        return GDN_E_SHAPE;
    if (C * d->T > (1LL << 31)) return GDN_E_SHAPE;
    if (!(d->l2_eps >= 0.0f)) return GDN_E_SHAPE;
    return GDN_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Tensor arguments (req / opt) must be 16-byte aligned, since the kernels
// move them in 16-byte vectors; the small per-row int32 arrays (cur, keep,
// err: ints4) only need their natural 4-byte alignment.
gdn_status check_ptrs(std::initializer_list<const void*> req, std::initializer_list<const void*> opt,
                      std::initializer_list<const void*> ints4 = {})
{
    for (const void* p : req)
        if (!p) return GDN_E_NULL;
    for (const void* p : req)
        if (!aligned(p)) return GDN_E_ALIGN;
    for (const void* p : opt)
        if (p && !aligned(p)) return GDN_E_ALIGN;
    for (const void* p : ints4)
        if (p && !aligned4(p)) return GDN_E_ALIGN;
    return GDN_OK;
}

// The HIP error behind the most recent GDN_E_HIP of this thread.
thread_local hipError_t g_last_hip_error = hipSuccess;

gdn_status from_hip(hipError_t e)
{
    if (e == hipSuccess) return GDN_OK;
    g_last_hip_error = e;
    return GDN_E_HIP;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

gdn_status scratch_address(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return from_hip(e);
    if (dev < 0 || dev >= 64) return GDN_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            gdn::clear_stale_error();
            return from_hip(e != hipSuccess ? e : hipErrorInvalidSymbol);
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GDN_OK;
}

RecParams rec_params(const gdn_dims* d)
{
    RecParams p{};
    p.L = d->L; p.B = d->B; p.T = d->T; p.HV = d->HV; p.HK = d->HK; p.S = d->S;
    p.C = channels(d);
    p.act = d->act; p.out = d->out;
    p.scale = d->scale; p.l2_eps = d->l2_eps; p.flags = d->flags;
    return p;
}

// Gated-norm epilogue operands: all null (raw o) or z and w both given.
struct NormEpi {
    const void* z = nullptr;
    const void* w = nullptr;
    float eps = 0.0f;
};

gdn_status check_epi(const NormEpi& e)
{
    if (!e.w && !e.z) return GDN_OK;
    if (!(e.eps >= 0.0f)) return GDN_E_SHAPE;
    return check_ptrs({e.z, e.w}, {}, {});
}

gdn_status verify_impl(const gdn_dims* d, const void* x, const void* conv_w, const void* conv_b,
                       const void* conv_state, const void* g, const void* beta, float* state,
                       const int32_t* cur, void* o, const NormEpi& epi, const uint8_t* active,
                       int32_t* err, void* stream)
{
    gdn_status st = check_dims(d);
    if (st != GDN_OK) return st;
    if (d->T > 4 || d->S < d->T + 1) return GDN_E_SHAPE;
    st = check_ptrs({x, conv_w, conv_state, g, beta, state, o}, {conv_b}, {cur, err});
    if (st != GDN_OK) return st;
    st = check_epi(epi);
    if (st != GDN_OK) return st;
    RecParams p = rec_params(d);
    p.x = x; p.conv_w = conv_w; p.conv_b = conv_b; p.conv_state = conv_state;
    p.g = g; p.beta = beta; p.state = state; p.cur = cur; p.o = o; p.active = active;
    p.keep = nullptr; p.err = err; p.mode = gdn::REC_VERIFY;
    p.z = epi.z; p.norm_w = epi.w; p.norm_eps = epi.eps;
    return from_hip(gdn::launch_recurrent(p, d->DK, d->DV, static_cast<hipStream_t>(stream)));
}

gdn_status verify_lazy_impl(const gdn_dims* d, const void* x_prev, const void* g_prev,
                            const void* beta_prev, const int32_t* keep_prev, const void* x,
                            const void* conv_w, const void* conv_b, void* conv_state,
                            const void* g, const void* beta, float* state, const int32_t* cur,
                            void* o, const NormEpi& epi, const uint8_t* active, int32_t* err,
                            void* stream)
{
    gdn_status st = check_dims(d);
    if (st != GDN_OK) return st;
    if (d->T > 4) return GDN_E_SHAPE;
    st = check_ptrs({x, conv_w, conv_state, g, beta, state, o}, {conv_b, x_prev, g_prev, beta_prev},
                    {cur, keep_prev, err});
    if (st != GDN_OK) return st;
    if (keep_prev && (!x_prev || !g_prev || !beta_prev)) return GDN_E_NULL;
    st = check_epi(epi);
    if (st != GDN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    RecParams p = rec_params(d);
    p.x = x; p.conv_w = conv_w; p.conv_b = conv_b; p.conv_state = conv_state;
    p.g = g; p.beta = beta; p.state = state; p.cur = cur; p.o = o; p.active = active;
    p.keep = keep_prev; p.err = err; p.mode = gdn::REC_LAZY;
    p.z = epi.z; p.norm_w = epi.w; p.norm_eps = epi.eps;
    // without a previous window nothing is replayed; its inputs are never
    // used but every load of the kernel is unconditional, so point them at x
    p.x_prev = keep_prev ? x_prev : x;
    p.g_prev = keep_prev ? g_prev : g;
    p.beta_prev = keep_prev ? beta_prev : beta;
    p.conv_out = conv_state;
    bool shifted = false;
    st = from_hip(gdn::launch_recurrent(p, d->DK, d->DV, s, &shifted));
    if (st != GDN_OK || !keep_prev || shifted) return st;
    // Otherwise (the fused norm, or more waves per qk head than a workgroup
    // holds) the conv cache is shifted by a second launch, after every wave
    // has read the old cache.
    WinParams w{};
    w.x = x_prev; w.conv_state = conv_state; w.cur = const_cast<int32_t*>(cur); w.keep = keep_prev;
    w.active = nullptr; w.err = err; w.L = d->L; w.B = d->B; w.T = d->T; w.S = d->S;
    w.C = p.C; w.act = d->act; w.mode = gdn::WIN_REWIND;
    return from_hip(gdn::launch_window(w, s));
}

// Chunked prefill (padded or ragged).  With use_scratch the chunk records go
// to the library's static device scratch instead of a caller's workspace;
// dims whose records do not fit it are refused before anything is launched.
// The fused conv's inputs (prefill_impl with conv = nullptr reads y).
struct ConvIn {
    const void* x;
    const void* conv_w;
    const void* conv_b;
    void* conv_state;
};

gdn_status prefill_impl(const gdn_dims* d, const void* y, const void* g, const void* beta, float* state,
                        const int32_t* cur, void* o, const int32_t* lengths, int32_t chunk, void* workspace,
                        size_t workspace_bytes, bool use_scratch, int32_t* err, void* stream,
                        const ConvIn* conv = nullptr)
{
    gdn_status st = check_dims(d);
    if (st != GDN_OK) return st;
    if (chunk != 64) return GDN_E_SHAPE;
    st = check_ptrs({y, g, beta, state, o}, {workspace}, {cur, lengths, err});
    if (st != GDN_OK) return st;
    if (conv) {
        st = check_ptrs({conv->x, conv->conv_w, conv->conv_state}, {conv->conv_b}, {});
        if (st != GDN_OK) return st;
        if (!gdn::prefill_conv_supported(d->DK, d->DV, d->act)) return GDN_E_UNSUPPORTED;
    }
    if (!gdn::prefill_supported(d->DK, d->DV, d->act)) return GDN_E_UNSUPPORTED;
    const size_t need = gdn::prefill_workspace_bytes(d->L, d->B, d->T, d->HV, d->DK, d->DV, d->act, chunk);
    if (use_scratch) {
        if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_E_WORKSPACE;
        st = scratch_address(&workspace);
        if (st != GDN_OK) return st;
        workspace_bytes = GDN_NOALLOC_SCRATCH_BYTES;
    }
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_E_WORKSPACE;
    gdn::PrefillParams p{};
    p.y = y; p.g = g; p.beta = beta; p.state = state; p.cur = cur; p.o = o; p.ws = workspace;
    p.err = err; p.lengths = lengths;
    p.L = d->L; p.B = d->B; p.T = d->T; p.HV = d->HV; p.HK = d->HK; p.S = d->S;
    p.C = channels(d); p.act = d->act; p.out = d->out;
    p.scale = d->scale; p.l2_eps = d->l2_eps; p.flags = d->flags;
    if (conv) {
        p.x = conv->x; p.conv_w = conv->conv_w; p.conv_b = conv->conv_b; p.conv_state = conv->conv_state;
    }
    return from_hip(gdn::launch_prefill(p, d->DK, d->DV, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s)
{
    switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_E_NULL: return "GDN_E_NULL: a required pointer is NULL";
    case GDN_E_SHAPE: return "GDN_E_SHAPE: a size is outside the supported range";
    case GDN_E_DTYPE: return "GDN_E_DTYPE: act/out must be GDN_F32 or GDN_BF16";
    case GDN_E_ALIGN: return "GDN_E_ALIGN: a tensor is not 16-byte aligned or an int32 array not 4-byte aligned";
    case GDN_E_UNSUPPORTED: return "GDN_E_UNSUPPORTED: not implemented for these arguments";
    case GDN_E_WORKSPACE: return "GDN_E_WORKSPACE: workspace missing or too small";
    case GDN_E_HIP: return "GDN_E_HIP: the HIP runtime reported a launch failure";
    }
    return "unknown gdn_status";
}

const char* gdn_version(void) { return "libgdn 0.1.0 (HIP, gfx950)"; }

const char* gdn_last_hip_error(void)
{
    return g_last_hip_error == hipSuccess ? "" : hipGetErrorString(g_last_hip_error);
}

gdn_status gdn_conv_step(const gdn_dims* d, const void* x, const void* conv_w, const void* conv_b,
                         void* conv_state, void* y, const uint8_t* active, int commit_state,
                         int32_t* err, void* stream)
{
    gdn_status st = check_dims(d);
    if (st != GDN_OK) return st;
    st = check_ptrs({x, conv_w, conv_state, y}, {conv_b}, {err});
    if (st != GDN_OK) return st;
    (void)err;
    ConvParams p{};
    p.x = x; p.conv_w = conv_w; p.conv_b = conv_b; p.conv_state = conv_state; p.y = y;
    p.active = active;
    p.L = d->L; p.B = d->B; p.T = d->T; p.C = channels(d);
    p.act = d->act; p.out = d->out; p.flags = d->flags;
    p.commit = commit_state ? 1 : 0;
    return from_hip(gdn::launch_conv(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_verify(const gdn_dims* d, const void* x, const void* conv_w, const void* conv_b,
                      const void* conv_state, const void* g, const void* beta, float* state,
                      const int32_t* cur, void* o, const uint8_t* active, int32_t* err,
                      void* stream)
{
    return verify_impl(d, x, conv_w, conv_b, conv_state, g, beta, state, cur, o, NormEpi{}, active, err,
                       stream);
}

gdn_status gdn_verify_gated_norm(const gdn_dims* d, const void* x, const void* conv_w,
                                 const void* conv_b, const void* conv_state, const void* g,
                                 const void* beta, float* state, const int32_t* cur,
                                 const void* z, const void* norm_w, float norm_eps, void* y,
                                 const uint8_t* active, int32_t* err, void* stream)
{
    if (!z || !norm_w) return GDN_E_NULL;
    NormEpi e;
    e.z = z; e.w = norm_w; e.eps = norm_eps;
    return verify_impl(d, x, conv_w, conv_b, conv_state, g, beta, state, cur, y, e, active, err, stream);
}

gdn_status gdn_commit(const gdn_dims* d, const void* x, void* conv_state, int32_t* cur,
                      const int32_t* keep, const uint8_t* active, int32_t* err, void* stream)
{
    gdn_status st = check_dims(d);
    if (st != GDN_OK) return st;
    if (d->T > 4 || d->S < d->T + 1) return GDN_E_SHAPE;
    if (!cur || !keep) return GDN_E_NULL;
    st = check_ptrs({x, conv_state}, {}, {cur, keep, err});
    if (st != GDN_OK) return st;
    WinParams w{};
    w.x = x; w.conv_state = conv_state; w.cur = cur; w.keep = keep; w.active = active;
    w.err = err; w.L = d->L; w.B = d->B; w.T = d->T; w.S = d->S; w.C = channels(d);
    w.act = d->act; w.mode = gdn::WIN_COMMIT;
    return from_hip(gdn::launch_window(w, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_rewind(const gdn_dims* d, const void* x, const void* conv_w, const void* conv_b,
                      void* conv_state, const void* g, const void* beta, float* state,
                      const int32_t* cur, const int32_t* keep, void* o, int32_t* err,
                      void* stream)
{
    gdn_status st = check_dims(d);
    if (st != GDN_OK) return st;
    if (d->T > 4) return GDN_E_SHAPE;
    if (!keep) return GDN_E_NULL;
    st = check_ptrs({x, conv_w, conv_state, g, beta, state}, {conv_b, o}, {cur, keep, err});
    if (st != GDN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    RecParams p = rec_params(d);
    p.x = x; p.conv_w = conv_w; p.conv_b = conv_b; p.conv_state = conv_state;
    p.g = g; p.beta = beta; p.state = state; p.cur = cur; p.o = o; p.active = nullptr;
    p.keep = keep; p.err = err; p.mode = gdn::REC_REWIND;
    p.conv_out = conv_state;
    bool shifted = false;
    st = from_hip(gdn::launch_recurrent(p, d->DK, d->DV, s, &shifted));
    if (st != GDN_OK || shifted) return st;
    // Otherwise (more waves per qk head than a workgroup holds) the conv cache
    // is shifted by a second launch, after every wave of the replay has read
    // the old cache.
    WinParams w{};
    w.x = x; w.conv_state = conv_state; w.cur = const_cast<int32_t*>(cur); w.keep = keep;
    w.active = nullptr; w.err = err; w.L = d->L; w.B = d->B; w.T = d->T; w.S = d->S;
    w.C = p.C; w.act = d->act; w.mode = gdn::WIN_REWIND;
    return from_hip(gdn::launch_window(w, s));
}

size_t gdn_workspace_size(const gdn_dims* d, int32_t chunk)
{
    if (check_dims(d) != GDN_OK || chunk != 64) return 0;
    return gdn::prefill_workspace_bytes(d->L, d->B, d->T, d->HV, d->DK, d->DV, d->act, chunk);
}

gdn_status gdn_verify_lazy(const gdn_dims* d, const void* x_prev, const void* g_prev,
                           const void* beta_prev, const int32_t* keep_prev, const void* x,
                           const void* conv_w, const void* conv_b, void* conv_state,
                           const void* g, const void* beta, float* state, const int32_t* cur,
                           void* o, const uint8_t* active, int32_t* err, void* stream)
{
    return verify_lazy_impl(d, x_prev, g_prev, beta_prev, keep_prev, x, conv_w, conv_b, conv_state, g, beta,
                            state, cur, o, NormEpi{}, active, err, stream);
}

gdn_status gdn_verify_lazy_gated_norm(const gdn_dims* d, const void* x_prev, const void* g_prev,
                                      const void* beta_prev, const int32_t* keep_prev, const void* x,
                                      const void* conv_w, const void* conv_b, void* conv_state,
                                      const void* g, const void* beta, float* state,
                                      const int32_t* cur, const void* z, const void* norm_w,
                                      float norm_eps, void* y, const uint8_t* active, int32_t* err,
                                      void* stream)
{
    if (!z || !norm_w) return GDN_E_NULL;
    NormEpi e;
    e.z = z; e.w = norm_w; e.eps = norm_eps;
    return verify_lazy_impl(d, x_prev, g_prev, beta_prev, keep_prev, x, conv_w, conv_b, conv_state, g, beta,
                            state, cur, y, e, active, err, stream);
}

gdn_status gdn_accept_greedy(const gdn_dims* d, const int32_t* draft_ids, const int32_t* target_ids,
                             const uint8_t* active, int32_t* keep, int32_t* next_ids, void* stream)
{
    gdn_status st = check_dims(d);
    if (st != GDN_OK) return st;
    if (d->T > 4) return GDN_E_SHAPE;
    if (!target_ids || !keep || (d->T > 1 && !draft_ids)) return GDN_E_NULL;
    st = check_ptrs({}, {}, {draft_ids, target_ids, keep, next_ids});
    if (st != GDN_OK) return st;
    gdn::AcceptParams p{};
    p.draft = d->T > 1 ? draft_ids : nullptr;
    p.target = target_ids; p.active = active; p.keep = keep; p.next = next_ids;
    p.B = d->B; p.T = d->T;
    return from_hip(gdn::launch_accept(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_gated_rmsnorm(const gdn_dims* d, const void* o, const void* z, const void* w,
                             float eps, void* y, const uint8_t* active, void* stream)
{
    gdn_status st = check_dims(d);
    if (st != GDN_OK) return st;
    if (!(eps >= 0.0f)) return GDN_E_SHAPE;
    st = check_ptrs({o, z, w, y}, {}, {});
    if (st != GDN_OK) return st;
    gdn::NormParams p{};
    p.o = o; p.z = z; p.w = w; p.y = y; p.active = active;
    p.L = d->L; p.B = d->B; p.T = d->T; p.HV = d->HV; p.DV = d->DV;
    p.act = d->act; p.out = d->out; p.eps = eps;
    return from_hip(gdn::launch_gated_rmsnorm(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_prefill_ragged(const gdn_dims* d, const void* y, const void* g, const void* beta,
                              float* state, const int32_t* cur, void* o, const int32_t* lengths,
                              int32_t chunk, void* workspace, size_t workspace_bytes, int32_t* err,
                              void* stream)
{
    return prefill_impl(d, y, g, beta, state, cur, o, lengths, chunk, workspace, workspace_bytes, false, err,
                        stream);
}

gdn_status gdn_prefill_chunked_noalloc(const gdn_dims* d, const void* y, const void* g, const void* beta,
                                       float* state, const int32_t* cur, void* o, int32_t chunk, int32_t* err,
                                       void* stream)
{
    return prefill_impl(d, y, g, beta, state, cur, o, nullptr, chunk, nullptr, 0, true, err, stream);
}

gdn_status gdn_prefill_conv_chunked(const gdn_dims* d, const void* x, const void* conv_w, const void* conv_b,
                                    void* conv_state, const void* g, const void* beta, float* state,
                                    const int32_t* cur, void* o, int32_t chunk, void* workspace,
                                    size_t workspace_bytes, int32_t* err, void* stream)
{
    const ConvIn conv{x, conv_w, conv_b, conv_state};
    // y is never read: x stands in for it in the pointer checks
    return prefill_impl(d, x, g, beta, state, cur, o, nullptr, chunk, workspace, workspace_bytes, false, err,
                        stream, &conv);
}


gdn_status gdn_prefill_chunked(const gdn_dims* d, const void* y, const void* g, const void* beta,
                               float* state, const int32_t* cur, void* o, int32_t chunk,
                               void* workspace, size_t workspace_bytes, int32_t* err,
                               void* stream)
{
    return gdn_prefill_ragged(d, y, g, beta, state, cur, o, nullptr, chunk, workspace, workspace_bytes, err,
                              stream);
}

}  // extern "C"
