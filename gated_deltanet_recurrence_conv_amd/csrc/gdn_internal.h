// gdn_internal.h -- kernel parameter blocks, launchers and small device
// helpers shared by the HIP sources of libgdn.so.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#ifndef GDN_PERMLANE_SWAP
#define GDN_PERMLANE_SWAP 1
#endif

namespace gdn {

enum { ACT_F32 = 0, ACT_BF16 = 1 };
enum { FLAG_SILU = 1u, FLAG_L2 = 2u };
enum { ERR_KEEP = 1, ERR_SLOT = 2, ERR_INACTIVE_KEEP = 4, ERR_LENGTH = 8 };

// ---------------------------------------------------------------------------
// Recurrent step kernel (verify and rewind share it, so that a rewind is
// bit-identical to the verify candidate it replaces).
enum RecMode { REC_VERIFY = 0, REC_REWIND = 1, REC_LAZY = 2 };

struct RecParams {
    const void* x;
    const void* x_prev;      // lazy mode: the previous window's x, g, beta
    const void* g_prev;
    const void* beta_prev;
    const void* conv_w;
    const void* conv_b;
    const void* conv_state;
    const void* g;
    const void* beta;
    float* state;
    const int32_t* cur;
    void* o;
    const uint8_t* active;
    const int32_t* keep;
    int32_t* err;
    int32_t L, B, T, HV, HK, S, C;
    int32_t act, out;
    float scale, l2_eps;
    uint32_t flags;
    int32_t mode;
    int32_t groups;     // L * B * HK
    int32_t per_group;  // workgroups per (layer, row, qk head)
    const void* z;      // gated RMSNorm epilogue: gate input [L][B][T][HV][DV] (act)
    const void* norm_w; // and weight [L][DV] (act); null: o is written raw
    float norm_eps;
    void* conv_out;     // lazy / rewind with one workgroup per qk head: the conv
                        // cache (= conv_state) that the kernel itself shifts
};

// ---------------------------------------------------------------------------
// Conv-window shift (commit, rewind, conv_step with commit_state).
enum WinMode { WIN_COMMIT = 0, WIN_REWIND = 1 };

struct WinParams {
    const void* x;
    void* conv_state;
    int32_t* cur;
    const int32_t* keep;
    const uint8_t* active;
    int32_t* err;
    int32_t L, B, T, S, C;
    int32_t act;
    int32_t mode;
};

// ---------------------------------------------------------------------------
// Standalone conv step (y over all tokens).
struct ConvParams {
    const void* x;
    const void* conv_w;
    const void* conv_b;
    void* conv_state;
    void* y;
    const uint8_t* active;
    int32_t L, B, T, C;
    int32_t act, out;
    uint32_t flags;
    int32_t commit;   // also shift the cache by T tokens
};

// Drops an error a previous runtime call may have left behind, so that the
// status read right after a launch belongs to that launch.
inline void clear_stale_error() { (void)hipGetLastError(); }

// Compute units of the current device, queried once per device (0 if the
// query fails; callers then keep their default launch shape).
inline int device_cus()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            clear_stale_error();
            return 0;
        }
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// *conv_shifted (if given) tells a lazy or rewind caller whether the launch
// also shifted the conv cache (p.conv_out), so that no window launch follows.
hipError_t launch_recurrent(const RecParams& p, int DK, int DV, hipStream_t s, bool* conv_shifted = nullptr);
hipError_t launch_window(const WinParams& p, hipStream_t s);
hipError_t launch_conv(const ConvParams& p, hipStream_t s);

// Chunked prefill.
struct PrefillParams {
    const void* y;
    const void* g;
    const void* beta;
    float* state;
    const int32_t* cur;
    void* o;
    void* ws;
    int32_t* err;
    const int32_t* lengths;   // per-row prompt length (ragged), or null: all T
    int32_t L, B, T, HV, HK, S, C;
    int32_t act, out;
    float scale, l2_eps;
    uint32_t flags;
    // fused conv (x non-null): y is the short conv (+ SiLU) of [conv_state ; x],
    // computed inside the prep kernel and rounded to the act dtype, and the
    // scan kernel commits conv_state <- the last 3 window rows
    const void* x;
    const void* conv_w;
    const void* conv_b;
    void* conv_state;
};
// Greedy acceptance of a verification window.
struct AcceptParams {
    const int32_t* draft;    // [B][T-1] (null when T == 1)
    const int32_t* target;   // [B][T]
    const uint8_t* active;   // [B] or null
    int32_t* keep;           // [B]
    int32_t* next;           // [B] or null
    int32_t B, T;
};
hipError_t launch_accept(const AcceptParams& p, hipStream_t s);

// Gated RMSNorm epilogue.
struct NormParams {
    const void* o;        // [L][B][T][HV][DV], out dtype
    const void* z;        // same shape, act dtype
    const void* w;        // [L][DV], act dtype
    void* y;              // like o (may alias it)
    const uint8_t* active;
    int32_t L, B, T, HV, DV;
    int32_t act, out;
    float eps;
};
hipError_t launch_gated_rmsnorm(const NormParams& p, hipStream_t s);

bool prefill_supported(int DK, int DV, int act);
bool prefill_conv_supported(int DK, int DV, int act);
size_t prefill_workspace_bytes(int L, int B, int T, int HV, int DK, int DV, int act, int chunk);
hipError_t launch_prefill(const PrefillParams& p, int DK, int DV, hipStream_t s);
// fp32 form of the chunked prefill (fp32 activations, d_k = 16): no workspace.
hipError_t launch_prefill_f32(const PrefillParams& p, int DK, int DV, hipStream_t s);

// ---------------------------------------------------------------------------
// Device helpers.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t u)
{
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

typedef __bf16 gdn_bf16x2 __attribute__((ext_vector_type(2)));
typedef float gdn_f32x2 __attribute__((ext_vector_type(2)));

// float -> bf16 bits, round to nearest, ties to even (gfx950's
// v_cvt_pk_bf16_f32; NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> packed bf16x2 (a in the low half), one instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b)
{
    const gdn_f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, gdn_bf16x2));
}

// Activation element as fp32; ACT is a compile-time dtype so that loads are
// never serialised behind a runtime dtype branch.
template <int ACT>
__device__ __forceinline__ float load_act(const void* base, size_t idx)
{
    if constexpr (ACT == ACT_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
    else return static_cast<const float*>(base)[idx];
}

// fp32 -> activation element (exact for a value that was loaded from it).
template <int ACT>
__device__ __forceinline__ void store_act(void* base, size_t idx, float v)
{
    if constexpr (ACT == ACT_BF16) static_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(v);
    else static_cast<float*>(base)[idx] = v;
}

// Workgroup barrier over LDS only: waits for this wave's LDS accesses, then
// for the other waves.  __syncthreads() also fences global memory, which on
// this architecture means waiting for every global load and store the wave
// has in flight (one counter covers both), so a prefetch issued before the
// barrier is waited for there and stores just issued stall the next phase.
// For kernels whose workgroups never read global memory they wrote
// themselves, LDS is all a barrier has to order.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// SiLU with the hardware exp2 and reciprocal (each within about 1 ulp):
// v * 1 / (1 + 2^(-v log2 e)).  Saturates to v and -0 at the extremes.
__device__ __forceinline__ float silu_hw(float v)
{
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
}

// Loads 8 contiguous activation values as fp32.
template <int ACT>
__device__ __forceinline__ void load_vec8(const void* base, size_t idx, float* v)
{
    if constexpr (ACT == ACT_BF16) {
        const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
        const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// 8 activation values held as raw 16-byte vectors -> fp32.
template <int ACT>
__device__ __forceinline__ void to_f32x8(const uint4 (&raw)[ACT == ACT_BF16 ? 1 : 2], float* v)
{
    if constexpr (ACT == ACT_BF16) {
        const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
    }
}

// Conv taps and bias of 8 consecutive channels (first channel index c0 of
// layer l's [C] axis, i.e. l * C + channel): w[j][c] multiplies window row j
// (row 3 = the token itself); a missing bias is 0.
template <int ACT>
__device__ __forceinline__ void conv_taps8(const void* conv_w, const void* conv_b, size_t lc0, float (&w)[4][8],
                                           float (&bias)[8])
{
    // conv_w[l][c][0..3] for 8 channels = 32 contiguous values
    float wr[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) load_vec8<ACT>(conv_w, lc0 * 4 + 8 * q, wr + 8 * q);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j][c] = wr[c * 4 + j];
    if (conv_b) {
        load_vec8<ACT>(conv_b, lc0, bias);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) bias[c] = 0.0f;
    }
}

// The short causal conv (+ SiLU) of 8 channels at one token from its 4 window
// rows; every kernel that computes the conv goes through this, so they all
// produce the same bits.
__device__ __forceinline__ void conv8_token(const float (&w)[4][8], const float (&win)[4][8], const float (&bias)[8],
                                            bool use_silu, float (&y)[8])
{
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float acc = w[0][c] * win[0][c];
        acc = fmaf(w[1][c], win[1][c], acc);
        acc = fmaf(w[2][c], win[2][c], acc);
        acc = fmaf(w[3][c], win[3][c], acc);
        acc += bias[c];
        y[c] = use_silu ? silu_hw(acc) : acc;
    }
}


// v + v[lane ^ OFF] across a wave64, OFF a power of two.  Lanes 8 apart
// inside a 16-lane row trade values with a DPP row rotation (row_ror:8 maps
// lane i of a row to i ^ 8), lanes 16 and 32 apart with a permlane swap;
// other distances go through ds_bpermute.  Both lanes of a pair add the same
// two values, so they hold the same sum.
template <int OFF>
__device__ __forceinline__ float xor_add(float v)
{
#if GDN_PERMLANE_SWAP
    // gfx950 permlane swaps: lanes 32 apart (rows 2-3 <-> 0-1) and 16 apart
    // (odd <-> even rows), on two copies of v, as one instruction whose two
    // registers are both read and written (s_nop: the VALU write -> permlane
    // read hazard).  Written as inline assembly because the compiler's
    // __builtin_amdgcn_permlane{16,32}_swap drops the second result here
    // (it adds the first result to itself).  Measured against ds_bpermute at
    // the B8/T2 cohort: one-layer verify 9.3 against 9.5 us, fused commit +
    // verify over 30 layers 148 against 171 us.
    if constexpr (OFF == 32 || OFF == 16) {
        unsigned x = __builtin_bit_cast(unsigned, v), y = x;
        if constexpr (OFF == 32)
            asm volatile("s_nop 4\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
        else
            asm volatile("s_nop 4\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
        return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
    }
#endif
    if constexpr (OFF == 8) {
        return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf,
                                                                         0xf, false));
    } else {
        return v + __shfl_xor(v, OFF, 64);
    }
}

}  // namespace gdn
