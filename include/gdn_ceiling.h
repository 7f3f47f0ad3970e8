/*
 * gdn_ceiling.h -- C ABI of libgdn_ceiling.so: hand-written HBM stream and
 * matrix-core loops that measure what one MI355X (gfx950) actually sustains,
 * so that the path's kernels are priced against a measured ceiling beside the
 * vendor peak (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s).  Measurement
 * infrastructure, not part of the Gated DeltaNet path.
 *
 * Every pointer is a caller-owned device pointer, 16-byte aligned; calls are
 * asynchronous on `stream` (a hipStream_t, NULL = legacy default stream) and
 * allocate, free and synchronise nothing.  Return value: 0 on success, -1 on
 * a bad argument (nothing launched), or the HIP error code of the launch.
 */
#ifndef GDN_CEILING_H
#define GDN_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streams n_vec16 16-byte vectors: reads the first n_read buffers of src[]
 * (0..2) and writes the first n_write buffers of dst[] (0..3), element for
 * element; each written vector is the sum of the read vectors (or a constant
 * when n_read = 0).  With n_write = 0 the read sums are folded and written as
 * one 16-byte vector per workgroup into sink (at least grid vectors).  grid
 * workgroups of 256 threads walk the buffers with a stride of the whole grid;
 * each thread moves unroll (1, 2, 4 or 8) vectors per buffer per pass, all
 * loads of a pass issued before its stores.  mode bit 0: loads and stores
 * are non-temporal; bit 1: blocked layout -- workgroup g streams the
 * contiguous 64 KiB blocks g, g + grid, ... instead of the grid striding
 * over the whole buffer. */
int gdn_ceiling_stream(const void* const* src, int n_read, void* const* dst, int n_write,
                       size_t n_vec16, void* sink, int grid, int unroll, int mode,
                       void* stream);

/* Dense bf16 matrix-core loop: grid workgroups of 256 threads (4 waves); each
 * wave runs iters rounds of 8 independent v_mfma_f32_16x16x32_bf16 chains on
 * register operands (16,384 flops per instruction) and writes its
 * accumulators to out (grid * 256 * 32 floats) so nothing is dead code.
 * flops = grid * 4 * iters * 8 * 16384. */
int gdn_ceiling_mfma_bf16(float* out, int grid, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_CEILING_H */
