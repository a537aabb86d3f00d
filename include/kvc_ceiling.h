/*
 * kvc_ceiling.h -- C ABI of libkvc_ceiling.so: streaming kernels that move
 * the bytes of the compressed-KV path's two headline kernels with no
 * arithmetic, used by the benchmark as a yardstick measured under the same
 * cache conditions as the kernels themselves.  They are not part of the path
 * (nothing in kvc.h calls them) and compute nothing of the method.
 *
 * Conventions: device pointers, 16-byte aligned; `stream` is a hipStream_t
 * (NULL = default stream); every call is asynchronous and allocates nothing.
 * Return 0 on success, -1 for a bad argument (nothing launched), -3 when the
 * launch fails.
 */
#ifndef KVC_CEILING_H
#define KVC_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* `items` units of the ratio-2 compressor's traffic for two rows into a
 * V41_FP4 cache: item i reads src[i*8192 .. +8192) bytes and writes
 * latent[i*2048 .. +2048), data[i*512 .. +512) and scale[i*64 .. +64).
 * Buffers must hold items times those sizes. */
int kvc_ceiling_compress_shape(const void* src, void* latent, void* data, void* scale,
                               int64_t items, void* stream);

/* `rows` units of the V41 dequant-gather's traffic with contiguous rows:
 * row r reads src[r*528 .. +528) and writes out[r*1024 .. +1024). */
int kvc_ceiling_gather_shape(const void* src, void* out, int64_t rows, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVC_CEILING_H */
