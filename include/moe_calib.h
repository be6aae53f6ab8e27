/*
 * moe_calib.h -- C ABI of libmoe_calib.so: measurement kernels that move
 * bytes in the shapes of the MoE dispatch and combine kernels but compute
 * nothing the method needs.  They give the ceilings the method's kernels are
 * compared with on the same device (a plain streaming copy, streams with the
 * read/write mix of each kernel, and the kernels' own access shapes with the
 * arithmetic taken out).  Nothing here is part of the dispatch / combine path.
 *
 * Conventions: pointers are device memory owned by the caller; every call
 * enqueues one kernel on `stream` (a hipStream_t; NULL = the legacy default
 * stream) and returns MOE_CALIB_OK, or MOE_CALIB_EINVAL (nothing enqueued)
 * for NULL pointers, misaligned pointers (16 bytes) or sizes that are not a
 * multiple of 16 or exceed 2^31 bytes, or MOE_CALIB_ELAUNCH if the launch
 * failed.  Buffers are only read or written within the sizes passed.
 */
#ifndef MOE_CALIB_H
#define MOE_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MOE_CALIB_OK = 0, MOE_CALIB_EINVAL = 1, MOE_CALIB_ELAUNCH = 3 };

/* Cache policy of the kernels' stores (loads of streamed data are
 * non-temporal; rows read by several blocks use the default policy). */
enum { MOE_CALIB_STORE_PLAIN = 0,     /* default (write-back in L2)            */
       MOE_CALIB_STORE_STREAM = 1,    /* non-temporal                          */
       MOE_CALIB_STORE_DEVICE = 2 };  /* device scope: written through to memory */

/*
 * A streaming kernel that reads read_bytes of src and writes write_bytes of
 * dst, both contiguous, spread evenly over one-shot blocks so that reads and
 * writes interleave in the given proportion (write_bytes = read_bytes: a
 * plain copy; 73.4 : 14.7 MB the combine's mix; 7.3 : 30.3 MB the
 * dispatch's).  Each wave access covers a contiguous kilobyte; loads are
 * non-temporal, stores take store_policy.  dst receives a function of src.
 */
int moe_calib_stream(const void *src, size_t read_bytes, void *dst, size_t write_bytes,
                     int store_policy, void *stream);

/*
 * The dispatch's access shape without the routing or the quantisation: block
 * i reads row i of x (bf16 [Bs, H]) and the K row numbers assist[i*K + k]
 * (int32, -1 = skip; each < n_rows), and writes one byte per element of the
 * row to each of those rows of out ([n_rows, H] bytes) -- the bytes an
 * 8-bit dispatch moves, in its order.  H in [1024, 8192] with H % 32 == 0,
 * 0 < Bs <= 512, 0 < K <= 16, n_rows <= Bs*K.  Stores take store_policy.
 */
int moe_calib_scatter_shape(const void *x, const int32_t *assist, int Bs, int H, int K,
                            int n_rows, void *out, int store_policy, void *stream);

/*
 * The combine's access shape without its arithmetic: block i reads the rows
 * rows[assist[i*K + k]] (bf16 [n_rows, H]; -1 = skip), row i of a and of b
 * (bf16 [Bs, H]; b may be NULL: the combine without a shared expert) and
 * gamma (bf16 [H]), adds them as integers, and writes two
 * rows (out1[i], out2[i], bf16 [Bs, H]) -- the bytes the combine moves, in
 * its order, with one block barrier like the RMSNorm's.  Limits as
 * moe_calib_scatter_shape; stores take store_policy.
 */
int moe_calib_gather_shape(const void *rows, const int32_t *assist, const void *a,
                           const void *b, const void *gamma, int Bs, int H, int K, int n_rows,
                           void *out1, void *out2, int store_policy, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CALIB_H */
