/*
 * nq.h -- C ABI of libnq: linear layers whose weight is a low-rank product of
 * bit-packed sign matrices and diagonal scales, on AMD Instinct MI355X (gfx950).
 *
 * The operation (NanoQuant pages: hardwired.dev article, section "Jak NanoQuant
 * funguje" -- the weight matrix is approximated by a product of binary matrices
 * holding only +1 and -1 and of diagonal scaling vectors; rapidrecap.app
 * summary, "Quantization Technique" -- the binary matrices are called U and V):
 *
 *     W_hat = diag(s1) . U . diag(g) . V^T . diag(s2)        (m x n)
 *     U in {-1,+1}^(m x r),  V in {-1,+1}^(n x r),  s1: m,  g: r,  s2: n
 *     y[b,:] = W_hat . x[b,:]  =  s1 * (U (g * (V^T (s2 * x[b,:]))))
 *
 * m is the number of output features and n the number of input features (the
 * orientation of a PyTorch linear layer).  W_hat is never formed: the kernels
 * read the packed sign bits and compute each product of a sign matrix with a
 * vector v as  2 * sum_{bit = 1} v - sum v  (bit 1 stands for +1, bit 0 for -1).
 *
 * Memory and threading conventions, for every entry point:
 *  - Every device buffer (layer blob, x, y, workspace) is allocated and freed by
 *    the caller.  The library never allocates or frees device memory.
 *  - Arguments are validated on the host before any HIP call; a bad argument
 *    returns an error code and launches nothing.  No C++ exception, abort or
 *    print crosses this interface.  nq_last_error() gives a text for the last
 *    failure on the calling thread.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 */
#ifndef NQ_H_
#define NQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NQ_ABI_VERSION 1

typedef enum {
  NQ_OK = 0,
  NQ_ERR_INVALID_ARG = -1, /* null pointer, dimension <= 0 or too large, bad dtype, misalignment */
  NQ_ERR_NOT_PM1 = -2,     /* a U or V entry is not exactly +1 or -1 (pack only)                */
  NQ_ERR_WORKSPACE = -3,   /* workspace smaller than nq_workspace_bytes()                         */
  NQ_ERR_UNSUPPORTED = -4, /* valid arguments that the chosen path does not handle                */
  NQ_ERR_HIP = -5,         /* a HIP runtime call or launch failed; see nq_last_error()           */
  NQ_ERR_INTERNAL = -6
} nq_status;

typedef enum { NQ_F32 = 0, NQ_F16 = 1, NQ_BF16 = 2 } nq_dtype;

/* Which kernels run the forward.  AUTO picks by batch size. */
typedef enum {
  NQ_PATH_AUTO = 0,
  NQ_PATH_GEMV = 1, /* 1 <= B <= 16: sign bits as fp4 MFMA operands, activations as fp8 pieces */
  NQ_PATH_GEMM = 2, /* any B: sign bits expanded to fp16 +-1 in registers, fp16 MFMA          */
  NQ_PATH_VALU = 3  /* B == 1 only: plain per-bit masked sums on the vector ALU (comparison)  */
} nq_path;

/* A packed layer.  `blob` is device memory of nq_layer_bytes(m, n, r, scale_dtype)
 * bytes, 256-byte aligned, owned by the caller and written by nq_pack_factors:
 * a 256-byte header, then the packed U, the packed V^T, then s1, g, s2 in
 * scale_dtype.  The blob is position independent and may be copied bytewise. */
typedef struct {
  int32_t m, n, r;     /* W_hat is m x n; rank r.  1 <= m, n <= 2^20, 1 <= r <= 2^16 */
  int32_t scale_dtype; /* nq_dtype of s1, g, s2: NQ_F16 or NQ_F32                    */
  void* blob;          /* device pointer                                              */
} nq_layer;

typedef void* nq_stream_t; /* hipStream_t */

/* Version of this interface (NQ_ABI_VERSION). */
int32_t nq_abi_version(void);

/* Bytes of device memory a packed layer occupies; 0 for invalid arguments.
 * Storage is r(m+n) sign bits (padded to whole tiles) plus the m+n+r scales
 * (hardwired.dev article, section "Jak NanoQuant funguje": r x (m+n) binary
 * values plus the scaling parameters). */
size_t nq_layer_bytes(int32_t m, int32_t n, int32_t r, int32_t scale_dtype);

/* Packs sign matrices and scales into L->blob.
 *   U  : device, m x r int8, row-major, every entry exactly +1 or -1
 *   V  : device, n x r int8, row-major, every entry exactly +1 or -1
 *   s1 : device, m values; g : device, r values; s2 : device, n values (L->scale_dtype)
 * The pages allow only +1 and -1 in the binary factors (hardwired.dev, section
 * "Jak NanoQuant funguje"); any other value, 0 included, makes the call return
 * NQ_ERR_NOT_PM1 (the blob is then unusable).  BLOCKING: synchronises `stream`
 * to read the validation result.  The scales are copied, so the inputs may be
 * freed afterwards. */
nq_status nq_pack_factors(const nq_layer* L, const int8_t* U, const int8_t* V, const void* s1,
                          const void* g, const void* s2, nq_stream_t stream);

/* Inverse of the sign part of nq_pack_factors: writes U (m x r) and V (n x r)
 * as int8 +-1 into caller buffers.  Test hook.  BLOCKING on `stream`. */
nq_status nq_unpack_factors(const nq_layer* L, int8_t* U, int8_t* V, nq_stream_t stream);

/* Bytes of device workspace nq_linear_fwd needs for batch B, for every path that
 * accepts B.  The workspace holds only intermediates (the rank-r vector t for
 * each row of x and its encodings); it needs no initial contents and is free
 * for other use between calls. */
size_t nq_workspace_bytes(const nq_layer* L, int32_t B);

/* y = x W_hat^T for a batch of B rows.
 *   x : device, B x n row-major, x_dtype NQ_BF16 or NQ_F32, 4-byte aligned
 *   y : device, B x m row-major, y_dtype NQ_BF16 or NQ_F32, 4-byte aligned; must not overlap x
 *   workspace : device, >= nq_workspace_bytes(L, B), 256-byte aligned
 * ASYNCHRONOUS: returns once the kernels are enqueued on `stream`; launch errors
 * are returned, faults surface at the caller's next synchronisation.  B == 0
 * returns NQ_OK and launches nothing.  Stateless and re-entrant; the call
 * sequence may be captured into a HIP graph.  Path chosen automatically:
 * NQ_PATH_GEMV for B <= 16, NQ_PATH_GEMM above. */
nq_status nq_linear_fwd(const nq_layer* L, const void* x, int32_t x_dtype, void* y, int32_t y_dtype,
                        int32_t B, void* workspace, size_t workspace_bytes, nq_stream_t stream);

/* As nq_linear_fwd, with the path forced (nq_path).  NQ_ERR_UNSUPPORTED when
 * the path does not accept B (GEMV: B <= 16; VALU: B == 1). */
nq_status nq_linear_fwd_path(const nq_layer* L, const void* x, int32_t x_dtype, void* y,
                             int32_t y_dtype, int32_t B, void* workspace, size_t workspace_bytes,
                             nq_stream_t stream, int32_t path);

/* Average bits per original weight: (r(m+n) + scale_bits (m+n+r)) / (m n)
 * (hardwired.dev, sections "Jak NanoQuant funguje" and 'Co znamena
 * "sub-1-bit"').  Padding is not counted.  Returns -1.0 for invalid arguments. */
double nq_bits_per_weight(int32_t m, int32_t n, int32_t r, int32_t scale_bits);

/* Largest rank r >= 1 with nq_bits_per_weight(m, n, r, scale_bits) <= bpw;
 * 0 when even r = 1 exceeds bpw; -1 for invalid arguments. */
int32_t nq_rank_for_bits(int32_t m, int32_t n, double bpw, int32_t scale_bits);

/* Static text for a status code. */
const char* nq_status_string(int32_t status);

/* Detail text for the last failed call on this thread ("" if none). */
const char* nq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NQ_H_ */
