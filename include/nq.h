/*
 * nq.h -- C ABI of libnq: linear layers whose weight is a low-rank product of
 * bit-packed sign matrices and diagonal scales, on AMD Instinct MI355X (gfx950).
 *
 * The operation (hardwired.dev NanoQuant article, section "Jak NanoQuant
 * funguje": the weight is factored into sign matrices and diagonal scales;
 * rapidrecap.app summary, "Quantization Technique": the sign factors are named
 * U and V), with one diagonal on each side of each sign factor:
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
  NQ_PATH_GEMV = 1,   /* 1 <= B <= 16: sign bits as fp4 MFMA operands, activations as fp8
                         pieces read from global images (4 or 5 launches)                    */
  NQ_PATH_GEMM = 2,   /* any B (auto for B > 16, prefill): signs packed in LDS, expanded to
                         fp16 +-1 in registers; fp16 MFMA with per-row power-of-two activation
                         scales, fp32 accumulate                                             */
  NQ_PATH_VALU = 3,   /* B == 1 only: plain per-bit masked sums on the vector ALU (comparison) */
  NQ_PATH_DECODE = 4  /* 1 <= B <= 16: the decode path, activation images staged in LDS
                         (2 launches per chunk of <= 4 batch rows, 3 when the stage-1
                         partials are too many to fold; B > 4 runs as consecutive chunks) */
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
 * Storage: the r(m+n) sign bits of U and V (padded to whole tiles) and the
 * m+n+r scales (storage rule of hardwired.dev, section "Jak NanoQuant
 * funguje"), plus the header and section alignment. */
size_t nq_layer_bytes(int32_t m, int32_t n, int32_t r, int32_t scale_dtype);

/* Packs sign matrices and scales into L->blob.
 *   U  : device, m x r int8, row-major, every entry exactly +1 or -1
 *   V  : device, n x r int8, row-major, every entry exactly +1 or -1
 *   s1 : device, m values; g : device, r values; s2 : device, n values (L->scale_dtype)
 * The sign factors hold signs only (hardwired.dev, section "Jak NanoQuant
 * funguje"); any other value, 0 included, makes the call return
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

/* Bytes of workspace one path needs for batch B (nq_path); 0 when the path does
 * not take B or for invalid arguments.  NQ_PATH_AUTO gives nq_workspace_bytes. */
size_t nq_workspace_bytes_path(const nq_layer* L, int32_t B, int32_t path);

/* y = x W_hat^T for a batch of B rows.
 *   x : device, B x n row-major, x_dtype NQ_BF16 or NQ_F32, aligned to its element size
 *       (rows that are not 16-byte aligned cost one extra copy launch)
 *   y : device, B x m row-major, y_dtype NQ_BF16 or NQ_F32, aligned to its element size;
 *       must not overlap x
 *   workspace : device, >= nq_workspace_bytes(L, B), 256-byte aligned
 * ASYNCHRONOUS: returns once the kernels are enqueued on `stream`; launch errors
 * are returned, faults surface at the caller's next synchronisation.  B == 0
 * returns NQ_OK and launches nothing.  Stateless and re-entrant; the call
 * sequence may be captured into a HIP graph.  Path chosen automatically:
 * NQ_PATH_DECODE for B <= 16 when its plan fits, else NQ_PATH_GEMV for B <= 16,
 * NQ_PATH_GEMM above. */
nq_status nq_linear_fwd(const nq_layer* L, const void* x, int32_t x_dtype, void* y, int32_t y_dtype,
                        int32_t B, void* workspace, size_t workspace_bytes, nq_stream_t stream);

/* As nq_linear_fwd, with the path forced (nq_path).  NQ_ERR_UNSUPPORTED when
 * the path does not accept B (GEMV: B <= 16; VALU: B == 1). */
nq_status nq_linear_fwd_path(const nq_layer* L, const void* x, int32_t x_dtype, void* y,
                             int32_t y_dtype, int32_t B, void* workspace, size_t workspace_bytes,
                             nq_stream_t stream, int32_t path);

/* Layer groups (the fused block decode).  In a transformer block several
 * linears read the same input: q, k and v, and gate and up (the 70B decode
 * measured on the hardwired.dev NanoQuant page, section "Cisla").  A group of
 * 1..NQ_GROUP_MAX layers with the same n and scale dtype is run on one x:
 * ys[l] = x W_hat_l^T for each l, B x m_l row-major, y_dtype.  For B <= 4 it
 * takes two launches in all: stage 1 over the V^T row tiles of every layer,
 * then a block-diagonal stage 2 (each layer its own U, t and y); larger B
 * runs the layers one after another on their automatic paths.  x must not
 * overlap any ys[l], nor the ys each other; NQ_ERR_INVALID_ARG for a group
 * whose layers differ in n or scale dtype.  Asynchronous like nq_linear_fwd. */
#define NQ_GROUP_MAX 4
size_t nq_workspace_bytes_group(const nq_layer* const* layers, int32_t L, int32_t B);
nq_status nq_linear_fwd_group(const nq_layer* const* layers, int32_t L, const void* x, int32_t x_dtype,
                              void* const* ys, int32_t y_dtype, int32_t B, void* workspace,
                              size_t workspace_bytes, nq_stream_t stream);
/* nq_linear_fwd_group with the timing marks of nq_linear_fwd_profiled (fused
 * path only, NQ_ERR_UNSUPPORTED otherwise). */
nq_status nq_linear_fwd_group_profiled(const nq_layer* const* layers, int32_t L, const void* x,
                                       int32_t x_dtype, void* const* ys, int32_t y_dtype, int32_t B,
                                       void* workspace, size_t workspace_bytes, nq_stream_t stream,
                                       void* const* events, int32_t n_events, int32_t* n_launches,
                                       int32_t* launch_dims);

/* The transposed product (the backward pass through a binary layer that block
 * reconstruction needs; hardwired.dev NanoQuant page, section "Trikrokovy
 * pipeline", step 3).  W_hat^T = diag(s2) V diag(g) U^T diag(s1) has the same
 * form with the roles swapped: U' = V, V' = U, s1' = s2, g' = g, s2' = s1.
 * Writes that layer into dst (dst->m = src->n, dst->n = src->m, dst->r =
 * src->r, same scale dtype, nq_layer_bytes(src->n, src->m, src->r) bytes, not
 * overlapping src): header, bit-transposed factors (padding bits zero, as
 * nq_pack_factors writes them) and the scales.  Then nq_linear_fwd(dst, dy)
 * gives dx[b] = W_hat^T dy[b] for dy of shape B x src->m, on every path.
 * BLOCKING: synchronises `stream`. */
nq_status nq_transpose_layer(const nq_layer* src, const nq_layer* dst, nq_stream_t stream);

/* Rank-l envelope (the MDBF variant; hardwired.dev NanoQuant page, section
 * "Kontext: co existuje kolem", MDBF: the single magnitude profile of DBF,
 * which is the form of nq_linear_fwd, replaced by an envelope of rank l).
 * Reading: W_hat = sum_t diag(s1_t) U diag(g) V^T diag(s2_t), t < env, with
 * U, V^T and g from the layer's blob and the env scale-vector pairs given here:
 * s1_env (env x m) and s2_env (env x n), device, row-major, scale dtype of the
 * layer (the blob's own s1 and s2 are not used).  y = x W_hat^T, x B x n, y
 * B x m.  The sign bits are read once for all terms (the env terms run as
 * extra batch rows and are summed in registers), so B x env <= 4, env <=
 * NQ_ENVELOPE_MAX; otherwise NQ_ERR_UNSUPPORTED.  The workspace holds padded
 * copies of the scale pairs plus the forward's own scratch. */
#define NQ_ENVELOPE_MAX 4
size_t nq_workspace_bytes_envelope(const nq_layer* L, int32_t env, int32_t B);
nq_status nq_linear_fwd_envelope(const nq_layer* L, int32_t env, const void* s1_env, const void* s2_env,
                                 const void* x, int32_t x_dtype, void* y, int32_t y_dtype, int32_t B,
                                 void* workspace, size_t workspace_bytes, nq_stream_t stream);

/* Bytes of the static device scratch used by nq_linear_fwd_noalloc. */
#define NQ_NOALLOC_SCRATCH_BYTES (16u << 20)

/* As nq_linear_fwd (automatic path), for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The intermediates live in a static
 * device array of NQ_NOALLOC_SCRATCH_BYTES (16 MiB) that every GPU the library
 * runs on holds until the process ends; nothing is allocated or freed.
 * NQ_ERR_WORKSPACE when the call needs more scratch than that (large prefill
 * batches: use nq_linear_fwd with a workspace).  All calls on one GPU share
 * that GPU's scratch: calls that overlap in time on one GPU (other streams,
 * other host threads) race and must be serialised by the caller.  The scratch
 * needs no initial contents.  The first call on a device resolves the
 * scratch's address on that device (with that device current). */
nq_status nq_linear_fwd_noalloc(const nq_layer* L, const void* x, int32_t x_dtype, void* y,
                                int32_t y_dtype, int32_t B, nq_stream_t stream);

/* As nq_linear_fwd_path, and for timing each kernel of the call: records
 * events[k] (hipEvent_t handles created by the caller) on `stream` just before
 * the k-th kernel launch and events[K] after the last of the K launches, for
 * the first n_events of them; *n_launches receives K.  If launch_dims is not
 * NULL it receives, for each of the first n_events - 1 launches, the number of
 * workgroups and the threads per workgroup (2 int32 per launch), so that a
 * profiler's dispatch records can be matched to the launches.  Only
 * NQ_PATH_DECODE and NQ_PATH_GEMM (or AUTO resolving to them) record marks;
 * other paths return NQ_ERR_UNSUPPORTED.  The launches are those of
 * nq_linear_fwd_path, in order (decode: stage 1, [mid image,] stage 2; gemm:
 * x image, product with V^T, t image, product with U). */
nq_status nq_linear_fwd_profiled(const nq_layer* L, const void* x, int32_t x_dtype, void* y,
                                 int32_t y_dtype, int32_t B, void* workspace, size_t workspace_bytes,
                                 nq_stream_t stream, int32_t path, void* const* events,
                                 int32_t n_events, int32_t* n_launches, int32_t* launch_dims);

/* Initialiser of the factors from a dense weight (hardwired.dev NanoQuant
 * page, section "Trikrokovy pipeline", step 2 and the paragraph after it:
 * an ADMM method whose iterations solve for the real-valued part by least
 * squares in closed form and then map onto the +-1 set by taking signs).  Reading, with an identity
 * Hessian: minimise ||W - A B^T||_F^2 with A = diag(s1) U diag(qA) and
 * B = diag(s2) V diag(qB); `iters` ADMM steps of penalty rho from the latent
 * factors A0, B0:
 *   A <- (W B + rho (ZA - LA)) (B^T B + rho I)^-1,  B <- (W^T A + rho (ZB - LB)) (A^T A + rho I)^-1,
 *   ZA <- proj(A + LA), ZB <- proj(B + LB), LA += A - ZA, LB += B - ZB,
 * proj(Y) = diag(p) sign(Y) diag(q) with (p, q) the leading singular pair of
 * |Y| from `power_iters` power steps (sign(0) = +1; ZA, ZB start at proj(A0),
 * proj(B0), the duals at 0).  Outputs (device, caller-owned): U (m x r) and V
 * (n x r) int8 +-1 row-major, s1 (m), g = qA qB (r), s2 (n) fp32, ready for
 * nq_pack_factors (after conversion to the scale dtype); if err is not NULL,
 * err[t] = ||W - W_hat_t||_F^2 / ||W||_F^2 after t steps, t = 0..iters.
 * Inputs: W (m x n), A0 (m x r), B0 (n x r), device fp32 row-major, 4-byte
 * aligned, not overlapping the outputs or the workspace.  All arithmetic is
 * fp32 (MFMA products, Gauss-Jordan inverse of the r x r Gram matrices) with
 * fixed reduction orders: repeated calls give identical bits.  rho > 0,
 * 0 <= iters <= 10000, 0 <= power_iters <= 1000, r <= min(m, n, 4096),
 * max(m, n) x r < 2^31, else NQ_ERR_INVALID_ARG; NQ_ERR_WORKSPACE for a
 * short workspace.  err is NaN when W is all zeros.  Asynchronous on `stream`. */
size_t nq_admm_workspace_bytes(int32_t m, int32_t n, int32_t r);
nq_status nq_admm_factorize(const float* W, int32_t m, int32_t n, int32_t r, const float* A0, const float* B0,
                            float rho, int32_t iters, int32_t power_iters, int8_t* U, int8_t* V, float* s1,
                            float* g, float* s2, float* err, void* workspace, size_t workspace_bytes,
                            nq_stream_t stream);

/* Magnitude balancing (same page and section, the paragraph after step 2,
 * which applies it after the initialiser to the scale factors).  In place on
 * device fp32 s1 (m), g (r), s2 (n): s1 *= c, s2 *= d, g /= c d with c, d the
 * powers of two that put the root-mean-square of s1 and of s2 in [1, 2) (1 for
 * a zero or non-finite one), so neither side's scales sit far from unit size.
 * W_hat is unchanged bit for bit.  NQ_ERR_INVALID_ARG for null pointers or
 * dimensions out of range.  Asynchronous on `stream`. */
nq_status nq_balance_scales(float* s1, float* g, float* s2, int32_t m, int32_t n, int32_t r, nq_stream_t stream);

/* Average bits per original weight: (r(m+n) + scale_bits (m+n+r)) / (m n)
 * (hardwired.dev, sections "Jak NanoQuant funguje" and 'Co znamena
 * "sub-1-bit"').  Padding is not counted.  Returns -1.0 for invalid arguments. */
double nq_bits_per_weight(int32_t m, int32_t n, int32_t r, int32_t scale_bits);

/* Largest rank r >= 1 with nq_bits_per_weight(m, n, r, scale_bits) <= bpw;
 * 0 when even r = 1 exceeds bpw; -1 for invalid arguments. */
int32_t nq_rank_for_bits(int32_t m, int32_t n, double bpw, int32_t scale_bits);

/* Measurement aid, not part of the layer's arithmetic: reads `bytes` of device
 * memory at `buf` once, with the load pattern of the forward kernels' weight
 * stream (each wave keeps sixteen 1 KiB loads in flight), and XORs every
 * 32-bit word into *sink (device memory, which the caller initialises; the
 * call adds XOR(words) to it).  Timing the call with events gives the read
 * rate a kernel of that shape reaches for that many bytes.  `bytes` must be a
 * positive multiple of 16384, `buf` 16-byte aligned, `sink` 4-byte aligned
 * and outside buf; NQ_ERR_INVALID_ARG otherwise.  If grid is not NULL it
 * receives the workgroups and threads per workgroup of the launch.
 * Asynchronous on `stream`. */
nq_status nq_read_probe(const void* buf, size_t bytes, uint32_t* sink, nq_stream_t stream, int32_t* grid);

/* Static text for a status code. */
const char* nq_status_string(int32_t status);

/* Detail text for the last failed call on this thread ("" if none). */
const char* nq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* NQ_H_ */
