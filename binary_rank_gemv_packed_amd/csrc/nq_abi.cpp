// C ABI of libnq (declared in include/nq.h).  Every argument is validated on the
// host before any HIP call, so every error path is reachable without a GPU.
#include "nq.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "nq_common.h"
#include "nq_internal.h"

namespace {

thread_local std::string g_last_error;

nq_status fail(nq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

nq_status ok() {
  g_last_error.clear();
  return NQ_OK;
}

constexpr int32_t MAX_DIM = 1 << 20;
constexpr int32_t MAX_RANK = 1 << 16;
constexpr int32_t MAX_BATCH = 1 << 20;
constexpr int32_t DEC_MAX_BATCH = 16;  // the decode path runs B > 4 as chunks of at most 4 rows

int scale_bytes(int32_t dt) { return dt == NQ_F32 ? 4 : (dt == NQ_F16 ? 2 : 0); }
int act_bytes(int32_t dt) { return dt == NQ_F32 ? 4 : (dt == NQ_BF16 ? 2 : 0); }

bool dims_ok(int32_t m, int32_t n, int32_t r) {
  return m >= 1 && m <= MAX_DIM && n >= 1 && n <= MAX_DIM && r >= 1 && r <= MAX_RANK;
}

nq_status check_layer(const nq_layer* L) {
  if (!L) return fail(NQ_ERR_INVALID_ARG, "layer is NULL");
  if (!dims_ok(L->m, L->n, L->r))
    return fail(NQ_ERR_INVALID_ARG, "dimensions out of range: m=%d n=%d r=%d (1..%d, rank 1..%d)", L->m, L->n, L->r,
                MAX_DIM, MAX_RANK);
  if (!scale_bytes(L->scale_dtype)) return fail(NQ_ERR_INVALID_ARG, "scale_dtype %d is not NQ_F16 or NQ_F32", L->scale_dtype);
  if (!L->blob) return fail(NQ_ERR_INVALID_ARG, "layer blob is NULL");
  if (reinterpret_cast<uintptr_t>(L->blob) % 256) return fail(NQ_ERR_INVALID_ARG, "layer blob is not 256-byte aligned");
  return NQ_OK;
}

nq_status hip_fail(hipError_t e, const char* what) {
  return fail(NQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Batch rows per launch pair of the decode path for a batch of B <= 16: the
// largest of min(B, 4) .. 1 whose plan fits (0: none).  Larger batches run as
// consecutive chunks of that many rows, each reading the weights again.
int dec_chunk(const nq_layer* L, int32_t B) {
  if (B < 1 || B > DEC_MAX_BATCH) return 0;
  for (int c = B < 4 ? B : 4; c >= 1; c--)
    if (nq::dec_plan(L->m, L->n, L->r, c, scale_bytes(L->scale_dtype)).ok) return c;
  return 0;
}

size_t plan_bytes(const nq_layer* L, int32_t B, int32_t path) {
  switch (path) {
    case NQ_PATH_GEMV: return nq::gemv_plan(L->m, L->n, L->r, B).bytes;
    case NQ_PATH_VALU: return nq::valu_plan(L->m, L->n, L->r).bytes;
    case NQ_PATH_GEMM: return nq::gemm_plan(L->m, L->n, L->r, B).bytes;
    case NQ_PATH_DECODE: {
      const int c = dec_chunk(L, B);
      if (!c) return 0;
      size_t need = nq::dec_plan(L->m, L->n, L->r, c, scale_bytes(L->scale_dtype)).bytes;
      if (B % c) {
        const size_t t = nq::dec_plan(L->m, L->n, L->r, B % c, scale_bytes(L->scale_dtype)).bytes;
        need = t > need ? t : need;
      }
      return need;
    }
  }
  return 0;
}

}  // namespace

extern "C" {

int32_t nq_abi_version(void) { return NQ_ABI_VERSION; }

size_t nq_layer_bytes(int32_t m, int32_t n, int32_t r, int32_t scale_dtype) {
  if (!dims_ok(m, n, r) || !scale_bytes(scale_dtype)) return 0;
  return nq::blob_layout(m, n, r, scale_bytes(scale_dtype)).total;
}

nq_status nq_pack_factors(const nq_layer* L, const int8_t* U, const int8_t* V, const void* s1, const void* g,
                          const void* s2, nq_stream_t stream) {
  nq_status st = check_layer(L);
  if (st) return st;
  if (!U || !V || !s1 || !g || !s2) return fail(NQ_ERR_INVALID_ARG, "U, V, s1, g and s2 must be non-NULL");
  const int sb = scale_bytes(L->scale_dtype);
  const nq::BlobLayout B = nq::blob_layout(L->m, L->n, L->r, sb);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* blob = static_cast<uint8_t*>(L->blob);

  nq::BlobHeader h;
  memset(&h, 0, sizeof(h));
  h.magic = nq::BLOB_MAGIC;
  h.version = nq::BLOB_VERSION;
  h.m = L->m;
  h.n = L->n;
  h.r = L->r;
  h.scale_dtype = L->scale_dtype;
  h.off_u = B.off_u;
  h.off_vt = B.off_vt;
  h.off_s1 = B.off_s1;
  h.off_g = B.off_g;
  h.off_s2 = B.off_s2;
  h.total = B.total;
  (void)hipGetLastError();
  hipError_t e = hipMemcpyAsync(blob, &h, sizeof(h), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "header copy");
  e = hipMemcpyAsync(blob + B.off_s1, s1, (size_t)L->m * sb, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(blob + B.off_g, g, (size_t)L->r * sb, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(blob + B.off_s2, s2, (size_t)L->n * sb, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "scale copy");
  int* bad = reinterpret_cast<int*>(blob + offsetof(nq::BlobHeader, bad_sign_count));
  // U: rows i (outputs), columns k (rank): U[i*r + k]
  e = nq::launch_pack(U, L->m, L->r, L->r, 1, reinterpret_cast<uint32_t*>(blob + B.off_u), bad, s);
  if (e != hipSuccess) return hip_fail(e, "pack U launch");
  // V^T: rows k (rank), columns j (inputs): V[j*r + k]
  e = nq::launch_pack(V, L->r, L->n, 1, L->r, reinterpret_cast<uint32_t*>(blob + B.off_vt), bad, s);
  if (e != hipSuccess) return hip_fail(e, "pack V launch");
  int bad_host = 0;
  e = hipMemcpyAsync(&bad_host, bad, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "pack synchronise");
  if (bad_host)
    return fail(NQ_ERR_NOT_PM1, "%d entries of U and V are not exactly +1 or -1", bad_host);
  return ok();
}

nq_status nq_transpose_layer(const nq_layer* src, const nq_layer* dst, nq_stream_t stream) {
  nq_status st = check_layer(src);
  if (st) return st;
  st = check_layer(dst);
  if (st) return st;
  if (dst->m != src->n || dst->n != src->m || dst->r != src->r)
    return fail(NQ_ERR_INVALID_ARG, "dst must be %d x %d of rank %d (the transpose of src), got %d x %d rank %d",
                src->n, src->m, src->r, dst->m, dst->n, dst->r);
  if (dst->scale_dtype != src->scale_dtype) return fail(NQ_ERR_INVALID_ARG, "dst and src differ in scale dtype");
  const int sb = scale_bytes(src->scale_dtype);
  const nq::BlobLayout S = nq::blob_layout(src->m, src->n, src->r, sb);
  const nq::BlobLayout D = nq::blob_layout(dst->m, dst->n, dst->r, sb);
  {
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src->blob), d0 = reinterpret_cast<uintptr_t>(dst->blob);
    if (s0 < d0 + D.total && d0 < s0 + S.total) return fail(NQ_ERR_INVALID_ARG, "src and dst blobs overlap");
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* in = static_cast<const uint8_t*>(src->blob);
  uint8_t* out = static_cast<uint8_t*>(dst->blob);
  nq::BlobHeader h;
  memset(&h, 0, sizeof(h));
  h.magic = nq::BLOB_MAGIC;
  h.version = nq::BLOB_VERSION;
  h.m = dst->m;
  h.n = dst->n;
  h.r = dst->r;
  h.scale_dtype = dst->scale_dtype;
  h.off_u = D.off_u;
  h.off_vt = D.off_vt;
  h.off_s1 = D.off_s1;
  h.off_g = D.off_g;
  h.off_s2 = D.off_s2;
  h.total = D.total;
  (void)hipGetLastError();
  hipError_t e = hipMemcpyAsync(out, &h, sizeof(h), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "header copy");
  // s1' = s2 (m' = n outputs), g' = g, s2' = s1 (n' = m inputs)
  e = hipMemcpyAsync(out + D.off_s1, in + S.off_s2, (size_t)src->n * sb, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(out + D.off_g, in + S.off_g, (size_t)src->r * sb, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(out + D.off_s2, in + S.off_s1, (size_t)src->m * sb, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "scale copy");
  // U' = V (n x r) is the transpose of the stored V^T (r x n); V'^T = U^T (r x m) that of U (m x r)
  e = nq::launch_transpose(reinterpret_cast<const uint32_t*>(in + S.off_vt), src->r, src->n,
                           reinterpret_cast<uint32_t*>(out + D.off_u), s);
  if (e == hipSuccess)
    e = nq::launch_transpose(reinterpret_cast<const uint32_t*>(in + S.off_u), src->m, src->r,
                             reinterpret_cast<uint32_t*>(out + D.off_vt), s);
  if (e != hipSuccess) return hip_fail(e, "transpose launch");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "transpose synchronise");
  return ok();
}

nq_status nq_unpack_factors(const nq_layer* L, int8_t* U, int8_t* V, nq_stream_t stream) {
  nq_status st = check_layer(L);
  if (st) return st;
  if (!U || !V) return fail(NQ_ERR_INVALID_ARG, "U and V must be non-NULL");
  const nq::BlobLayout B = nq::blob_layout(L->m, L->n, L->r, scale_bytes(L->scale_dtype));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* blob = static_cast<const uint8_t*>(L->blob);
  (void)hipGetLastError();
  hipError_t e = nq::launch_unpack(reinterpret_cast<const uint32_t*>(blob + B.off_u), L->m, L->r, L->r, 1, U, s);
  if (e == hipSuccess)
    e = nq::launch_unpack(reinterpret_cast<const uint32_t*>(blob + B.off_vt), L->r, L->n, 1, L->r, V, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "unpack");
  return ok();
}

size_t nq_workspace_bytes(const nq_layer* L, int32_t B) {
  if (check_layer(L) || B <= 0 || B > MAX_BATCH) return 0;
  size_t need = plan_bytes(L, B, NQ_PATH_GEMM);
  if (B <= 4) {
    size_t d = plan_bytes(L, B, NQ_PATH_DECODE);
    need = d > need ? d : need;
  }
  if (B <= 16) {
    size_t g = plan_bytes(L, B, NQ_PATH_GEMV);
    need = g > need ? g : need;
  }
  if (B == 1) {
    size_t v = plan_bytes(L, B, NQ_PATH_VALU);
    need = v > need ? v : need;
  }
  return need;
}

size_t nq_workspace_bytes_path(const nq_layer* L, int32_t B, int32_t path) {
  if (check_layer(L) || B <= 0 || B > MAX_BATCH) return 0;
  if (path == NQ_PATH_AUTO) return nq_workspace_bytes(L, B);
  if (path == NQ_PATH_GEMV && B > 16) return 0;
  if (path == NQ_PATH_VALU && B != 1) return 0;
  if (path == NQ_PATH_DECODE && !dec_chunk(L, B)) return 0;
  if (path < NQ_PATH_AUTO || path > NQ_PATH_DECODE) return 0;
  return plan_bytes(L, B, path);
}

static int32_t auto_path(const nq_layer* L, int32_t B) {
  if (B <= DEC_MAX_BATCH && dec_chunk(L, B)) return NQ_PATH_DECODE;
  return B <= 16 ? NQ_PATH_GEMV : NQ_PATH_GEMM;
}

// Scratch of nq_linear_fwd_noalloc: a static device array, so that call never
// allocates.  Host code only ever uses its per-device address from
// hipGetSymbolAddress (kept in g_scratch_ptr), never the array's name.
static __device__ __align__(256) uint8_t scratch[NQ_NOALLOC_SCRATCH_BYTES];
static constexpr int MAX_DEVICES = 64;
static void* g_scratch_ptr[MAX_DEVICES] = {};
static std::mutex g_scratch_mu;

static nq_status fwd_impl(const nq_layer* L, const void* x, int32_t x_dtype, void* y, int32_t y_dtype, int32_t B,
                          void* workspace, size_t workspace_bytes, nq_stream_t stream, int32_t path,
                          nq::LaunchMarks* marks) {
  nq_status st = check_layer(L);
  if (st) return st;
  if (B < 0 || B > MAX_BATCH) return fail(NQ_ERR_INVALID_ARG, "batch %d out of range 0..%d", B, MAX_BATCH);
  if (path < NQ_PATH_AUTO || path > NQ_PATH_DECODE) return fail(NQ_ERR_INVALID_ARG, "unknown path %d", path);
  const int xb = act_bytes(x_dtype), yb = act_bytes(y_dtype);
  if (!xb) return fail(NQ_ERR_INVALID_ARG, "x_dtype %d is not NQ_BF16 or NQ_F32", x_dtype);
  if (!yb) return fail(NQ_ERR_INVALID_ARG, "y_dtype %d is not NQ_BF16 or NQ_F32", y_dtype);
  if (B == 0) return ok();
  if (!x || !y) return fail(NQ_ERR_INVALID_ARG, "x and y must be non-NULL");
  if (reinterpret_cast<uintptr_t>(x) % xb || reinterpret_cast<uintptr_t>(y) % yb)
    return fail(NQ_ERR_INVALID_ARG, "x or y is not aligned to its element size");
  {
    uintptr_t x0 = reinterpret_cast<uintptr_t>(x), x1 = x0 + (uintptr_t)B * L->n * xb;
    uintptr_t y0 = reinterpret_cast<uintptr_t>(y), y1 = y0 + (uintptr_t)B * L->m * yb;
    if (x0 < y1 && y0 < x1) return fail(NQ_ERR_INVALID_ARG, "x and y overlap");
  }
  if (path == NQ_PATH_AUTO) path = auto_path(L, B);
  if (path == NQ_PATH_GEMV && B > 16) return fail(NQ_ERR_UNSUPPORTED, "gemv path takes B <= 16 (got %d)", B);
  if (path == NQ_PATH_VALU && B != 1) return fail(NQ_ERR_UNSUPPORTED, "valu path takes B == 1 (got %d)", B);
  if (path == NQ_PATH_DECODE && !dec_chunk(L, B))
    return fail(NQ_ERR_UNSUPPORTED, "decode path takes B <= %d and a rank whose image fits in LDS (B=%d r=%d)",
                DEC_MAX_BATCH, B, L->r);
  const size_t need = plan_bytes(L, B, path);
  if (workspace_bytes < need)
    return fail(NQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes, need);
  if (need && !workspace) return fail(NQ_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(NQ_ERR_INVALID_ARG, "workspace is not 256-byte aligned");

  nq::FwdArgs a;
  a.m = L->m;
  a.n = L->n;
  a.r = L->r;
  a.B = B;
  a.scale_dtype = L->scale_dtype;
  a.x_dtype = x_dtype;
  a.y_dtype = y_dtype;
  a.blob = static_cast<const uint8_t*>(L->blob);
  a.x = x;
  a.y = y;
  a.ws = static_cast<uint8_t*>(workspace);
  a.ws_bytes = workspace_bytes;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  a.marks = marks;
  if (marks && path != NQ_PATH_DECODE && path != NQ_PATH_GEMM)
    return fail(NQ_ERR_UNSUPPORTED, "timing marks are recorded by the decode and gemm paths only");
  (void)hipGetLastError();
  hipError_t e;
  switch (path) {
    case NQ_PATH_GEMV: e = nq::gemv_forward(a, nq::gemv_plan(a.m, a.n, a.r, B)); break;
    case NQ_PATH_VALU: e = nq::valu_forward(a, nq::valu_plan(a.m, a.n, a.r)); break;
    case NQ_PATH_DECODE: {  // chunks of dec_chunk rows, one after another on the stream
      const int c = dec_chunk(L, B);
      e = hipSuccess;
      for (int b0 = 0; b0 < B && e == hipSuccess; b0 += c) {
        nq::FwdArgs ac = a;
        ac.B = B - b0 < c ? B - b0 : c;
        ac.x = static_cast<const uint8_t*>(x) + (size_t)b0 * L->n * xb;
        ac.y = static_cast<uint8_t*>(y) + (size_t)b0 * L->m * yb;
        e = nq::dec_forward(ac, nq::dec_plan(a.m, a.n, a.r, ac.B, scale_bytes(a.scale_dtype)));
      }
      break;
    }
    default: e = nq::gemm_forward(a, nq::gemm_plan(a.m, a.n, a.r, B)); break;
  }
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return ok();
}

static bool spans_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// ------------------------------------------------------------------ rank-l envelope
// The env scale-vector pairs are first copied into the workspace, each row
// padded (s1 rows to 16 elements, s2 rows to 8) so that the kernels' whole-word
// reads never leave the buffer; the forward's own workspace follows.
struct EnvLayout {
  size_t s1_pitch, s2_pitch;  // bytes between rows
  size_t off_s1, off_s2, off_fwd, bytes;
};

static EnvLayout env_layout(const nq_layer* L, int32_t env, size_t fwd_bytes) {
  const int sb = scale_bytes(L->scale_dtype);
  EnvLayout e;
  e.s1_pitch = (size_t)(L->m + 15) / 16 * 16 * sb;
  e.s2_pitch = (size_t)(L->n + 7) / 8 * 8 * sb;
  e.off_s1 = 0;
  e.off_s2 = (e.off_s1 + env * e.s1_pitch + 255) / 256 * 256;
  e.off_fwd = (e.off_s2 + env * e.s2_pitch + 255) / 256 * 256;
  e.bytes = e.off_fwd + fwd_bytes;
  return e;
}

static nq::DecPlan env_plan(const nq_layer* L, int32_t env, int32_t B) {
  nq::DecPlan p = nq::dec_plan(L->m, L->n, L->r, B * env, scale_bytes(L->scale_dtype), true);
  if (!p.rows2) p.ok = false;  // the envelope sum lives in the row-split stage 2
  return p;
}

size_t nq_workspace_bytes_envelope(const nq_layer* L, int32_t env, int32_t B) {
  if (check_layer(L) || env < 1 || env > NQ_ENVELOPE_MAX || B < 1 || B * env > 4) return 0;
  const nq::DecPlan p = env_plan(L, env, B);
  return p.ok ? env_layout(L, env, p.bytes).bytes : 0;
}

nq_status nq_linear_fwd_envelope(const nq_layer* L, int32_t env, const void* s1_env, const void* s2_env,
                                 const void* x, int32_t x_dtype, void* y, int32_t y_dtype, int32_t B,
                                 void* workspace, size_t workspace_bytes, nq_stream_t stream) {
  nq_status st = check_layer(L);
  if (st) return st;
  if (env < 1 || env > NQ_ENVELOPE_MAX)
    return fail(NQ_ERR_INVALID_ARG, "envelope of %d terms (1..%d)", env, NQ_ENVELOPE_MAX);
  if (B < 0 || B > MAX_BATCH) return fail(NQ_ERR_INVALID_ARG, "batch %d out of range 0..%d", B, MAX_BATCH);
  const int xb = act_bytes(x_dtype), yb = act_bytes(y_dtype), sb = scale_bytes(L->scale_dtype);
  if (!xb) return fail(NQ_ERR_INVALID_ARG, "x_dtype %d is not NQ_BF16 or NQ_F32", x_dtype);
  if (!yb) return fail(NQ_ERR_INVALID_ARG, "y_dtype %d is not NQ_BF16 or NQ_F32", y_dtype);
  if (B == 0) return ok();
  if (!x || !y || !s1_env || !s2_env) return fail(NQ_ERR_INVALID_ARG, "x, y, s1_env and s2_env must be non-NULL");
  if (reinterpret_cast<uintptr_t>(x) % xb || reinterpret_cast<uintptr_t>(y) % yb ||
      reinterpret_cast<uintptr_t>(s1_env) % sb || reinterpret_cast<uintptr_t>(s2_env) % sb)
    return fail(NQ_ERR_INVALID_ARG, "x, y or an envelope scale array is not aligned to its element size");
  if (spans_overlap(x, (size_t)B * L->n * xb, y, (size_t)B * L->m * yb))
    return fail(NQ_ERR_INVALID_ARG, "x and y overlap");
  if (B * env > 4)
    return fail(NQ_ERR_UNSUPPORTED, "the envelope path takes B x terms <= 4 (got %d x %d)", B, env);
  const nq::DecPlan p = env_plan(L, env, B);
  if (!p.ok) return fail(NQ_ERR_UNSUPPORTED, "no envelope plan for m=%d n=%d r=%d", L->m, L->n, L->r);
  const EnvLayout e = env_layout(L, env, p.bytes);
  if (workspace_bytes < e.bytes)
    return fail(NQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes,
                e.bytes);
  if (!workspace) return fail(NQ_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(NQ_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipError_t he = hipMemcpy2DAsync(ws + e.off_s1, e.s1_pitch, s1_env, (size_t)L->m * sb, (size_t)L->m * sb, env,
                                   hipMemcpyDeviceToDevice, s);
  if (he == hipSuccess)
    he = hipMemcpy2DAsync(ws + e.off_s2, e.s2_pitch, s2_env, (size_t)L->n * sb, (size_t)L->n * sb, env,
                          hipMemcpyDeviceToDevice, s);
  if (he != hipSuccess) return hip_fail(he, "envelope scale copy");
  nq::FwdArgs a;
  a.m = L->m;
  a.n = L->n;
  a.r = L->r;
  a.B = B * env;
  a.scale_dtype = L->scale_dtype;
  a.x_dtype = x_dtype;
  a.y_dtype = y_dtype;
  a.blob = static_cast<const uint8_t*>(L->blob);
  a.x = x;
  a.y = y;
  a.ws = ws + e.off_fwd;
  a.ws_bytes = workspace_bytes - e.off_fwd;
  a.stream = s;
  a.env = env;
  a.s1_env = ws + e.off_s1;
  a.s2_env = ws + e.off_s2;
  a.s1_env_stride = (int)(e.s1_pitch / sb);
  a.s2_env_stride = (int)(e.s2_pitch / sb);
  he = nq::dec_forward(a, p);
  if (he != hipSuccess) return hip_fail(he, "envelope forward launch");
  return ok();
}

// ------------------------------------------------------------------ layer groups
static_assert(NQ_GROUP_MAX == nq::GROUP_MAX, "one group size for the header and the kernels");
static nq::GroupPlan group_plan_of(const nq_layer* const* layers, int32_t L, int32_t B) {
  int m[NQ_GROUP_MAX], r[NQ_GROUP_MAX];
  for (int l = 0; l < L; l++) {
    m[l] = layers[l]->m;
    r[l] = layers[l]->r;
  }
  return nq::group_plan(m, r, L, layers[0]->n, B, scale_bytes(layers[0]->scale_dtype));
}

static nq_status check_group(const nq_layer* const* layers, int32_t L) {
  if (!layers) return fail(NQ_ERR_INVALID_ARG, "layers is NULL");
  if (L < 1 || L > NQ_GROUP_MAX) return fail(NQ_ERR_INVALID_ARG, "group of %d layers (1..%d)", L, NQ_GROUP_MAX);
  for (int l = 0; l < L; l++) {
    nq_status st = check_layer(layers[l]);
    if (st) return st;
    if (layers[l]->n != layers[0]->n)
      return fail(NQ_ERR_INVALID_ARG, "layer %d has n=%d, layer 0 has n=%d: a group shares x", l, layers[l]->n,
                  layers[0]->n);
    if (layers[l]->scale_dtype != layers[0]->scale_dtype)
      return fail(NQ_ERR_INVALID_ARG, "layer %d has another scale dtype than layer 0", l);
  }
  return NQ_OK;
}

// Batch rows per pass of the fused group path for a batch of B rows: the
// largest of min(B, 4) .. 1 that has a group plan (0: none).  Larger batches
// run as consecutive passes of that many rows, each reading the weights again.
static int group_chunk(const nq_layer* const* layers, int32_t L, int32_t B) {
  for (int c = B < 4 ? B : 4; c >= 1; c--)
    if (group_plan_of(layers, L, c).ok) return c;
  return 0;
}

size_t nq_workspace_bytes_group(const nq_layer* const* layers, int32_t L, int32_t B) {
  if (check_group(layers, L) || B <= 0 || B > MAX_BATCH) return 0;
  const nq::GroupPlan p = group_plan_of(layers, L, B);
  if (p.ok) return p.bytes;
  const int c = group_chunk(layers, L, B);
  if (c) {  // passes of c rows (and one of B mod c)
    size_t need = group_plan_of(layers, L, c).bytes;
    if (B % c) {
      const nq::GroupPlan t = group_plan_of(layers, L, B % c);
      if (t.ok && t.bytes > need) need = t.bytes;
    }
    return need;
  }
  size_t need = 0;  // one layer after another
  for (int l = 0; l < L; l++) {
    const size_t b = plan_bytes(layers[l], B, auto_path(layers[l], B));
    need = b > need ? b : need;
  }
  return need;
}

static nq_status group_impl(const nq_layer* const* layers, int32_t L, const void* x, int32_t x_dtype,
                            void* const* ys, int32_t y_dtype, int32_t B, void* workspace, size_t workspace_bytes,
                            nq_stream_t stream, nq::LaunchMarks* marks) {
  nq_status st = check_group(layers, L);
  if (st) return st;
  if (B < 0 || B > MAX_BATCH) return fail(NQ_ERR_INVALID_ARG, "batch %d out of range 0..%d", B, MAX_BATCH);
  const int xb = act_bytes(x_dtype), yb = act_bytes(y_dtype);
  if (!xb) return fail(NQ_ERR_INVALID_ARG, "x_dtype %d is not NQ_BF16 or NQ_F32", x_dtype);
  if (!yb) return fail(NQ_ERR_INVALID_ARG, "y_dtype %d is not NQ_BF16 or NQ_F32", y_dtype);
  if (B == 0) return ok();
  if (!x || !ys) return fail(NQ_ERR_INVALID_ARG, "x and ys must be non-NULL");
  if (reinterpret_cast<uintptr_t>(x) % xb) return fail(NQ_ERR_INVALID_ARG, "x is not aligned to its element size");
  const size_t xn = (size_t)B * layers[0]->n * xb;
  for (int l = 0; l < L; l++) {
    if (!ys[l]) return fail(NQ_ERR_INVALID_ARG, "ys[%d] is NULL", l);
    if (reinterpret_cast<uintptr_t>(ys[l]) % yb)
      return fail(NQ_ERR_INVALID_ARG, "ys[%d] is not aligned to its element size", l);
    const size_t yn = (size_t)B * layers[l]->m * yb;
    if (spans_overlap(x, xn, ys[l], yn)) return fail(NQ_ERR_INVALID_ARG, "x and ys[%d] overlap", l);
    for (int k = 0; k < l; k++)
      if (spans_overlap(ys[k], (size_t)B * layers[k]->m * yb, ys[l], yn))
        return fail(NQ_ERR_INVALID_ARG, "ys[%d] and ys[%d] overlap", k, l);
  }
  const nq::GroupPlan p = group_plan_of(layers, L, B);
  const size_t need = nq_workspace_bytes_group(layers, L, B);
  if (workspace_bytes < need)
    return fail(NQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes, need);
  if (need && !workspace) return fail(NQ_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(NQ_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const int chunk = p.ok ? B : group_chunk(layers, L, B);
  if (!p.ok && chunk) {  // passes of `chunk` batch rows through the fused group path
    if (marks) return fail(NQ_ERR_UNSUPPORTED, "timing marks need a single pass of the fused group path (B <= 4)");
    for (int b0 = 0; b0 < B; b0 += chunk) {
      const int cb = B - b0 < chunk ? B - b0 : chunk;
      const nq::GroupPlan pc = group_plan_of(layers, L, cb);
      if (!pc.ok) return fail(NQ_ERR_INTERNAL, "no group plan for a pass of %d rows", cb);
      nq::GroupArgs a;
      a.L = L;
      a.n = layers[0]->n;
      a.B = cb;
      for (int l = 0; l < L; l++) {
        a.m[l] = layers[l]->m;
        a.r[l] = layers[l]->r;
        a.blob[l] = static_cast<const uint8_t*>(layers[l]->blob);
        a.y[l] = static_cast<uint8_t*>(ys[l]) + (size_t)b0 * layers[l]->m * yb;
      }
      a.scale_dtype = layers[0]->scale_dtype;
      a.x_dtype = x_dtype;
      a.y_dtype = y_dtype;
      a.x = static_cast<const uint8_t*>(x) + (size_t)b0 * layers[0]->n * xb;
      a.ws = static_cast<uint8_t*>(workspace);
      a.stream = reinterpret_cast<hipStream_t>(stream);
      a.marks = nullptr;
      (void)hipGetLastError();
      const hipError_t e = nq::group_forward(a, pc);
      if (e != hipSuccess) return hip_fail(e, "group forward launch");
    }
    return ok();
  }
  if (!p.ok) {
    if (marks) return fail(NQ_ERR_UNSUPPORTED, "timing marks need the fused group path (B <= 4)");
    for (int l = 0; l < L; l++) {  // one layer after another, each on its automatic path
      st = fwd_impl(layers[l], x, x_dtype, ys[l], y_dtype, B, workspace, workspace_bytes, stream, NQ_PATH_AUTO,
                    nullptr);
      if (st) return st;
    }
    return ok();
  }
  nq::GroupArgs a;
  a.L = L;
  a.n = layers[0]->n;
  a.B = B;
  for (int l = 0; l < L; l++) {
    a.m[l] = layers[l]->m;
    a.r[l] = layers[l]->r;
    a.blob[l] = static_cast<const uint8_t*>(layers[l]->blob);
    a.y[l] = ys[l];
  }
  a.scale_dtype = layers[0]->scale_dtype;
  a.x_dtype = x_dtype;
  a.y_dtype = y_dtype;
  a.x = x;
  a.ws = static_cast<uint8_t*>(workspace);
  a.stream = reinterpret_cast<hipStream_t>(stream);
  a.marks = marks;
  (void)hipGetLastError();
  const hipError_t e = nq::group_forward(a, p);
  if (e != hipSuccess) return hip_fail(e, "group forward launch");
  return ok();
}

nq_status nq_linear_fwd_group(const nq_layer* const* layers, int32_t L, const void* x, int32_t x_dtype,
                              void* const* ys, int32_t y_dtype, int32_t B, void* workspace, size_t workspace_bytes,
                              nq_stream_t stream) {
  return group_impl(layers, L, x, x_dtype, ys, y_dtype, B, workspace, workspace_bytes, stream, nullptr);
}

nq_status nq_linear_fwd_group_profiled(const nq_layer* const* layers, int32_t L, const void* x, int32_t x_dtype,
                                       void* const* ys, int32_t y_dtype, int32_t B, void* workspace,
                                       size_t workspace_bytes, nq_stream_t stream, void* const* events,
                                       int32_t n_events, int32_t* n_launches, int32_t* launch_dims) {
  if (!events || n_events < 1 || !n_launches) return fail(NQ_ERR_INVALID_ARG, "events and n_launches must be given");
  nq::LaunchMarks marks;
  marks.ev = reinterpret_cast<hipEvent_t*>(const_cast<void**>(events));
  marks.n = n_events;
  marks.dims = launch_dims;
  nq_status st = group_impl(layers, L, x, x_dtype, ys, y_dtype, B, workspace, workspace_bytes, stream, &marks);
  *n_launches = marks.k > 0 ? marks.k - 1 : 0;
  return st;
}

nq_status nq_linear_fwd_path(const nq_layer* L, const void* x, int32_t x_dtype, void* y, int32_t y_dtype, int32_t B,
                             void* workspace, size_t workspace_bytes, nq_stream_t stream, int32_t path) {
  return fwd_impl(L, x, x_dtype, y, y_dtype, B, workspace, workspace_bytes, stream, path, nullptr);
}

nq_status nq_linear_fwd_profiled(const nq_layer* L, const void* x, int32_t x_dtype, void* y, int32_t y_dtype,
                                 int32_t B, void* workspace, size_t workspace_bytes, nq_stream_t stream, int32_t path,
                                 void* const* events, int32_t n_events, int32_t* n_launches,
                                 int32_t* launch_dims) {
  if (!events || n_events < 1 || !n_launches) return fail(NQ_ERR_INVALID_ARG, "events and n_launches must be given");
  nq::LaunchMarks marks;
  marks.ev = reinterpret_cast<hipEvent_t*>(const_cast<void**>(events));
  marks.dims = launch_dims;
  marks.n = n_events;
  nq_status st = fwd_impl(L, x, x_dtype, y, y_dtype, B, workspace, workspace_bytes, stream, path, &marks);
  *n_launches = marks.k > 0 ? marks.k - 1 : 0;
  return st;
}

nq_status nq_linear_fwd_noalloc(const nq_layer* L, const void* x, int32_t x_dtype, void* y, int32_t y_dtype,
                                int32_t B, nq_stream_t stream) {
  nq_status st = check_layer(L);
  if (st) return st;
  if (B < 0 || B > MAX_BATCH) return fail(NQ_ERR_INVALID_ARG, "batch %d out of range 0..%d", B, MAX_BATCH);
  if (B == 0) return nq_linear_fwd_path(L, x, x_dtype, y, y_dtype, 0, nullptr, 0, stream, NQ_PATH_AUTO);
  const size_t need = plan_bytes(L, B, auto_path(L, B));
  if (need > (size_t)NQ_NOALLOC_SCRATCH_BYTES)
    return fail(NQ_ERR_WORKSPACE, "this call needs %zu bytes of workspace; the no-allocation scratch holds %zu",
                need, (size_t)NQ_NOALLOC_SCRATCH_BYTES);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(NQ_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {  // once per device, with that device current
      e = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        g_scratch_ptr[dev] = nullptr;
        return hip_fail(e, "hipGetSymbolAddress(scratch)");
      }
    }
    ptr = g_scratch_ptr[dev];
  }
  return nq_linear_fwd_path(L, x, x_dtype, y, y_dtype, B, ptr, (size_t)NQ_NOALLOC_SCRATCH_BYTES, stream,
                            NQ_PATH_AUTO);
}

nq_status nq_linear_fwd(const nq_layer* L, const void* x, int32_t x_dtype, void* y, int32_t y_dtype, int32_t B,
                        void* workspace, size_t workspace_bytes, nq_stream_t stream) {
  return nq_linear_fwd_path(L, x, x_dtype, y, y_dtype, B, workspace, workspace_bytes, stream, NQ_PATH_AUTO);
}

nq_status nq_read_probe(const void* buf, size_t bytes, uint32_t* sink, nq_stream_t stream, int32_t* grid) {
  if (!buf || !sink) return fail(NQ_ERR_INVALID_ARG, "buf and sink must be given");
  if (bytes == 0 || bytes % nq::PROBE_BATCH_BYTES)
    return fail(NQ_ERR_INVALID_ARG, "bytes (%zu) must be a positive multiple of %zu", bytes, nq::PROBE_BATCH_BYTES);
  if (reinterpret_cast<uintptr_t>(buf) % 16) return fail(NQ_ERR_INVALID_ARG, "buf is not 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(sink) % 4) return fail(NQ_ERR_INVALID_ARG, "sink is not 4-byte aligned");
  if (spans_overlap(buf, bytes, sink, 4)) return fail(NQ_ERR_INVALID_ARG, "sink lies inside buf");
  dim3 g;
  const hipError_t e = nq::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream), &g);
  if (e != hipSuccess) return hip_fail(e, "read probe launch");
  if (grid) {
    grid[0] = (int32_t)g.x;
    grid[1] = 64 * 4;
  }
  return NQ_OK;
}

size_t nq_admm_workspace_bytes(int32_t m, int32_t n, int32_t r) {
  if (!dims_ok(m, n, r) || r > 4096 || r > m || r > n || (long long)(m > n ? m : n) * r >= (1LL << 31)) return 0;
  return nq::admm_workspace_bytes(m, n, r);
}

nq_status nq_admm_factorize(const float* W, int32_t m, int32_t n, int32_t r, const float* A0, const float* B0,
                            float rho, int32_t iters, int32_t power_iters, int8_t* U, int8_t* V, float* s1,
                            float* g, float* s2, float* err, void* workspace, size_t workspace_bytes,
                            nq_stream_t stream) {
  if (!W || !A0 || !B0 || !U || !V || !s1 || !g || !s2 || !workspace)
    return fail(NQ_ERR_INVALID_ARG, "W, A0, B0, U, V, s1, g, s2 and workspace must be given");
  if (!dims_ok(m, n, r) || r > 4096 || r > m || r > n)
    return fail(NQ_ERR_INVALID_ARG, "dimensions out of range: m=%d n=%d r=%d (r <= min(m, n, 4096))", m, n, r);
  if ((long long)(m > n ? m : n) * r >= (1LL << 31))
    return fail(NQ_ERR_INVALID_ARG, "max(m, n) x r = %lld elements (below 2^31 required)", (long long)(m > n ? m : n) * r);
  if (!(rho > 0.0f) || !std::isfinite(rho)) return fail(NQ_ERR_INVALID_ARG, "rho must be positive and finite");
  if (iters < 0 || iters > 10000 || power_iters < 0 || power_iters > 1000)
    return fail(NQ_ERR_INVALID_ARG, "iters (%d) must be in 0..10000, power_iters (%d) in 0..1000", iters, power_iters);
  const void* fp[] = {W, A0, B0, s1, g, s2, err};
  for (const void* p : fp)
    if (p && reinterpret_cast<uintptr_t>(p) % 4) return fail(NQ_ERR_INVALID_ARG, "fp32 arrays must be 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(NQ_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  const size_t need = nq::admm_workspace_bytes(m, n, r);
  if (workspace_bytes < need) return fail(NQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  nq::AdmmArgs a{W, m, n, r, A0, B0, rho, iters, power_iters, U, V, s1, g, s2, err,
                 static_cast<uint8_t*>(workspace), static_cast<hipStream_t>(stream)};
  const hipError_t e = nq::admm_run(a);
  if (e != hipSuccess) return hip_fail(e, "initialiser launch");
  return ok();
}

nq_status nq_balance_scales(float* s1, float* g, float* s2, int32_t m, int32_t n, int32_t r, nq_stream_t stream) {
  if (!s1 || !g || !s2) return fail(NQ_ERR_INVALID_ARG, "s1, g and s2 must be given");
  if (!dims_ok(m, n, r)) return fail(NQ_ERR_INVALID_ARG, "dimensions out of range: m=%d n=%d r=%d", m, n, r);
  const hipError_t e = nq::launch_balance(s1, g, s2, m, n, r, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "balance launch");
  return ok();
}

double nq_bits_per_weight(int32_t m, int32_t n, int32_t r, int32_t scale_bits) {
  if (m < 1 || n < 1 || r < 0 || scale_bits < 0) return -1.0;
  return ((double)r * ((double)m + n) + (double)scale_bits * ((double)m + n + r)) / ((double)m * n);
}

int32_t nq_rank_for_bits(int32_t m, int32_t n, double bpw, int32_t scale_bits) {
  if (m < 1 || n < 1 || scale_bits < 0 || !(bpw >= 0.0) || std::isinf(bpw)) return -1;
  if (nq_bits_per_weight(m, n, 1, scale_bits) > bpw) return 0;
  double est = std::floor((bpw * (double)m * n - (double)scale_bits * ((double)m + n)) / ((double)m + n + scale_bits));
  if (est > 2147483000.0) est = 2147483000.0;
  int32_t r = est < 1.0 ? 1 : (int32_t)est;
  while (r > 1 && nq_bits_per_weight(m, n, r, scale_bits) > bpw) r--;
  while (r < 2147483000 && nq_bits_per_weight(m, n, r + 1, scale_bits) <= bpw) r++;
  return r;
}

const char* nq_status_string(int32_t s) {
  switch (s) {
    case NQ_OK: return "ok";
    case NQ_ERR_INVALID_ARG: return "invalid argument";
    case NQ_ERR_NOT_PM1: return "sign matrix entry is not +1 or -1";
    case NQ_ERR_WORKSPACE: return "workspace too small";
    case NQ_ERR_UNSUPPORTED: return "unsupported by the chosen path";
    case NQ_ERR_HIP: return "HIP runtime error";
    case NQ_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

const char* nq_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
