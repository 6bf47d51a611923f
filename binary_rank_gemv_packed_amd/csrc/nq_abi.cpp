// C ABI of libnq (declared in include/nq.h).  Every argument is validated on the
// host before any HIP call, so every error path is reachable without a GPU.
#include "nq.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
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

size_t plan_bytes(const nq_layer* L, int32_t B, int32_t path) {
  switch (path) {
    case NQ_PATH_GEMV: return nq::gemv_plan(L->m, L->n, L->r, B).bytes;
    case NQ_PATH_VALU: return nq::valu_plan(L->m, L->n, L->r).bytes;
    case NQ_PATH_GEMM: return nq::gemm_plan(L->m, L->n, L->r, B).bytes;
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

nq_status nq_linear_fwd_path(const nq_layer* L, const void* x, int32_t x_dtype, void* y, int32_t y_dtype, int32_t B,
                             void* workspace, size_t workspace_bytes, nq_stream_t stream, int32_t path) {
  nq_status st = check_layer(L);
  if (st) return st;
  if (B < 0 || B > MAX_BATCH) return fail(NQ_ERR_INVALID_ARG, "batch %d out of range 0..%d", B, MAX_BATCH);
  if (path < NQ_PATH_AUTO || path > NQ_PATH_VALU) return fail(NQ_ERR_INVALID_ARG, "unknown path %d", path);
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
  if (path == NQ_PATH_AUTO) path = B <= 16 ? NQ_PATH_GEMV : NQ_PATH_GEMM;
  if (path == NQ_PATH_GEMV && B > 16) return fail(NQ_ERR_UNSUPPORTED, "gemv path takes B <= 16 (got %d)", B);
  if (path == NQ_PATH_VALU && B != 1) return fail(NQ_ERR_UNSUPPORTED, "valu path takes B == 1 (got %d)", B);
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
  (void)hipGetLastError();
  hipError_t e;
  switch (path) {
    case NQ_PATH_GEMV: e = nq::gemv_forward(a, nq::gemv_plan(a.m, a.n, a.r, B)); break;
    case NQ_PATH_VALU: e = nq::valu_forward(a, nq::valu_plan(a.m, a.n, a.r)); break;
    default: e = nq::gemm_forward(a, nq::gemm_plan(a.m, a.n, a.r, B)); break;
  }
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return ok();
}

nq_status nq_linear_fwd(const nq_layer* L, const void* x, int32_t x_dtype, void* y, int32_t y_dtype, int32_t B,
                        void* workspace, size_t workspace_bytes, nq_stream_t stream) {
  return nq_linear_fwd_path(L, x, x_dtype, y, y_dtype, B, workspace, workspace_bytes, stream, NQ_PATH_AUTO);
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
