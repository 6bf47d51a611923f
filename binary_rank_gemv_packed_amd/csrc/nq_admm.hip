// Initialiser of the binary factorisation (ADMM with a sign projection) and
// magnitude balancing of the scale vectors.
//
// Reading of the hardwired.dev NanoQuant article, section "Trikrokovy
// pipeline", step 2 and the paragraph after it (an ADMM method whose
// iterations solve for the real-valued part by least squares in closed form
// and map onto the +-1 set by taking signs; then balancing of the scales,
// here by powers of two).  With an
// identity Hessian the problem is
//
//     minimise ||W - A B^T||_F^2,  A = diag(pA) U diag(qA),  B = diag(pB) V diag(qB)
//
// and one ADMM step is
//
//     A   <- (W B + rho (ZA - LA)) (B^T B + rho I)^-1
//     B   <- (W^T A + rho (ZB - LB)) (A^T A + rho I)^-1
//     ZA  <- proj(A + LA),  ZB <- proj(B + LB),  LA += A - ZA,  LB += B - ZB
//
// proj(Y) = diag(p) sign(Y) diag(q), (p, q) the leading singular pair of |Y|
// by K power steps from the constant vector.  The result is the stored form:
// U = sign(A + LA), V = sign(B + LB), s1 = pA, g = qA * qB, s2 = pB.
//
// Kernels: an fp32 MFMA GEMM (v_mfma_f32_16x16x4f32, 64 x 64 tiles, operand
// strides as arguments so W and W^T share it) for the four products and the
// two Gram matrices; the r x r inverse by block Gauss-Jordan (64 pivots a
// step: the pivot block inverted in LDS, then a rank-64 update of the whole
// matrix; symmetric positive definite, so no pivoting); the power steps as row and column
// products of |Y| with deterministic, fixed-order reductions.  Everything is
// fp32; every reduction order is fixed, so a run is reproducible bit for bit.
#include "nq_common.h"
#include "nq_internal.h"

namespace nq {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int GT = 64;   // GEMM block tile (rows and columns)
constexpr int GK = 16;   // GEMM K step
constexpr int PAD = 4;   // LDS row padding (floats)
constexpr int COL_CHUNKS = 64;  // row chunks of the column products of |Y|

// C[i][j] = sum_k A(i, k) B(k, j) + epilogue, A(i, k) = A[i * sai + k * sak],
// B(k, j) = B[k * sbk + j * sbj].  EPI 0: nothing; 1: + rho (Z - L)[i][j]
// (Z, L with row stride ldz); 2: + rho on the diagonal.
struct GemmF32 {
  const float* A;
  long long sai, sak;
  const float* B;
  long long sbk, sbj;
  float* C;
  long long ldc;
  int M, N, K;
  const float* Z;
  const float* L;
  long long ldz;
  float rho;
};

template <int EPI>
__global__ void __launch_bounds__(256) gemm_f32_kernel(GemmF32 g) {
  __shared__ float As[GK][GT + PAD];  // As[k][i]
  __shared__ float Bs[GK][GT + PAD];  // Bs[k][j]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const bool a_kfast = g.sak == 1, b_jfast = g.sbj == 1;
  v4f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < g.K; k0 += GK) {
#pragma unroll
    for (int c = 0; c < (GT * GK) / 256; c++) {
      const int e = tid + 256 * c;
      // A tile: 64 rows x 16 k, consecutive threads along the contiguous index
      const int ai = a_kfast ? e / GK : e % GT, ak = a_kfast ? e % GK : e / GT;
      const int gi = m0 + ai, gk = k0 + ak;
      As[ak][ai] = (gi < g.M && gk < g.K) ? g.A[(long long)gi * g.sai + (long long)gk * g.sak] : 0.0f;
      const int bj = b_jfast ? e % GT : e / GK, bk = b_jfast ? e / GT : e % GK;
      const int gj = n0 + bj, gk2 = k0 + bk;
      Bs[bk][bj] = (gj < g.N && gk2 < g.K) ? g.B[(long long)gk2 * g.sbk + (long long)gj * g.sbj] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GK; kk += 4) {
      const int kr = kk + (lane >> 4);
      float af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; i++) af[i] = As[kr][wm + 16 * i + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; j++) bf[j] = Bs[kr][wn + 16 * j + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // lane holds rows 4 * (lane >> 4) + v of each 16 x 16 tile, column lane & 15
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int row = m0 + wm + 16 * i + 4 * (lane >> 4) + v;
      if (row >= g.M) continue;
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int col = n0 + wn + 16 * j + (lane & 15);
        if (col >= g.N) continue;
        float c = acc[i][j][v];
        if (EPI == 1) c += g.rho * (g.Z[row * g.ldz + col] - g.L[row * g.ldz + col]);
        if (EPI == 2 && row == col) c += g.rho;
        g.C[row * g.ldc + col] = c;
      }
    }
}

// Block Gauss-Jordan inverse of a symmetric positive definite r x r matrix M,
// in place, one pivot block K = [k0, k0 + bk) (bk <= GJB) per step; every
// pivot block of an SPD matrix (and of its partial sweeps) is SPD, so no
// pivoting is needed.  With P = M[K][K], C = M[:][K] and
// R[t][j] = (P^-1 M[K][:])[t][j] for j outside K, (P^-1)[t][j - k0] inside,
// one step is
//     M[i][j] <- R[i - k0][j]                                   i in K
//     M[i][j] <- (j in K ? 0 : M[i][j]) - sum_t C[i][t] R[t][j]  i outside K
// (the exchange of the pivot block: after all blocks M holds its inverse).
constexpr int GJB = 64;

// P^-1 of the bk x bk pivot block by scalar Gauss-Jordan sweeps in LDS (one
// workgroup of 1024 threads: thread (i, c) holds row i = tid / 16, columns
// c + 16 u; two buffers so that a sweep reads only the previous one).
constexpr int GJL = GJB + 1;  // LDS row stride (column reads hit distinct banks)
__global__ void __launch_bounds__(1024) gj_block_inv_kernel(const float* __restrict__ M, int r, int k0, int bk,
                                                            float* __restrict__ Pinv) {
  __shared__ float buf[2][GJB * GJL];
  const int i = threadIdx.x >> 4, c0 = threadIdx.x & 15;
#pragma unroll
  for (int u = 0; u < GJB / 16; u++) {
    const int j = c0 + 16 * u;
    buf[0][i * GJL + j] = (i < bk && j < bk) ? M[(long long)(k0 + i) * r + k0 + j] : 0.0f;
  }
  __syncthreads();
  int cur = 0;
  for (int k = 0; k < bk; k++) {
    const float* in = buf[cur];
    float* out = buf[cur ^ 1];
    const float ip = 1.0f / in[k * GJL + k];
    const float fi = in[i * GJL + k];
#pragma unroll
    for (int u = 0; u < GJB / 16; u++) {
      const int j = c0 + 16 * u;
      const float rowk = (j == k ? 1.0f : in[k * GJL + j]) * ip;
      out[i * GJL + j] = i == k ? rowk : (j == k ? 0.0f : in[i * GJL + j]) - fi * rowk;
    }
    __syncthreads();
    cur ^= 1;
  }
#pragma unroll
  for (int u = 0; u < GJB / 16; u++) {
    const int j = c0 + 16 * u;
    if (i < bk && j < bk) Pinv[i * bk + j] = buf[cur][i * GJL + j];
  }
}

// R (bk x r) and C (r x GJB, first bk columns) of one step from the current M
// (thread per element R[t][j] and C[j][t], t = blockIdx.y).
__global__ void __launch_bounds__(256) gj_panel_kernel(const float* __restrict__ M, int r, int k0, int bk,
                                                       const float* __restrict__ Pinv, float* __restrict__ R,
                                                       float* __restrict__ C) {
  const int j = blockIdx.x * 256 + threadIdx.x, t = blockIdx.y;
  if (j >= r) return;
  float v;
  if (j >= k0 && j < k0 + bk) {
    v = Pinv[t * bk + (j - k0)];
  } else {
    v = 0.0f;
    for (int u = 0; u < bk; u++) v += Pinv[t * bk + u] * M[(long long)(k0 + u) * r + j];
  }
  R[(long long)t * r + j] = v;
  C[(long long)j * GJB + t] = M[(long long)j * r + k0 + t];
}

// The rank-bk update of one step, 64 x 64 tiles of M (4 x 4 per thread).
__global__ void __launch_bounds__(256) gj_update_kernel(float* __restrict__ M, int r, int k0, int bk,
                                                        const float* __restrict__ R, const float* __restrict__ C) {
  __shared__ float Cs[64][GJB + 1];  // Cs[row][t]
  __shared__ float Rs[GJB][64 + 1];  // Rs[t][col]
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64, tid = threadIdx.x;
  for (int e = tid; e < 64 * GJB; e += 256) {
    const int a = e / GJB, t = e % GJB;
    Cs[a][t] = (i0 + a < r && t < bk) ? C[(long long)(i0 + a) * GJB + t] : 0.0f;
    const int t2 = e / 64, b = e % 64;
    Rs[t2][b] = (j0 + b < r && t2 < bk) ? R[(long long)t2 * r + j0 + b] : 0.0f;
  }
  __syncthreads();
  const int ti = (tid / 16) * 4, tj = (tid % 16) * 4;
  float acc[4][4] = {};
  for (int t = 0; t < bk; t++) {
    float c[4], q[4];
#pragma unroll
    for (int a = 0; a < 4; a++) c[a] = Cs[ti + a][t];
#pragma unroll
    for (int b = 0; b < 4; b++) q[b] = Rs[t][tj + b];
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
      for (int b = 0; b < 4; b++) acc[a][b] += c[a] * q[b];
  }
#pragma unroll
  for (int a = 0; a < 4; a++) {
    const int i = i0 + ti + a;
    if (i >= r) continue;
    const bool iK = i >= k0 && i < k0 + bk;
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int j = j0 + tj + b;
      if (j >= r) continue;
      const bool jK = j >= k0 && j < k0 + bk;
      float* mp = M + (long long)i * r + j;
      *mp = iK ? R[(long long)(i - k0) * r + j] : (jK ? 0.0f : *mp) - acc[a][b];
    }
  }
}

// y = x + z elementwise (the projection input A + L).
__global__ void __launch_bounds__(256) add_kernel(const float* __restrict__ x, const float* __restrict__ z,
                                                  float* __restrict__ y, long long n) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e < n) y[e] = x[e] + z[e];
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// p[i] = sum_k |Y[i][k]| q[k]: one wave per row, lanes over k, fixed tree.
__global__ void __launch_bounds__(256) absmv_rows_kernel(const float* __restrict__ Y, int rows, int r,
                                                         const float* __restrict__ q, float* __restrict__ p) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;  // whole waves leave together
  const float* y = Y + (long long)row * r;
  float s = 0.0f;
  for (int k = lane; k < r; k += 64) s += fabsf(y[k]) * q[k];
  s = wave_sum(s);
  if (lane == 0) p[row] = s;
}

// part[c][k] = sum over row chunk c of |Y[i][k]| p[i] (thread per column).
__global__ void __launch_bounds__(256) absmv_cols_kernel(const float* __restrict__ Y, int rows, int r,
                                                         const float* __restrict__ p, float* __restrict__ part) {
  const int k = blockIdx.x * 256 + threadIdx.x, c = blockIdx.y;
  if (k >= r) return;
  const int per = (rows + COL_CHUNKS - 1) / COL_CHUNKS;
  const int i0 = c * per, i1 = min(rows, i0 + per);
  float s = 0.0f;
  for (int i = i0; i < i1; i++) s += fabsf(Y[(long long)i * r + k]) * p[i];
  part[(long long)c * r + k] = s;
}

__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.0f;
  for (int i = 0; i < nw; i++) t += red[i];
  return t;
}

// q[k] = sum_c part[c][k] (when part != null), then v /= ||v|| (if > 0) and
// *norm_out = ||v||.  One workgroup of 1024 threads.
__global__ void __launch_bounds__(1024) normalize_kernel(const float* __restrict__ part, float* __restrict__ v, int len,
                                                         float* __restrict__ norm_out) {
  __shared__ float red[16];
  float s = 0.0f;
  for (int k = threadIdx.x; k < len; k += 1024) {
    float x;
    if (part) {
      x = 0.0f;
      for (int c = 0; c < COL_CHUNKS; c++) x += part[(long long)c * len + k];
      v[k] = x;
    } else {
      x = v[k];
    }
    s += x * x;
  }
  // the column sums above are written and re-read by the same thread
  const float nrm = sqrtf(block_sum(s, red));
  const float inv = nrm > 0.0f ? 1.0f / nrm : 1.0f;
  for (int k = threadIdx.x; k < len; k += 1024) v[k] = nrm > 0.0f ? v[k] * inv : v[k];
  if (threadIdx.x == 0 && norm_out) *norm_out = nrm;
}

__global__ void __launch_bounds__(256) fill_kernel(float* __restrict__ v, long long n, float val) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e < n) v[e] = val;
}

// Z = diag(p) sign(Y) diag(q) * sigma (p, q unit vectors, sigma = ||.||),
// optional dual update L += X - Z, optional int8 signs.  Also writes the
// scaled vectors ps = p sqrt(sigma), qs = q sqrt(sigma) (block 0).
__global__ void __launch_bounds__(256) finish_proj_kernel(const float* __restrict__ Y, int rows, int r,
                                                          const float* __restrict__ p, const float* __restrict__ q,
                                                          const float* __restrict__ sigma, float* __restrict__ Z,
                                                          float* __restrict__ L, const float* __restrict__ X,
                                                          int8_t* __restrict__ S) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)rows * r) return;
  const int i = (int)(e / r), k = (int)(e % r);
  const float root = sqrtf(*sigma);
  const float y = Y[e];
  const float sg = y >= 0.0f ? 1.0f : -1.0f;
  const float z = sg * (p[i] * root) * (q[k] * root);
  Z[e] = z;
  if (L) L[e] += X[e] - z;
  if (S) S[e] = (int8_t)(y >= 0.0f ? 1 : -1);
}

// ps = p sqrt(sigma) (len values).
__global__ void __launch_bounds__(256) scale_vec_kernel(const float* __restrict__ p, const float* __restrict__ sigma,
                                                        float* __restrict__ out, int len, const float* __restrict__ mul) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= len) return;
  float v = p[e] * sqrtf(*sigma);
  if (mul) v *= mul[e];
  out[e] = v;
}

// sum over e of x[e] * y[e] -> *out, one workgroup (fixed order).
__global__ void __launch_bounds__(1024) dot_kernel(const float* __restrict__ x, const float* __restrict__ y,
                                                   long long n, float* __restrict__ out) {
  __shared__ float red[16];
  float s = 0.0f;
  for (long long e = threadIdx.x; e < n; e += 1024) s += x[e] * y[e];
  s = block_sum(s, red);
  if (threadIdx.x == 0) *out = s;
}

// err = (w2 - 2 cross + gram) / w2 from the three scalars.
__global__ void err_kernel(const float* __restrict__ sc, float* __restrict__ err) {
  const float w2 = sc[0], cross = sc[1], gram = sc[2];
  *err = (w2 - 2.0f * cross + gram) / w2;
}

// Power-of-two balancing of s1 (m), g (r), s2 (n) in place; one workgroup.
__device__ float balance_factor(float ss, int len) {
  const float rms = sqrtf(ss / (float)len);
  if (!(rms > 0.0f) || !(rms <= 3.4028235e38f)) return 1.0f;
  const int e = __builtin_amdgcn_frexp_expf(rms);  // rms = f 2^e, f in [0.5, 1)
  return __builtin_ldexpf(1.0f, 1 - e);
}

__global__ void __launch_bounds__(1024) balance_kernel(float* __restrict__ s1, float* __restrict__ g,
                                                       float* __restrict__ s2, int m, int n, int r) {
  __shared__ float red[16];
  float a = 0.0f, b = 0.0f;
  for (int i = threadIdx.x; i < m; i += 1024) a += s1[i] * s1[i];
  for (int i = threadIdx.x; i < n; i += 1024) b += s2[i] * s2[i];
  a = block_sum(a, red);
  b = block_sum(b, red);
  const float c = balance_factor(a, m), d = balance_factor(b, n);
  __syncthreads();
  for (int i = threadIdx.x; i < m; i += 1024) s1[i] *= c;
  for (int i = threadIdx.x; i < n; i += 1024) s2[i] *= d;
  const float gd = 1.0f / (c * d);  // a power of two: exact
  for (int i = threadIdx.x; i < r; i += 1024) g[i] *= gd;
}

inline unsigned blocks(long long n, int t) { return (unsigned)((n + t - 1) / t); }

struct AdmmWs {
  float *A, *B, *ZA, *ZB, *LA, *LB, *T, *G, *Gi;
  float *pA, *qA, *pB, *qB, *pv, *qv, *part, *sig, *sc;
  float *Pinv, *R, *C;
};

AdmmWs ws_layout(uint8_t* base, int m, int n, int r, size_t* total) {
  size_t o = 0;
  auto take = [&](size_t floats) {
    size_t at = o;
    o = align_up(o + floats * 4, 256);
    return reinterpret_cast<float*>(base + at);
  };
  const size_t mr = (size_t)m * r, nr = (size_t)n * r, rr = (size_t)r * r;
  const int mx = m > n ? m : n;
  AdmmWs w;
  w.A = take(mr);
  w.B = take(nr);
  w.ZA = take(mr);
  w.ZB = take(nr);
  w.LA = take(mr);
  w.LB = take(nr);
  w.T = take((size_t)mx * r);
  w.G = take(rr);
  w.Gi = take(rr);
  w.pA = take(m);
  w.qA = take(r);
  w.pB = take(n);
  w.qB = take(r);
  w.pv = take(mx);
  w.qv = take(r);
  w.part = take((size_t)COL_CHUNKS * r);
  w.sig = take(4);
  w.sc = take(4);
  w.Pinv = take((size_t)GJB * GJB);
  w.R = take((size_t)GJB * r);
  w.C = take((size_t)GJB * r);
  *total = o;
  return w;
}

void gemm(hipStream_t st, int epi, const float* A, long long sai, long long sak, const float* B, long long sbk,
          long long sbj, float* C, long long ldc, int M, int N, int K, const float* Z = nullptr,
          const float* L = nullptr, long long ldz = 0, float rho = 0.0f) {
  GemmF32 g{A, sai, sak, B, sbk, sbj, C, ldc, M, N, K, Z, L, ldz, rho};
  dim3 grid(blocks(N, GT), blocks(M, GT));
  if (epi == 1) hipLaunchKernelGGL(gemm_f32_kernel<1>, grid, dim3(256), 0, st, g);
  else if (epi == 2) hipLaunchKernelGGL(gemm_f32_kernel<2>, grid, dim3(256), 0, st, g);
  else hipLaunchKernelGGL(gemm_f32_kernel<0>, grid, dim3(256), 0, st, g);
}

// G (r x r, SPD) -> its inverse, in place (block Gauss-Jordan, GJB pivots a step).
void spd_inverse(hipStream_t st, const AdmmWs& w, float* G, int r) {
  for (int k0 = 0; k0 < r; k0 += GJB) {
    const int bk = r - k0 < GJB ? r - k0 : GJB;
    hipLaunchKernelGGL(gj_block_inv_kernel, dim3(1), dim3(1024), 0, st, G, r, k0, bk, w.Pinv);
    hipLaunchKernelGGL(gj_panel_kernel, dim3(blocks(r, 256), bk), dim3(256), 0, st, G, r, k0, bk, w.Pinv, w.R, w.C);
    hipLaunchKernelGGL(gj_update_kernel, dim3(blocks(r, 64), blocks(r, 64)), dim3(256), 0, st, G, r, k0, bk, w.R,
                       w.C);
  }
}

// proj(Y) of a rows x r matrix: Z, optional dual update with X, optional
// signs; the scaled singular vectors go to ps (rows) and qs (r).
void project(hipStream_t st, const AdmmWs& w, const float* Y, int rows, int r, int K, float* Z, float* L,
             const float* X, int8_t* S, float* ps, float* qs) {
  hipLaunchKernelGGL(fill_kernel, dim3(blocks(r, 256)), dim3(256), 0, st, w.qv, (long long)r, 1.0f / sqrtf((float)r));
  hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(256), 0, st, w.sig, 1LL, 0.0f);
  for (int it = 0; it < K; it++) {
    hipLaunchKernelGGL(absmv_rows_kernel, dim3(blocks(rows, 4)), dim3(256), 0, st, Y, rows, r, w.qv, w.pv);
    hipLaunchKernelGGL(normalize_kernel, dim3(1), dim3(1024), 0, st, nullptr, w.pv, rows, nullptr);
    hipLaunchKernelGGL(absmv_cols_kernel, dim3(blocks(r, 256), COL_CHUNKS), dim3(256), 0, st, Y, rows, r, w.pv,
                       w.part);
    hipLaunchKernelGGL(normalize_kernel, dim3(1), dim3(1024), 0, st, w.part, w.qv, r, w.sig);
  }
  if (K == 0) hipLaunchKernelGGL(fill_kernel, dim3(blocks(rows, 256)), dim3(256), 0, st, w.pv, (long long)rows, 0.0f);
  hipLaunchKernelGGL(finish_proj_kernel, dim3(blocks((long long)rows * r, 256)), dim3(256), 0, st, Y, rows, r, w.pv,
                     w.qv, w.sig, Z, L, X, S);
  hipLaunchKernelGGL(scale_vec_kernel, dim3(blocks(rows, 256)), dim3(256), 0, st, w.pv, w.sig, ps, rows, nullptr);
  hipLaunchKernelGGL(scale_vec_kernel, dim3(blocks(r, 256)), dim3(256), 0, st, w.qv, w.sig, qs, r, nullptr);
}

// err = ||W - ZA ZB^T||^2 / ||W||^2 via W ZB, the Gram matrices and two dots.
void rel_err(hipStream_t st, const AdmmWs& w, const float* W, int m, int n, int r, float* err) {
  hipLaunchKernelGGL(dot_kernel, dim3(1), dim3(1024), 0, st, W, W, (long long)m * n, w.sc + 0);
  gemm(st, 0, W, n, 1, w.ZB, r, 1, w.T, r, m, r, n);                       // W ZB
  hipLaunchKernelGGL(dot_kernel, dim3(1), dim3(1024), 0, st, w.ZA, w.T, (long long)m * r, w.sc + 1);
  gemm(st, 0, w.ZA, 1, r, w.ZA, r, 1, w.G, r, r, r, m);                    // ZA^T ZA
  gemm(st, 0, w.ZB, 1, r, w.ZB, r, 1, w.Gi, r, r, r, n);                   // ZB^T ZB
  hipLaunchKernelGGL(dot_kernel, dim3(1), dim3(1024), 0, st, w.G, w.Gi, (long long)r * r, w.sc + 2);
  hipLaunchKernelGGL(err_kernel, dim3(1), dim3(1), 0, st, w.sc, err);
}

}  // namespace

size_t admm_workspace_bytes(int m, int n, int r) {
  size_t total = 0;
  ws_layout(nullptr, m, n, r, &total);
  return total;
}

hipError_t admm_run(const AdmmArgs& a) {
  size_t total = 0;
  const AdmmWs w = ws_layout(a.ws, a.m, a.n, a.r, &total);
  const int m = a.m, n = a.n, r = a.r;
  hipStream_t st = a.stream;
  const long long mr = (long long)m * r, nr = (long long)n * r;
  hipMemcpyAsync(w.A, a.A0, mr * 4, hipMemcpyDeviceToDevice, st);
  hipMemcpyAsync(w.B, a.B0, nr * 4, hipMemcpyDeviceToDevice, st);
  hipLaunchKernelGGL(fill_kernel, dim3(blocks(mr, 256)), dim3(256), 0, st, w.LA, mr, 0.0f);
  hipLaunchKernelGGL(fill_kernel, dim3(blocks(nr, 256)), dim3(256), 0, st, w.LB, nr, 0.0f);
  const bool last0 = a.iters == 0;
  project(st, w, w.A, m, r, a.power_iters, w.ZA, nullptr, nullptr, last0 ? a.U : nullptr, w.pA, w.qA);
  project(st, w, w.B, n, r, a.power_iters, w.ZB, nullptr, nullptr, last0 ? a.V : nullptr, w.pB, w.qB);
  if (a.err) rel_err(st, w, a.W, m, n, r, a.err);
  for (int t = 0; t < a.iters; t++) {
    const bool last = t == a.iters - 1;
    const float* Ginv = w.G;
    // A <- (W B + rho (ZA - LA)) (B^T B + rho I)^-1
    gemm(st, 2, w.B, 1, r, w.B, r, 1, w.G, r, r, r, n, nullptr, nullptr, 0, a.rho);
    spd_inverse(st, w, w.G, r);
    gemm(st, 1, a.W, n, 1, w.B, r, 1, w.T, r, m, r, n, w.ZA, w.LA, r, a.rho);
    gemm(st, 0, w.T, r, 1, Ginv, r, 1, w.A, r, m, r, r);
    // B <- (W^T A + rho (ZB - LB)) (A^T A + rho I)^-1
    gemm(st, 2, w.A, 1, r, w.A, r, 1, w.G, r, r, r, m, nullptr, nullptr, 0, a.rho);
    spd_inverse(st, w, w.G, r);
    gemm(st, 1, a.W, 1, n, w.A, r, 1, w.T, r, n, r, m, w.ZB, w.LB, r, a.rho);
    gemm(st, 0, w.T, r, 1, Ginv, r, 1, w.B, r, n, r, r);
    // ZA <- proj(A + LA), LA += A - ZA; the same for B
    hipLaunchKernelGGL(add_kernel, dim3(blocks(mr, 256)), dim3(256), 0, st, w.A, w.LA, w.T, mr);
    project(st, w, w.T, m, r, a.power_iters, w.ZA, w.LA, w.A, last ? a.U : nullptr, w.pA, w.qA);
    hipLaunchKernelGGL(add_kernel, dim3(blocks(nr, 256)), dim3(256), 0, st, w.B, w.LB, w.T, nr);
    project(st, w, w.T, n, r, a.power_iters, w.ZB, w.LB, w.B, last ? a.V : nullptr, w.pB, w.qB);
    if (a.err) rel_err(st, w, a.W, m, n, r, a.err + t + 1);
  }
  // s1 = pA, g = qA * qB, s2 = pB (the scaled vectors of the last projections)
  hipMemcpyAsync(a.s1, w.pA, (size_t)m * 4, hipMemcpyDeviceToDevice, st);
  hipMemcpyAsync(a.s2, w.pB, (size_t)n * 4, hipMemcpyDeviceToDevice, st);
  hipLaunchKernelGGL(fill_kernel, dim3(1), dim3(256), 0, st, w.sc + 3, 1LL, 1.0f);
  hipLaunchKernelGGL(scale_vec_kernel, dim3(blocks(r, 256)), dim3(256), 0, st, w.qA, w.sc + 3, a.g, r, w.qB);
  return hipGetLastError();
}

hipError_t launch_balance(float* s1, float* g, float* s2, int m, int n, int r, hipStream_t st) {
  hipLaunchKernelGGL(balance_kernel, dim3(1), dim3(1024), 0, st, s1, g, s2, m, n, r);
  return hipGetLastError();
}

}  // namespace nq
