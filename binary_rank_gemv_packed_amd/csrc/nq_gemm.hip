// Large-batch forward ("gemm" path, prefill): both sign-matrix products as
// dense fp16 MFMA GEMMs.  The activation operand is staged through LDS; the
// sign operand stays packed (one bit per weight) in LDS and each wave expands
// its own B fragments to exact fp16 +-1 in registers.
//
//   prep  : X' = s2 * x per row, scaled by a per-row power of two 2^-e and
//           rounded to fp16 (columns padded to whole 128-column tiles with 0)
//   gemm  : T = X' V             (fp32, rows rescaled by 2^e)
//   mid   : T' = g * T per row, scaled by a per-row power of two, fp16
//   gemm  : y = s1 * (T' U^T)    (rows rescaled, stored as fp32 or bf16)
//
// The sign operand is exact in fp16.  The activation operand is rounded to
// fp16 (11 significant bits, relative error <= 2^-11 per value) after a
// power-of-two row scale that puts the row maximum in [2^13, 2^14), so no value
// overflows and the scale is undone exactly in the fp32 epilogue.  At B = 2048
// the work is a dense contraction (2 B r (m + n) flops, ~2.8 TFLOP per 70B
// block), so it runs on the matrix cores rather than as B separate GEMVs.
#include "nq_common.h"
#include "nq_internal.h"

namespace nq {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BKG = 64;  // block tile and K step (two 32-column sign groups)
constexpr int KG = BKG / 32;                 // sign words per W row per K step
constexpr int LDA_S = BKG + 8;               // LDS row stride of A in halves (pad against bank conflicts)
constexpr int TARGET_EXP = 13;               // row maximum lands in [2^13, 2^14)

__device__ inline int frexp_exp(float a) { return __builtin_amdgcn_frexp_expf(a); }

template <typename T> __device__ inline float ldf(const T* p, size_t i);
template <> __device__ inline float ldf<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ inline float ldf<_Float16>(const _Float16* p, size_t i) { return (float)p[i]; }
template <> __device__ inline float ldf<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

__device__ inline float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); i++) m = fmaxf(m, red[i]);
  __syncthreads();
  return m;
}

// Exponent e with max * 2^-e in [2^TARGET_EXP, 2^(TARGET_EXP+1)); 0 for a
// zero or non-finite row (non-finite values then stay non-finite in fp16).
__device__ inline int row_exp(float mx) {
  if (!(mx > 0.0f) || !(mx <= 3.4028235e38f)) return 0;
  return (frexp_exp(mx) - 1) - TARGET_EXP;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// V consecutive values p[k .. k+V-1] as fp32 (V = 4: one vector load; the
// caller guarantees the alignment)
template <int V, typename T> __device__ inline f32x4 ldv(const T* p, size_t k);
template <> __device__ inline f32x4 ldv<1, float>(const float* p, size_t k) { return f32x4{p[k], 0.f, 0.f, 0.f}; }
template <> __device__ inline f32x4 ldv<1, _Float16>(const _Float16* p, size_t k) {
  return f32x4{(float)p[k], 0.f, 0.f, 0.f};
}
template <> __device__ inline f32x4 ldv<1, uint16_t>(const uint16_t* p, size_t k) {
  return f32x4{ldf(p, k), 0.f, 0.f, 0.f};
}
template <> __device__ inline f32x4 ldv<4, float>(const float* p, size_t k) {
  return *reinterpret_cast<const f32x4*>(p + k);
}
template <> __device__ inline f32x4 ldv<4, _Float16>(const _Float16* p, size_t k) {
  return __builtin_convertvector(*reinterpret_cast<const f16x4*>(p + k), f32x4);
}
template <> __device__ inline f32x4 ldv<4, uint16_t>(const uint16_t* p, size_t k) {
  const u16x4 b = *reinterpret_cast<const u16x4*>(p + k);
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; i++) r[i] = __uint_as_float((uint32_t)b[i] << 16);
  return r;
}

// One workgroup (256 threads) per row: out[row][k] = fp16(scale_in[k] * in[row][k] * 2^-e)
// for k < K, 0 for K <= k < Kpad; rexp[row] = e.  in[row][k] is the sum of
// nsplit partial copies split_stride elements apart (the K splits of the GEMM
// that wrote them), added in copy order.  Each thread takes V consecutive
// columns at a time (V = 4 needs K, ld_in and split_stride multiples of 4 and
// in, scale aligned to 4 elements).
template <typename IT, typename ST, int V>
__global__ void __launch_bounds__(256) row_to_f16_kernel(const IT* __restrict__ in, size_t ld_in, int nsplit,
                                                         size_t split_stride, const ST* __restrict__ scale, int K,
                                                         int Kpad, _Float16* __restrict__ out,
                                                         int* __restrict__ rexp) {
  __shared__ float red[4];
  const int row = blockIdx.x;
  const IT* src = in + (size_t)row * ld_in;
  auto value = [&](int k) {
    f32x4 v = ldv<V>(src, k);
    for (int s = 1; s < nsplit; s++) v += ldv<V>(src + s * split_stride, k);
    return v * ldv<V>(scale, k);
  };
  float mx = 0.0f;
  for (int k = V * threadIdx.x; k < K; k += 256 * V) {
    const f32x4 v = value(k);
#pragma unroll
    for (int i = 0; i < V; i++) mx = fmaxf(mx, fabsf(v[i]));
  }
  mx = block_max(mx, red);
  const int e = row_exp(mx);
  const float f = __builtin_ldexpf(1.0f, -e);
  _Float16* dst = out + (size_t)row * Kpad;
  for (int k = V * threadIdx.x; k < Kpad; k += 256 * V) {
    const f32x4 v = k < K ? value(k) * f : f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (V == 4) {
      *reinterpret_cast<f16x4*>(dst + k) = __builtin_convertvector(v, f16x4);
    } else {
      dst[k] = (_Float16)v[0];
    }
  }
  if (threadIdx.x == 0) rexp[row] = e;
}

// Launches row_to_f16_kernel with V = 4 where the sizes and pointers allow it.
template <typename IT, typename ST>
void launch_row_to_f16(hipStream_t st, int rows, const IT* in, size_t ld_in, int nsplit, size_t split_stride,
                       const ST* scale, int K, int Kpad, _Float16* out, int* rexp) {
  const bool v4 = K % 4 == 0 && ld_in % 4 == 0 && split_stride % 4 == 0 &&
                  reinterpret_cast<uintptr_t>(in) % (4 * sizeof(IT)) == 0 &&
                  reinterpret_cast<uintptr_t>(scale) % (4 * sizeof(ST)) == 0;
  if (v4)
    hipLaunchKernelGGL((row_to_f16_kernel<IT, ST, 4>), dim3(rows), dim3(256), 0, st, in, ld_in, nsplit, split_stride,
                       scale, K, Kpad, out, rexp);
  else
    hipLaunchKernelGGL((row_to_f16_kernel<IT, ST, 1>), dim3(rows), dim3(256), 0, st, in, ld_in, nsplit, split_stride,
                       scale, K, Kpad, out, rexp);
}

// C = 2^e_row * (A W^T): A [M x Kpad] fp16 row-major (lda = Kpad), W the packed
// sign matrix with N rows and KT column tiles (Kpad = 128 KT).  EPI 0: fp32 out
// (ldc); EPI 1: out = colscale[n] * C as fp32 (ydt 0) or bf16 (ydt 2).  With
// S > 1 (EPI 0 only) the K steps are cut into S contiguous ranges, one
// workgroup per (tile, range), and range s writes its partial C at
// C + s * split_stride; the consumer adds the S partials.
struct GemmArgs {
  const _Float16* A;
  const int* rexp;
  const uint32_t* W;
  int M, N, KT;
  void* C;
  size_t ldc;
  const void* colscale;
  int ydt;
  int MB, NB;  // block counts
  int S;       // K splits
  size_t split_stride;
};

// One plane of a sign word as the 8 fp16 +-1 values of an MFMA B fragment.
// The word covers row n, columns 32g .. 32g+31 of a tile, bit 4p + j for
// column 8j + p (bit set = +1), and half p of the result is column 8j + p.
// ev = ~word & (0x01010101 << j) keeps the "-1" bits of the even halves (half
// 2q at bit j of byte q), od = (~word & (0x10101010 << j)) >> 4 those of the
// odd halves (half 2q + 1 at bit j of byte q).  One byte permute puts byte q
// of each at bits 8 + j and 24 + j with nothing else set, and one shift-or by
// sh = 7 - j moves them to the fp16 sign bits 15 and 31 and adds the
// magnitude 1.0: two integer operations per pair of values, on the lane that
// consumes them.
__device__ __forceinline__ h8 sign_plane(uint32_t ev, uint32_t od, int sh) {
  u32x4 d;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    // result byte 1 = ev byte q, byte 3 = od byte q, bytes 0 and 2 = 0
    const uint32_t sel = 0x0Cu | ((uint32_t)q << 8) | (0x0Cu << 16) | ((uint32_t)(4 + q) << 24);
    d[q] = (__builtin_amdgcn_perm(od, ev, sel) << sh) | 0x3C003C00u;
  }
  return __builtin_bit_cast(h8, d);
}

template <int EPI, typename SC>
__global__ void __launch_bounds__(256) gemm_kernel(GemmArgs a) {
  __shared__ __align__(16) _Float16 As[2][BM * LDA_S];
  __shared__ __align__(16) uint32_t Ws[2][BN * KG];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // XCD-aware tile order: the 8 XCDs take contiguous runs of tiles, M-block
  // major, so the workgroups one XCD runs together share an activation block
  const int T = a.MB * a.NB, TS = T * a.S;
  const int per = (TS + 7) / 8;
  const int id = blockIdx.x;
  const int ts = (id % 8) * per + id / 8;
  if (ts >= TS) return;
  const int t = ts % T, split = ts / T;
  const int mb = t / a.NB, nb = t % a.NB;
  const int m0 = mb * BM, n0 = nb * BN;
  const int Kpad = a.KT * 128;
  const int nk_all = Kpad / BKG, nks = (nk_all + a.S - 1) / a.S;
  const int kbeg = split * nks;
  const int nk = min(nk_all - kbeg, nks);  // K steps of this range (<= 0: an empty range, writes zeros)

  // global -> register staging.  A: 128 rows x 64 halves as 1024 16-byte
  // chunks; chunk 256 i + tid is row 32 i + tid / 8, columns 8 (tid % 8) .. +7,
  // so one load instruction covers 8 whole 128-byte row segments (rows past M
  // re-read row M - 1; their results are never stored).  W: the packed word of
  // block row tid / 2, sign group tid % 2 of the step (row tiles past the last
  // re-read it).  The signs stay packed in LDS; each wave expands its own B
  // fragments in registers.
  const int a_row = tid >> 3, a_col = (tid & 7) * 8;
  const _Float16* a_src0 = a.A + (size_t)min(m0 + a_row, a.M - 1) * Kpad + a_col;
  const _Float16* a_src1 = a.A + (size_t)min(m0 + a_row + 32, a.M - 1) * Kpad + a_col;
  const _Float16* a_src2 = a.A + (size_t)min(m0 + a_row + 64, a.M - 1) * Kpad + a_col;
  const _Float16* a_src3 = a.A + (size_t)min(m0 + a_row + 96, a.M - 1) * Kpad + a_col;
  const int w_row = tid >> 1, w_g = tid & 1, w_l = w_row & 15;
  const int w_rtg = min((n0 >> 4) + (w_row >> 4), (a.N + 15) / 16 - 1);
  const uint32_t* w_tile = a.W + (size_t)w_rtg * a.KT * 64;

  uint4 ra0, ra1, ra2, ra3;
  uint32_t rw;
#define NQ_GLOAD(ks)                                                          \
  do {                                                                        \
    const int k0_ = (ks) * BKG;                                               \
    ra0 = *reinterpret_cast<const uint4*>(a_src0 + k0_);                      \
    ra1 = *reinterpret_cast<const uint4*>(a_src1 + k0_);                      \
    ra2 = *reinterpret_cast<const uint4*>(a_src2 + k0_);                      \
    ra3 = *reinterpret_cast<const uint4*>(a_src3 + k0_);                      \
    const int kt_ = k0_ >> 7, g_ = ((k0_ >> 5) & 3) + w_g;                    \
    const int q_ = kt_ >> 2;                                                  \
    const int f_ = min(4, a.KT - 4 * q_);                                     \
    rw = w_tile[(size_t)q_ * 256 + (w_l + 16 * g_) * f_ + (kt_ & 3)];         \
  } while (0)
#define NQ_LSTORE(buf)                                                                     \
  do {                                                                                     \
    *reinterpret_cast<uint4*>(&As[(buf)][(a_row + 0) * LDA_S + a_col]) = ra0;              \
    *reinterpret_cast<uint4*>(&As[(buf)][(a_row + 32) * LDA_S + a_col]) = ra1;             \
    *reinterpret_cast<uint4*>(&As[(buf)][(a_row + 64) * LDA_S + a_col]) = ra2;             \
    *reinterpret_cast<uint4*>(&As[(buf)][(a_row + 96) * LDA_S + a_col]) = ra3;             \
    Ws[(buf)][w_row * KG + w_g] = rw;                                                      \
  } while (0)

  // wave tile 64 x 64 = 4 x 4 MFMA tiles of 16 x 16
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    NQ_GLOAD(kbeg);
    NQ_LSTORE(0);
  }
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;  // fragment row/column and K offset
  const int sh = 7 - (lane >> 4);                  // plane j = lane / 16 of each sign word
  const uint32_t emask = 0x01010101u << (lane >> 4), omask = emask << 4;
  for (int ks = 0; ks < nk; ks++) {
    const int buf = ks & 1;
    if (ks + 1 < nk) NQ_GLOAD(kbeg + ks + 1);
    uint2 wv[4];
#pragma unroll
    for (int j = 0; j < 4; j++) wv[j] = *reinterpret_cast<const uint2*>(&Ws[buf][(wn + 16 * j + fr) * KG]);
#pragma unroll
    for (int s = 0; s < KG; s++) {
      h8 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        af[i] = *reinterpret_cast<const h8*>(&As[buf][(wm + 16 * i + fr) * LDA_S + 32 * s + fk]);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t nw = ~(s == 0 ? wv[j].x : wv[j].y);
        bf[j] = sign_plane(nw & emask, (nw & omask) >> 4, sh);
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nk) NQ_LSTORE(buf ^ 1);
    __syncthreads();
  }

#undef NQ_GLOAD
#undef NQ_LSTORE
  // epilogue: lane holds rows 4 * (lane >> 4) + v of each 16 x 16 tile, column lane & 15
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int row = m0 + wm + 16 * i + 4 * (lane >> 4) + v;
      if (row >= a.M) continue;
      const float rs = __builtin_ldexpf(1.0f, a.rexp[row]);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int col = n0 + wn + 16 * j + (lane & 15);
        if (col >= a.N) continue;
        const float c = acc[i][j][v] * rs;
        if (EPI == 0) {
          reinterpret_cast<float*>(a.C)[split * a.split_stride + (size_t)row * a.ldc + col] = c;
        } else {
          const float yv = c * ldf(reinterpret_cast<const SC*>(a.colscale), col);
          const size_t yi = (size_t)row * a.ldc + col;
          if (a.ydt == 0) reinterpret_cast<float*>(a.C)[yi] = yv;
          else reinterpret_cast<uint16_t*>(a.C)[yi] = f32_to_bf16(yv);
        }
      }
    }
  }
}

}  // namespace

GemmPlan gemm_plan(int m, int n, int r, int B) {
  GemmPlan p{};
  p.Bpad = B;
  p.KT1 = ceil_div(n, 128);  // stage 1 contraction: inputs
  p.KT2 = ceil_div(r, 128);  // stage 2 contraction: rank
  p.RT1 = ceil_div(r, 16);
  p.RT2 = ceil_div(m, 16);
  // K splits of the first GEMM when its tiles alone cannot fill the 256 CUs
  // (a small rank: k and v of a 70B block have 96 tiles at 2048 tokens):
  // double S while there are fewer than 384 (tile, range) pairs, each range
  // keeps at least 4 K steps, and S <= 8; then drop splits that would be empty.
  const int T1 = ceil_div(B, BM) * ceil_div(r, BN), nk1 = p.KT1 * 128 / BKG;
  int S = 1;
  while (T1 * S < 384 && S < 8 && nk1 / (2 * S) >= 4) S *= 2;
  p.S1 = ceil_div(nk1, ceil_div(nk1, S));
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  p.off_x16 = take((size_t)B * p.KT1 * 128 * 2);  // X' fp16
  p.off_xexp = take((size_t)B * 4);
  p.off_t32 = take((size_t)p.S1 * B * r * 4);     // T fp32, one partial per K split
  p.off_t16 = take((size_t)B * p.KT2 * 128 * 2);  // T' fp16
  p.off_texp = take((size_t)B * 4);
  p.bytes = o;
  return p;
}

template <typename XT, typename ST>
static hipError_t gemm_forward_t(const FwdArgs& a, const GemmPlan& p) {
  const BlobLayout L = blob_layout(a.m, a.n, a.r, sizeof(ST));
  const uint32_t* U = reinterpret_cast<const uint32_t*>(a.blob + L.off_u);
  const uint32_t* Vt = reinterpret_cast<const uint32_t*>(a.blob + L.off_vt);
  const ST* s1 = reinterpret_cast<const ST*>(a.blob + L.off_s1);
  const ST* g = reinterpret_cast<const ST*>(a.blob + L.off_g);
  const ST* s2 = reinterpret_cast<const ST*>(a.blob + L.off_s2);
  _Float16* x16 = reinterpret_cast<_Float16*>(a.ws + p.off_x16);
  int* xexp = reinterpret_cast<int*>(a.ws + p.off_xexp);
  float* t32 = reinterpret_cast<float*>(a.ws + p.off_t32);
  _Float16* t16 = reinterpret_cast<_Float16*>(a.ws + p.off_t16);
  int* texp = reinterpret_cast<int*>(a.ws + p.off_texp);
  hipStream_t st = a.stream;
  const int B = a.B;

  mark(a, dim3(B), dim3(256));
  launch_row_to_f16(st, B, reinterpret_cast<const XT*>(a.x), (size_t)a.n, 1, (size_t)0, s2, a.n, p.KT1 * 128, x16,
                    xexp);
  const size_t tstride = (size_t)B * a.r;  // elements between the K-split partials of T
  GemmArgs g1{x16, xexp, Vt, B, a.r, p.KT1, t32, (size_t)a.r, nullptr, 0, ceil_div(B, BM), ceil_div(a.r, BN),
              p.S1, tstride};
  const dim3 grid1(8 * ceil_div(g1.MB * g1.NB * g1.S, 8));
  mark(a, grid1, dim3(256));
  hipLaunchKernelGGL((gemm_kernel<0, ST>), grid1, dim3(256), 0, st, g1);
  mark(a, dim3(B), dim3(256));
  launch_row_to_f16(st, B, static_cast<const float*>(t32), (size_t)a.r, p.S1, tstride, g, a.r, p.KT2 * 128, t16,
                    texp);
  GemmArgs g2{t16, texp, U, B, a.m, p.KT2, a.y, (size_t)a.m, s1, a.y_dtype == 0 ? 0 : 2, ceil_div(B, BM),
              ceil_div(a.m, BN), 1, 0};
  mark(a, dim3(8 * ceil_div(g2.MB * g2.NB, 8)), dim3(256));
  hipLaunchKernelGGL((gemm_kernel<1, ST>), dim3(8 * ceil_div(g2.MB * g2.NB, 8)), dim3(256), 0, st, g2);
  mark(a);
  return hipGetLastError();
}

hipError_t gemm_forward(const FwdArgs& a, const GemmPlan& p) {
  if (a.x_dtype == 2) {
    return a.scale_dtype == 1 ? gemm_forward_t<uint16_t, _Float16>(a, p) : gemm_forward_t<uint16_t, float>(a, p);
  }
  return a.scale_dtype == 1 ? gemm_forward_t<float, _Float16>(a, p) : gemm_forward_t<float, float>(a, p);
}

}  // namespace nq
