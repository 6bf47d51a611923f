// Batch 1..4 forward ("dec" path): the decode hot path.
//
// y = s1 * (U (g * (V^T (s2 * x)))) with U, V sign matrices.  Each sign-matrix
// product is  out[row] = 2 * sum_{col: bit=1} v[col] - sum_col v[col]  and the
// masked sum runs on the gfx950 scaled MFMA (16x16x128, fp4 A x fp8 B): a
// packed 32-bit sign word becomes the fp4 A operand with four ANDs (plane j of
// the word is eight nibbles worth 0 or 2^(j-1); plane 3 is shifted down one
// bit), and the activations are the fp8 B operand, each value split into four
// e4m3 pieces with a power-of-two scale per 32-value block (the MFMA's e8m0
// block scale).  Column c = b*4 + q of the MFMA carries piece q of batch row b.
//
// Launches per forward (all asynchronous, no host synchronisation, nothing
// that waits on another workgroup; a kernel boundary is the only global sync,
// because agent-scope fences cost far more on this part than a launch):
//   s1   : t partials = V^T x' over split column ranges.  Each workgroup first
//          issues the loads of its row tiles of packed V^T (a ring of
//          outstanding 1 KiB loads per wave), then encodes x' = s2 * x for its
//          column range straight into LDS, then streams the row tiles.
//   mid  : (only when the partials are too many to fold into s2) t' = g * sum
//          of partials -> image of t' (global)
//   s2   : issues its packed U loads, encodes t' = g * sum of partials into
//          LDS (or copies the mid image), streams U and writes y = s1 * z.
// Every prologue issues all of its loads before it uses any, so it costs one
// memory round trip.
#include "nq_common.h"
#include "nq_internal.h"

namespace nq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

namespace {

constexpr int P = 4;                    // e4m3 pieces per value
constexpr int DEC_MAX_B = 4;
constexpr int VMCNT0 = 0x0F70;          // s_waitcnt immediate: vmcnt(0), other counters untouched            // batch rows of the decode path (4 pieces x B <= 16 MFMA columns)
constexpr int TARGET_WG = 256;          // one workgroup per CU of an MI355X
constexpr size_t LDS_S1 = 64 * 1024;    // image bytes a stage-1 workgroup may stage
constexpr size_t LDS_S2 = 64 * 1024;    // image (+ reduction) bytes of a stage-2 workgroup

// Image of a vector range of KL column tiles, for B batch rows (CW = 4B MFMA
// columns in use):
//   data  [KL][4 lane groups][CW columns][32 bytes]  (the fp8 B-operand register
//         of lane c + 16 g: K values 16g+[0,16) then 64+16g+[0,16))
//   scale [KL][4 K blocks][CW columns] bytes  (e8m0 of the 32-value block)
//   sum   [KL][B] floats  (sum of the represented values of the tile)
__host__ __device__ inline size_t img_data_bytes(int CW) { return (size_t)128 * CW; }
__host__ __device__ inline size_t img_scale_bytes(int CW) { return (size_t)4 * CW; }
__host__ __device__ inline size_t img_tile_bytes(int CW, int B) {
  return img_data_bytes(CW) + img_scale_bytes(CW) + 4 * (size_t)B;
}

struct Img {
  uint8_t* data;
  uint8_t* scale;
  float* sum;
};

__device__ inline Img img_at(uint8_t* base, int KL, int CW) {
  Img im;
  im.data = base;
  im.scale = base + (size_t)KL * img_data_bytes(CW);
  im.sum = reinterpret_cast<float*>(im.scale + (size_t)KL * img_scale_bytes(CW));
  return im;
}

// Cross-lane steps on the VALU (DPP): xor 1 / xor 2 inside a quad, rotate by
// 4 / 8 inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_ROR4 = 0x124, DPP_ROR8 = 0x128;
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  return fmaxf(v, dpp<DPP_XOR2>(v));
}
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<DPP_XOR1>(v);
  return v + dpp<DPP_XOR2>(v);
}
__device__ __forceinline__ float row16_sum(float v) {
  v = quad_sum(v);
  v += dpp<DPP_ROR4>(v);
  return v + dpp<DPP_ROR8>(v);
}

// Encodes 8 consecutive values (chunk j8 of 16 in column tile ktl) of batch row
// b.  The 16 chunks of one (b, ktl) must sit in 16 consecutive active lanes
// (lane & 15 == j8): four lanes form a 32-value block for the block maximum and
// the sixteen form the tile sum.
__device__ __forceinline__ void encode_chunk(const float (&v)[8], int b, int ktl, int j8, int CW, int B, Img im) {
  const int j = j8 & 3;                                   // sign-bit plane of these 8 columns
  const float inv_c = j == 0 ? 2.0f : (j == 1 ? 1.0f : 0.5f);
  const float c = j == 0 ? 0.5f : (j == 1 ? 1.0f : 2.0f);
  float w[8];
  float M = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    w[i] = v[i] * inv_c;
    M = fmaxf(M, fabsf(w[i]));
  }
  M = quad_max(M);
  int e0 = 0;
  if (M > 0.0f && M <= 3.4028235e38f) e0 = (__builtin_amdgcn_frexp_expf(M) - 1) - 7;  // max -> [128, 256)
  e0 = e0 < -127 + 4 * (P - 1) ? -127 + 4 * (P - 1) : e0;
  float orig[8];
#pragma unroll
  for (int i = 0; i < 8; i++) orig[i] = w[i];
  const int g = (j8 & 7) >> 1;                            // lane group holding these K values
  const int off = 8 * (j8 & 1) + 16 * (j8 >> 3);          // byte offset inside the lane record
  const int kb = j8 >> 2;                                 // 32-value block
#pragma unroll
  for (int q = 0; q < P; q++) {
    const int e = e0 - 4 * q;
    const float sc = __builtin_ldexpf(1.0f, -e), us = __builtin_ldexpf(1.0f, e);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(w[0] * sc, w[1] * sc, 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(w[2] * sc, w[3] * sc, lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(w[4] * sc, w[5] * sc, 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(w[6] * sc, w[7] * sc, hi, true);
    w[0] -= __builtin_amdgcn_cvt_f32_fp8(lo, 0) * us;
    w[1] -= __builtin_amdgcn_cvt_f32_fp8(lo, 1) * us;
    w[2] -= __builtin_amdgcn_cvt_f32_fp8(lo, 2) * us;
    w[3] -= __builtin_amdgcn_cvt_f32_fp8(lo, 3) * us;
    w[4] -= __builtin_amdgcn_cvt_f32_fp8(hi, 0) * us;
    w[5] -= __builtin_amdgcn_cvt_f32_fp8(hi, 1) * us;
    w[6] -= __builtin_amdgcn_cvt_f32_fp8(hi, 2) * us;
    w[7] -= __builtin_amdgcn_cvt_f32_fp8(hi, 3) * us;
    const int col = b * P + q;
    uint2 pk;
    pk.x = (uint32_t)lo;
    pk.y = (uint32_t)hi;
    *reinterpret_cast<uint2*>(im.data + ((size_t)(ktl * 4 + g) * CW + col) * 32 + off) = pk;
    if ((j8 & 3) == 0) im.scale[(size_t)ktl * 4 * CW + kb * CW + col] = (uint8_t)(e + 127);
  }
  float rep = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) rep += orig[i] - w[i];     // represented value, exact
  rep = row16_sum(rep * c);
  if (j8 == 0) im.sum[(size_t)ktl * B + b] = rep;
}

// ------------------------------------------------------------------ sources
template <typename T> __device__ inline float ld_f32(const T* p, size_t i);
template <> __device__ inline float ld_f32<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ inline float ld_f32<_Float16>(const _Float16* p, size_t i) { return (float)p[i]; }
template <> __device__ inline float ld_f32<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

// Raw 16-byte words of 8 consecutive elements of type T (1 word for 2-byte
// types, 2 for fp32).
template <typename T> struct Raw8 {
  static constexpr int W = sizeof(T) == 2 ? 1 : 2;
  uint4 w[W];
};

// Loads elements [k, k+8) of p (zero past `end`).  `vec`: p + k is 16-byte
// aligned and k + 8 <= end, so whole 16-byte words are loaded.
template <typename T>
__device__ inline void raw_load(const T* __restrict__ p, int k, int end, bool vec, Raw8<T>& r) {
  if (vec) {
    const uint4* q = reinterpret_cast<const uint4*>(p + k);
#pragma unroll
    for (int i = 0; i < Raw8<T>::W; i++) r.w[i] = q[i];
  } else {
    T t[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      T z;
      __builtin_memset(&z, 0, sizeof(T));
      t[i] = (k + i < end) ? p[k + i] : z;
    }
    __builtin_memcpy(r.w, t, sizeof(t));
  }
}

template <typename T>
__device__ inline void raw_to_f32(const Raw8<T>& r, float (&v)[8]) {
  T t[8];
  __builtin_memcpy(t, r.w, sizeof(t));
#pragma unroll
  for (int i = 0; i < 8; i++) v[i] = ld_f32(t, i);
}

// Encodes x' = s2 * x for column tiles [kt0, kt0 + KL) of every batch row into
// an LDS image, CPT chunks per thread per pass.  Split into the loads of one
// pass and their encoding, so that a kernel can issue the loads of its first
// pass before its weight loads and encode while the weights stream in.
template <typename XT, typename ST>
struct XPass {
  static constexpr int CPT = 4;
  Raw8<XT> rx[CPT];
  Raw8<ST> rs[CPT];

  __device__ __forceinline__ void load(const XT* __restrict__ x, const ST* __restrict__ s2, int n, int B, int kt0,
                                       int KL, bool xvec, int base) {
    const int total = B * KL * 16, nt = blockDim.x;
#pragma unroll
    for (int c = 0; c < CPT; c++) {
      const int ci = base + c * nt + threadIdx.x;
      if (ci < total) {
        const int j8 = ci & 15, ktl = (ci >> 4) % KL, b = (ci >> 4) / KL;
        const int k = (kt0 + ktl) * 128 + 8 * j8;
        const bool in = k + 8 <= n;
        raw_load(x + (size_t)b * n, k, n, xvec && in, rx[c]);
        raw_load(s2, k, n, in, rs[c]);
      }
    }
  }

  __device__ __forceinline__ void encode(int B, int KL, int CW, int base, Img li) {
    const int total = B * KL * 16, nt = blockDim.x;
#pragma unroll
    for (int c = 0; c < CPT; c++) {
      const int ci = base + c * nt + threadIdx.x;
      if (ci < total) {  // whole 16-lane groups (total and nt are multiples of 16)
        const int j8 = ci & 15, ktl = (ci >> 4) % KL, b = (ci >> 4) / KL;
        float xv[8], sv[8], v[8];
        raw_to_f32(rx[c], xv);
        raw_to_f32(rs[c], sv);
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = xv[i] * sv[i];
        encode_chunk(v, b, ktl, j8, CW, B, li);
      }
    }
  }
};

// Encodes t' = g * (sum over the S1 stage-1 splits) for all KT column tiles
// into an LDS image, CPT chunks (all splits) per thread per pass; split into
// loads and encoding like XPass.
template <typename ST>
struct TPass {
  static constexpr int CPT = 2, SMAX = 4;
  float4 pv[CPT][SMAX][2];
  Raw8<ST> rg[CPT];

  __device__ __forceinline__ void load(const float* __restrict__ part, int S1, int B, int Rpad,
                                       const ST* __restrict__ g, int r, int KT, int base) {
    const int total = B * KT * 16, nt = blockDim.x;
#pragma unroll
    for (int c = 0; c < CPT; c++) {
      const int ci = base + c * nt + threadIdx.x;
      if (ci < total) {
        const int j8 = ci & 15, kt = (ci >> 4) % KT, b = (ci >> 4) / KT;
        const int k = kt * 128 + 8 * j8;
        // k < Rpad implies k + 8 <= Rpad (Rpad is a multiple of 16); values past r are masked at encode
#pragma unroll
        for (int s = 0; s < SMAX; s++) {
          if (s < S1 && k < Rpad) {
            const float4* pp = reinterpret_cast<const float4*>(part + ((size_t)s * B + b) * Rpad + k);
            pv[c][s][0] = pp[0];
            pv[c][s][1] = pp[1];
          } else {
            pv[c][s][0] = float4{0.f, 0.f, 0.f, 0.f};
            pv[c][s][1] = float4{0.f, 0.f, 0.f, 0.f};
          }
        }
        raw_load(g, k, r, k + 8 <= r, rg[c]);
      }
    }
  }

  __device__ __forceinline__ void encode(int B, int r, int KT, int CW, int base, Img li) {
    const int total = B * KT * 16, nt = blockDim.x;
#pragma unroll
    for (int c = 0; c < CPT; c++) {
      const int ci = base + c * nt + threadIdx.x;
      if (ci < total) {
        const int j8 = ci & 15, kt = (ci >> 4) % KT, b = (ci >> 4) / KT;
        const int k = kt * 128 + 8 * j8;
        float gv[8], v[8];
        raw_to_f32(rg[c], gv);
        float4 a0 = pv[c][0][0], a1 = pv[c][0][1];
#pragma unroll
        for (int s = 1; s < SMAX; s++) {
          a0.x += pv[c][s][0].x; a0.y += pv[c][s][0].y; a0.z += pv[c][s][0].z; a0.w += pv[c][s][0].w;
          a1.x += pv[c][s][1].x; a1.y += pv[c][s][1].y; a1.z += pv[c][s][1].z; a1.w += pv[c][s][1].w;
        }
        const float t[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = (k + i < r) ? t[i] * gv[i] : 0.0f;
        encode_chunk(v, b, kt, j8, CW, B, li);
      }
    }
  }
};

// ------------------------------------------------------------------ image kernels
// Image of g * (sum of stage-1 partials) into global memory, one chunk per
// thread (used when S1 * B is too large to fold this into stage 2).
template <typename ST>
__global__ void __launch_bounds__(256) dec_mid_kernel(const float* __restrict__ part, int S1, int Rpad,
                                                      const ST* __restrict__ g, int r, int B, int KT, int CW,
                                                      uint8_t* __restrict__ img) {
  const int ci = blockIdx.x * 256 + threadIdx.x;
  if (ci >= B * KT * 16) return;  // whole 16-lane groups leave together (the total is a multiple of 16)
  const int j8 = ci & 15, kt = (ci >> 4) % KT, b = (ci >> 4) / KT;
  const int k = kt * 128 + 8 * j8;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float t = 0.0f;
    if (k + i < r) {
      for (int s = 0; s < S1; s++) t += part[((size_t)s * B + b) * Rpad + k + i];
      t *= ld_f32(g, k + i);
    }
    v[i] = t;
  }
  encode_chunk(v, b, kt, j8, CW, B, img_at(img, KT, CW));
}

// Copies KL tiles [kt0, kt0 + KL) of a global image (KT tiles) into LDS; each
// pass issues up to 8 16-byte loads per thread before writing any of them.
__device__ __forceinline__ void copy_image(const uint8_t* __restrict__ gimg, int KT, int kt0, int KL, int CW, int B,
                                  uint8_t* lds) {
  const Img src = img_at(const_cast<uint8_t*>(gimg), KT, CW);
  const Img dst = img_at(lds, KL, CW);
  const int nt = blockDim.x, t = threadIdx.x;
  // the three regions as one list of 16-byte words: data, scale, then sums
  const int nd = KL * (int)img_data_bytes(CW) / 16;
  const int ns = KL * (int)img_scale_bytes(CW) / 16;
  const int nsum = (KL * B + 3) / 4;  // sums copied as whole words; the tail word may overrun into padding
  const uint4* sd = reinterpret_cast<const uint4*>(src.data + (size_t)kt0 * img_data_bytes(CW));
  const uint4* ss = reinterpret_cast<const uint4*>(src.scale + (size_t)kt0 * img_scale_bytes(CW));
  uint4* dd = reinterpret_cast<uint4*>(dst.data);
  uint4* ds = reinterpret_cast<uint4*>(dst.scale);
  const int total = nd + ns;
  constexpr int CPT = 8;
  for (int base = 0; base < total; base += CPT * nt) {
    uint4 w[CPT];
#pragma unroll
    for (int c = 0; c < CPT; c++) {
      const int i0 = base + c * nt + t;
      const int i = i0 < total ? i0 : 0;  // past the end: re-read word 0 (in bounds), never stored
      const uint4* src = i < nd ? sd + i : ss + (i - nd);
      w[c] = *src;
    }
#pragma unroll
    for (int c = 0; c < CPT; c++) {
      const int i = base + c * nt + t;
      uint4* dst = i < nd ? dd + i : ds + (i - nd);
      if (i < total) *dst = w[c];
    }
  }
  (void)nsum;
  for (int i = t; i < KL * B; i += nt) dst.sum[i] = src.sum[(size_t)kt0 * B + i];
}

// ------------------------------------------------------------------ stage loop
// Per-lane view of an LDS image.  Lane L (column c = L & 15, lane group
// g = L >> 4) reads the record of column c mod CW: MFMA columns c >= CW only
// feed output columns that are never read, so they may carry any finite or
// non-finite copy, and no lane needs a branch or a zero fill.
template <int CW>
struct LaneImg {
  const uint8_t* data;   // this lane's record in column tile 0
  const uint8_t* scale;  // this lane's scale byte in column tile 0
  __device__ LaneImg(const Img& im, int lane) {
    const int c = (lane & 15) % CW, g = lane >> 4;
    data = im.data + (g * CW + c) * 32;
    scale = im.scale + g * CW + c;
  }
};

__device__ inline v8i sign_planes(uint32_t word) {
  return v8i{(int)(word & 0x11111111u), (int)(word & 0x22222222u), (int)(word & 0x44444444u),
             (int)((word >> 1) & 0x44444444u), 0, 0, 0, 0};
}

__device__ inline int full_quads(int KT, int q0, int q1) {
  const int qf = KT >> 2;
  const int e = q1 < qf ? q1 : qf;
  return e > q0 ? e - q0 : 0;
}

// One wave's work: RM row tiles rt0 .. rt0+RM-1 of a packed sign matrix with
// KT column tiles (rows past RT re-read the last row tile and are not stored),
// over quads [qa, qb) (wave-uniform, at most 16/RM of them full).  All loads
// are issued up front into a 16-quad (64-VGPR) buffer; then for every column
// tile the B operand is read from LDS once and feeds one MFMA per row tile,
// each row tile with its own accumulator.
template <int RM>
struct WaveWork {
  static constexpr int QW = 16 / RM;
  u4v w[RM][QW];
  int rt0, qa, qb, nfull;
};

template <int RM>
__device__ __forceinline__ void wave_load(const uint32_t* __restrict__ P, int KT, int RT, WaveWork<RM>& ww, int lane) {
  constexpr int QW = WaveWork<RM>::QW;
  ww.nfull = full_quads(KT, ww.qa, ww.qb);
  if (ww.nfull == 0) return;  // only the short last quad (read word by word later), or nothing
  const int last = ww.qa + ww.nfull - 1;
#pragma unroll
  for (int r = 0; r < RM; r++) {
    const int rt = min(ww.rt0 + r, RT - 1);
    const u4v* qp = reinterpret_cast<const u4v*>(P + (size_t)rt * KT * 64) + lane;
#pragma unroll
    for (int j = 0; j < QW; j++) {
      const int q = ww.qa + j < last ? ww.qa + j : last;
      ww.w[r][j] = __builtin_nontemporal_load(qp + (size_t)q * 64);
    }
  }
}

template <int CW>
__device__ __forceinline__ v8i image_b(const LaneImg<CW>& im, int kl, int* sb) {
  const uint4* d = reinterpret_cast<const uint4*>(im.data + kl * (4 * CW * 32));
  const uint4 lo = d[0], hi = d[1];
  *sb = im.scale[kl * (4 * CW)];
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int CW, int RM>
__device__ __forceinline__ void wave_mma(const uint32_t* __restrict__ P, int KT, int RT, const WaveWork<RM>& ww,
                                         const LaneImg<CW>& im, int ktbase, int lane, v4f (&acc)[RM]) {
  constexpr int QW = WaveWork<RM>::QW;
#pragma unroll
  for (int j = 0; j < QW; j++) {
    if (j < ww.nfull) {
#pragma unroll
      for (int t = 0; t < 4; t++) {
        int sb;
        const v8i Bv = image_b<CW>(im, 4 * (ww.qa + j) + t - ktbase, &sb);
#pragma unroll
        for (int r = 0; r < RM; r++) {
          const uint32_t word = t == 0 ? ww.w[r][j].x : (t == 1 ? ww.w[r][j].y : (t == 2 ? ww.w[r][j].z : ww.w[r][j].w));
          acc[r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sign_planes(word), Bv, acc[r], 4, 0, 0, 127, 0, sb);
        }
      }
    }
  }
  const int qf = KT >> 2;
  if (ww.qb > qf && qf >= ww.qa) {  // the row tiles' last quad holds f < 4 words per lane
    const int f = KT - 4 * qf;
    for (int i = 0; i < f; i++) {
      int sb;
      const v8i Bv = image_b<CW>(im, 4 * qf + i - ktbase, &sb);
#pragma unroll
      for (int r = 0; r < RM; r++) {
        const int rt = min(ww.rt0 + r, RT - 1);
        const uint32_t word = P[(size_t)rt * KT * 64 + (size_t)qf * 256 + lane * f + i];
        acc[r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sign_planes(word), Bv, acc[r], 4, 0, 0, 127, 0, sb);
      }
    }
  }
}

// Total of the represented values of column tiles [0, KL) of the image sums,
// per batch row, in every lane.
__device__ __forceinline__ void range_sums(const float* sum_lds, int KL, int B, int lane, float (&S)[4]) {
#pragma unroll
  for (int b = 0; b < 4; b++) {
    float s = 0.0f;
    if (b < B) {
      for (int k = lane; k < KL; k += 64) s += sum_lds[k * B + b];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    }
    S[b] = s;
  }
}

// Sum over the pieces (MFMA columns 4b .. 4b+3) and the "2 * masked - total"
// step for one accumulator.  Valid in lanes whose column is 4b (b < B); rows
// 4 * (lane >> 4) + v of the row tile.
__device__ __forceinline__ void finish_acc(v4f acc, const float (&S)[4], int lane, float (&z)[4]) {
  const int b = (lane & 15) >> 2;
  const float Sb = b == 0 ? S[0] : (b == 1 ? S[1] : (b == 2 ? S[2] : S[3]));
#pragma unroll
  for (int v = 0; v < 4; v++) z[v] = 2.0f * quad_sum(acc[v]) - Sb;  // the 4 pieces of row b are one quad
}

// Adds the per-wave results of the KS column parts of a workgroup in a fixed
// order through LDS (red: KS x RM x 16 lanes-with-results x 4 floats) and
// calls out(r, b, 4 row values) for row tile r < RG, the rows spread over the
// waves (row tile r is written by wave r mod KS).
template <int RM, typename F>
__device__ __forceinline__ void reduce_parts(float* red, const float (&z)[RM][4], int RG, int KS, int ks, int lane,
                                             int B, F&& out) {
  const int c = lane & 15, b = c >> 2;
  const bool valid = (c & 3) == 0 && b < B;
  const int slot = b * 4 + (lane >> 4);  // 16 slots: batch row x lane group
  if (KS == 1) {
    if (valid) {
#pragma unroll
      for (int r = 0; r < RM; r++)
        if (r < RG) out(r, b, float4{z[r][0], z[r][1], z[r][2], z[r][3]});
    }
    return;
  }
  if (valid) {
#pragma unroll
    for (int r = 0; r < RM; r++) {
      float4* dst = reinterpret_cast<float4*>(red + (((size_t)ks * RM + r) * 16 + slot) * 4);
      *dst = float4{z[r][0], z[r][1], z[r][2], z[r][3]};
    }
  }
  __syncthreads();
  if (!valid) return;
  for (int r = ks; r < RG; r += KS) {
    float4 t = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < KS; k++) {
      const float4 u = *reinterpret_cast<const float4*>(red + (((size_t)k * RM + r) * 16 + slot) * 4);
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    }
    out(r, b, t);
  }
}

// ------------------------------------------------------------------ stage 1
// Workgroup = (row group of RG row tiles, column split); its KS waves split
// the split's quads.  Writes part[(split * B + b) * Rpad + row].
struct S1Args {
  const uint32_t* vt;  // packed V^T: rows = rank, columns = inputs
  int RT, KT, KL, RG, KS;
  const void* x;       // B x n activations
  const void* s2;      // n input scales
  int n;
  bool xvec;           // x rows may be read in aligned 16-byte words
  int CW, B;
  float* part;
  int Rpad;
  int red_off;         // byte offset of the reduction buffer in LDS
};

template <typename XT, typename ST, int BB, int RM>
__global__ void __launch_bounds__(512) dec_s1_kernel(S1Args a) {
  constexpr int CW = 4 * BB;
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.y;
  const int kt0 = split * a.KL;
  const int kt1 = min(a.KT, kt0 + a.KL);
  const int KLr = kt1 - kt0;
  const int q0 = kt0 >> 2, q1 = (kt1 + 3) >> 2;
  WaveWork<RM> ww;
  ww.rt0 = blockIdx.x * RM;
  const int RG = min(RM, a.RT - ww.rt0);
  ww.qa = q0 + (int)(((long long)(q1 - q0) * wave) / a.KS);
  ww.qb = q0 + (int)(((long long)(q1 - q0) * (wave + 1)) / a.KS);
  const XT* x = reinterpret_cast<const XT*>(a.x);
  const ST* s2 = reinterpret_cast<const ST*>(a.s2);
  const Img li = img_at(lds, KLr, CW);
  const int per_pass = XPass<XT, ST>::CPT * blockDim.x, total = BB * KLr * 16;
  XPass<XT, ST> xp;
  xp.load(x, s2, a.n, BB, kt0, KLr, a.xvec, 0);
  // the prologue's loads return first: once the weight stream is issued, a
  // load that misses the caches waits behind it
  __builtin_amdgcn_s_waitcnt(VMCNT0);
  wave_load<RM>(a.vt, a.KT, a.RT, ww, lane);
  xp.encode(BB, KLr, CW, 0, li);
  for (int base = per_pass; base < total; base += per_pass) {
    xp.load(x, s2, a.n, BB, kt0, KLr, a.xvec, base);
    xp.encode(BB, KLr, CW, base, li);
  }
  __syncthreads();
  const LaneImg<CW> im(li, lane);
  v4f acc[RM];
#pragma unroll
  for (int r = 0; r < RM; r++) acc[r] = v4f{0.f, 0.f, 0.f, 0.f};
  wave_mma<CW, RM>(a.vt, a.KT, a.RT, ww, im, kt0, lane, acc);
  float S[4];
  const int kta = 4 * ww.qa - kt0, ktb = min(kt1, 4 * ww.qb) - kt0;
  range_sums(li.sum + (size_t)kta * BB, ktb - kta, BB, lane, S);
  float z[RM][4];
#pragma unroll
  for (int r = 0; r < RM; r++) finish_acc(acc[r], S, lane, z[r]);
  float* red = reinterpret_cast<float*>(lds + a.red_off);
  reduce_parts<RM>(red, z, RG, a.KS, wave, lane, BB, [&](int r, int b, float4 t) {
    *reinterpret_cast<float4*>(a.part + ((size_t)split * BB + b) * a.Rpad + (ww.rt0 + r) * 16 + 4 * (lane >> 4)) = t;
  });
}

// ------------------------------------------------------------------ stage 2
// Workgroup = row group of RG row tiles; its KS waves split the quads of the
// rank dimension.  Prologue: t' = g * (sum of partials) encoded into LDS (or a
// copy of the mid image).  Epilogue: y = s1 * z.
struct S2Args {
  const uint32_t* u;  // packed U: rows = outputs, columns = rank
  int RT, KT, RG, KS;
  const uint8_t* img;  // global image of t' (not fused) or null
  const float* part;
  int S1, Rpad1, r;
  const void* g;
  int CW, B;
  const void* s1;
  int sdt;
  void* y;
  int ydt, m;
  int red_off;
};

template <typename ST, bool FUSED, int BB, int RM>
__global__ void __launch_bounds__(512) dec_s2_kernel(S2Args a) {
  constexpr int CW = 4 * BB;
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nq = (a.KT + 3) >> 2;
  WaveWork<RM> ww;
  ww.rt0 = blockIdx.x * RM;
  const int RG = min(RM, a.RT - ww.rt0);
  ww.qa = (int)(((long long)nq * wave) / a.KS);
  ww.qb = (int)(((long long)nq * (wave + 1)) / a.KS);
  const Img li = img_at(lds, a.KT, CW);
  if (FUSED) {
    const ST* g = reinterpret_cast<const ST*>(a.g);
    const int per_pass = TPass<ST>::CPT * blockDim.x, total = BB * a.KT * 16;
    TPass<ST> tp;
    tp.load(a.part, a.S1, BB, a.Rpad1, g, a.r, a.KT, 0);
    __builtin_amdgcn_s_waitcnt(VMCNT0);  // prologue loads first, then the weight stream
    wave_load<RM>(a.u, a.KT, a.RT, ww, lane);
    tp.encode(BB, a.r, a.KT, CW, 0, li);
    for (int base = per_pass; base < total; base += per_pass) {
      tp.load(a.part, a.S1, BB, a.Rpad1, g, a.r, a.KT, base);
      tp.encode(BB, a.r, a.KT, CW, base, li);
    }
  } else {
    wave_load<RM>(a.u, a.KT, a.RT, ww, lane);
    copy_image(a.img, a.KT, 0, a.KT, CW, BB, lds);
  }
  __syncthreads();
  const LaneImg<CW> im(li, lane);
  v4f acc[RM];
#pragma unroll
  for (int r = 0; r < RM; r++) acc[r] = v4f{0.f, 0.f, 0.f, 0.f};
  wave_mma<CW, RM>(a.u, a.KT, a.RT, ww, im, 0, lane, acc);
  float S[4];
  const int kta = 4 * ww.qa, ktb = min(a.KT, 4 * ww.qb);
  range_sums(li.sum + (size_t)kta * BB, ktb - kta, BB, lane, S);
  float z[RM][4];
#pragma unroll
  for (int r = 0; r < RM; r++) finish_acc(acc[r], S, lane, z[r]);
  float* red = reinterpret_cast<float*>(lds + a.red_off);
  const ST* s1 = reinterpret_cast<const ST*>(a.s1);
  reduce_parts<RM>(red, z, RG, a.KS, wave, lane, BB, [&](int r, int b, float4 t) {
    const float zz[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int row = (ww.rt0 + r) * 16 + 4 * (lane >> 4) + v;
      if (row < a.m) {
        const float yv = ld_f32(s1, row) * zz[v];
        const size_t yi = (size_t)b * a.m + row;
        if (a.ydt == 0) reinterpret_cast<float*>(a.y)[yi] = yv;
        else reinterpret_cast<uint16_t*>(a.y)[yi] = f32_to_bf16(yv);
      }
    }
  });
}

}  // namespace

// ------------------------------------------------------------------ plan
// Rows per workgroup (RM, a power of two <= 8) and column-part waves (KS <= 8)
// for a stage of RT row tiles, `splits` column splits, whose waves share
// `quads` quads.  The largest RM that still gives `groups` row groups and
// whose 16-quad buffer holds RM x ceil(quads/KS); KS as large as the quads
// allow (the prologue's parallelism) while the whole grid stays within 8
// resident waves per CU (2 per SIMD at up to 256 VGPRs), so that it runs in
// one round.  False if no shape fits.
static bool pick_shape(int RT, int splits, int quads, int groups, int* RM, int* KS) {
  for (int rm = 8; rm >= 1; rm /= 2) {
    const int wgs = ceil_div(RT, rm) * splits;
    if (rm > 1 && ceil_div(RT, rm) < groups) continue;
    int ks = quads < 8 ? quads : 8;
    const int per_cu = ceil_div(wgs, TARGET_WG);  // workgroups a CU must hold at once
    while (ks > 1 && per_cu * ks > 8) ks--;
    const int qw = ceil_div(quads, ks);
    if (rm * qw > 16) continue;
    *RM = rm;
    *KS = ks;
    return true;
  }
  return false;
}

DecPlan dec_plan(int m, int n, int r, int B) {
  DecPlan p{};
  p.ok = false;
  if (B < 1 || B > DEC_MAX_B) return p;
  p.B = B;
  p.CW = B * P;
  const size_t tb = img_tile_bytes(p.CW, B);
  const size_t red_bytes = (size_t)8 * 8 * 16 * 16;  // KS <= 8 parts x RM <= 8 row tiles x 16 slots x float4
  // stage 1: rows = rank, columns = inputs; column splits of KL1 tiles (the
  // split's image is built in LDS), at most four partial sums per rank value
  p.RT1 = ceil_div(r, 16);
  p.KT1 = ceil_div(n, 128);
  const int quads1 = ceil_div(p.KT1, 4);
  int klmax = (int)((LDS_S1 - red_bytes) / tb) / 4 * 4;
  if (klmax < 4) return p;
  {
    int rm, ks;
    if (!pick_shape(p.RT1, 1, 4, 128, &rm, &ks)) return p;  // provisional row groups for the split count
    const int rowgroups = ceil_div(p.RT1, rm);
    // every stage-2 workgroup reads all S1 partial vectors of t: keep S1 small
    // where the rank is large (the reads are S1 x r x 4 bytes per workgroup)
    const int smax = r >= 2048 ? 2 : 4;
    int s = ceil_div(TARGET_WG, rowgroups);
    s = s > smax ? smax : s;
    s = s > quads1 ? quads1 : s;
    s = s < 1 ? 1 : s;
    const int s_lds = ceil_div(p.KT1, klmax);
    if (s < s_lds) s = s_lds;
    p.KL1 = 4 * ceil_div(ceil_div(p.KT1, s), 4);
    p.S1 = ceil_div(p.KT1, p.KL1);
    if (!pick_shape(p.RT1, p.S1, ceil_div(p.KL1, 4), ceil_div(TARGET_WG, p.S1), &p.RG1, &p.KS1)) return p;
  }
  p.QM1 = ceil_div(ceil_div(p.KL1, 4), p.KS1);
  p.Rpad1 = p.RT1 * 16;
  p.red1 = align_up((size_t)p.KL1 * tb, 16);
  p.lds1 = p.red1 + red_bytes;
  // stage 2: rows = outputs, columns = rank
  p.RT2 = ceil_div(m, 16);
  p.KT2 = ceil_div(r, 128);
  const int quads2 = ceil_div(p.KT2, 4);
  if (!pick_shape(p.RT2, 1, quads2, TARGET_WG, &p.RG2, &p.KS2)) return p;
  {
    // the prologue encodes B x KT2 x 16 chunks, 2 per thread per pass: prefer
    // a shape that does it in one pass, if that keeps >= 3/4 of the CUs busy
    const int chunks = B * p.KT2 * 16;
    int rm, ks;
    if (chunks > 2 * 64 * p.KS2 && pick_shape(p.RT2, 1, quads2, TARGET_WG * 3 / 4, &rm, &ks) &&
        chunks <= 2 * 64 * ks) {
      p.RG2 = rm;
      p.KS2 = ks;
    }
  }
  p.QM2 = ceil_div(quads2, p.KS2);
  p.red2 = align_up((size_t)p.KT2 * tb, 16);
  p.lds2 = p.red2 + red_bytes;
  if (p.lds2 > LDS_S2) return p;
  p.fused_mid = p.S1 <= 4 && p.S1 * B <= 4;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  p.off_img1 = 0;
  p.off_part = take((size_t)p.S1 * B * p.Rpad1 * 4);
  p.off_img2 = take(p.fused_mid ? 0 : (size_t)p.KT2 * tb);
  p.bytes = o;
  p.ok = true;
  return p;
}

template <typename XT, typename ST, int BB>
static hipError_t dec_forward_t(const FwdArgs& a, const DecPlan& p) {
  const int sb = sizeof(ST);
  BlobLayout L = blob_layout(a.m, a.n, a.r, sb);
  const uint32_t* U = reinterpret_cast<const uint32_t*>(a.blob + L.off_u);
  const uint32_t* Vt = reinterpret_cast<const uint32_t*>(a.blob + L.off_vt);
  const ST* s1 = reinterpret_cast<const ST*>(a.blob + L.off_s1);
  const ST* g = reinterpret_cast<const ST*>(a.blob + L.off_g);
  const ST* s2 = reinterpret_cast<const ST*>(a.blob + L.off_s2);
  hipStream_t st = a.stream;
  float* part = reinterpret_cast<float*>(a.ws + p.off_part);
  uint8_t* img2 = a.ws + p.off_img2;
  const bool xvec = (a.n % 8 == 0) && (reinterpret_cast<uintptr_t>(a.x) % 16 == 0);

  S1Args k1{Vt, p.RT1, p.KT1, p.KL1, p.RG1, p.KS1, a.x, s2, a.n, xvec, p.CW, a.B, part, p.Rpad1, (int)p.red1};
  mark(a);
  {
    dim3 g1(ceil_div(p.RT1, p.RG1), p.S1), b1(64 * p.KS1);
    switch (p.RG1) {
      case 8: hipLaunchKernelGGL((dec_s1_kernel<XT, ST, BB, 8>), g1, b1, p.lds1, st, k1); break;
      case 4: hipLaunchKernelGGL((dec_s1_kernel<XT, ST, BB, 4>), g1, b1, p.lds1, st, k1); break;
      case 2: hipLaunchKernelGGL((dec_s1_kernel<XT, ST, BB, 2>), g1, b1, p.lds1, st, k1); break;
      default: hipLaunchKernelGGL((dec_s1_kernel<XT, ST, BB, 1>), g1, b1, p.lds1, st, k1); break;
    }
  }
  if (!p.fused_mid) {
    const int c2 = a.B * p.KT2 * 16;
    mark(a);
    hipLaunchKernelGGL((dec_mid_kernel<ST>), dim3(ceil_div(c2, 256)), dim3(256), 0, st, part, p.S1, p.Rpad1, g,
                       a.r, a.B, p.KT2, p.CW, img2);
  }
  S2Args k2{U, p.RT2, p.KT2, p.RG2, p.KS2, p.fused_mid ? nullptr : img2, part, p.S1, p.Rpad1, a.r, g, p.CW, a.B,
            s1, a.scale_dtype, a.y, a.y_dtype == 0 ? 0 : 2, a.m, (int)p.red2};
  dim3 g2(ceil_div(p.RT2, p.RG2)), b2(64 * p.KS2);
  mark(a);
#define NQ_S2(F, RM) hipLaunchKernelGGL((dec_s2_kernel<ST, F, BB, RM>), g2, b2, p.lds2, st, k2)
  if (p.fused_mid) {
    switch (p.RG2) {
      case 8: NQ_S2(true, 8); break;
      case 4: NQ_S2(true, 4); break;
      case 2: NQ_S2(true, 2); break;
      default: NQ_S2(true, 1); break;
    }
  } else {
    switch (p.RG2) {
      case 8: NQ_S2(false, 8); break;
      case 4: NQ_S2(false, 4); break;
      case 2: NQ_S2(false, 2); break;
      default: NQ_S2(false, 1); break;
    }
  }
#undef NQ_S2
  mark(a);
  return hipGetLastError();
}

template <typename XT, typename ST>
static hipError_t dec_forward_b(const FwdArgs& a, const DecPlan& p) {
  switch (a.B) {
    case 1: return dec_forward_t<XT, ST, 1>(a, p);
    case 2: return dec_forward_t<XT, ST, 2>(a, p);
    case 3: return dec_forward_t<XT, ST, 3>(a, p);
    default: return dec_forward_t<XT, ST, 4>(a, p);
  }
}

hipError_t dec_forward(const FwdArgs& a, const DecPlan& p) {
  if (a.x_dtype == 2) {
    return a.scale_dtype == 1 ? dec_forward_b<uint16_t, _Float16>(a, p) : dec_forward_b<uint16_t, float>(a, p);
  }
  return a.scale_dtype == 1 ? dec_forward_b<float, _Float16>(a, p) : dec_forward_b<float, float>(a, p);
}

}  // namespace nq
