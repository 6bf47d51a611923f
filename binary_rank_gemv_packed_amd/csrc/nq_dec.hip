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
// that waits on another workgroup; a kernel boundary is the only global sync):
//   s1   : t partials = V^T x' over split column ranges.  Each workgroup issues
//          the loads of its slice of x and s2, then its packed V^T row tiles
//          (16 x 1 KiB per wave, all in flight), encodes x' = s2 * x for its
//          column range into LDS while the weights stream in, then runs the
//          MFMAs and writes its partial sums.
//   mid  : (only when the partials are too many to fold into s2) t' = g * sum
//          of partials -> image of t' (global)
//   s2   : the same on packed U, with t' = g * sum of partials encoded in the
//          prologue (or the mid image copied); writes y = s1 * z.
// Every load of a prologue is issued before the weights and without a branch,
// so a prologue costs one memory round trip and the encoder never waits for
// the weight stream.
#include <climits>
#include <type_traits>

#include "nq_common.h"
#include "nq_internal.h"

namespace nq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

namespace {

constexpr int P = 4;                    // e4m3 pieces per value
constexpr int DEC_MAX_B = 4;           // batch rows of the decode path (4 pieces x B <= 16 MFMA columns)
constexpr int TARGET_WG = 256;          // one workgroup per CU of an MI355X
constexpr int MIN_WG = 128;             // fewest workgroups a stage is cut into (half the CUs)
constexpr int WAVE_BUDGET = 256 * 12;   // resident waves of the chip at <= 168 VGPRs (3 per SIMD)
constexpr int MIN_ROW_WAVES = 256;      // fewest waves a row-split stage 2 may have
constexpr int TALL_ROW_TILES = 2048;    // row tiles from which stage 2 takes two row tiles per wave
constexpr int RM2_QUADS = 10;           // quads per row tile the two-row-tile waves hold (20-quad buffer)
// prologue chunks per thread of the two-row-tile stage 2 for B batch rows:
// enough for B x 10 quads x 64 chunks in one pass of 512 threads
__host__ __device__ constexpr int rm2_chunks_per_thread(int B) { return B == 1 ? 2 : (B == 2 ? 3 : (B == 3 ? 4 : 5)); }
constexpr size_t S1_LDS_BYTES = 8 * 16 * 4;  // output scales of a stage-2 workgroup's <= 8 row tiles
constexpr size_t LDS_S1 = 64 * 1024;    // image bytes a stage-1 workgroup may stage
constexpr size_t LDS_S2 = 64 * 1024;    // image (+ reduction) bytes of a stage-2 workgroup
// LDS of one gfx950 workgroup (160 KiB).  A plan first keeps to the budgets
// above (the measured shapes of the B = 1 and 2 chains); when that gives no
// plan (three or four batch rows, or envelope terms, at ranks of several
// thousand: the image of t' then needs 85 KiB at rank 5079) it is made again
// with this budget for both stages, rather than falling back to chunks that
// read the weights once per two batch rows.
constexpr size_t LDS_MAX = 160 * 1024;

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
//
// The fp4 plane of these columns multiplies the piece by c = 2^cexp (0.5, 1,
// 2, 2 for planes 0..3), so the MFMA sees piece * 2^(e + cexp): pieces are cut
// from v * 2^-cexp, with the plane factor folded into each piece's scale and
// the residual kept in the domain of v.
__device__ __forceinline__ void encode_chunk(const float (&v)[8], int b, int ktl, int j8, int CW, int B, Img im) {
  const int j = j8 & 3;                                   // sign-bit plane of these 8 columns
  const int cexp = j == 0 ? -1 : (j == 1 ? 0 : 1);
  float M = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) M = fmaxf(M, fabsf(v[i]));
  M = quad_max(__builtin_ldexpf(M, -cexp));               // block maximum of v * 2^-cexp
  int e0 = 0;
  if (M > 0.0f && M <= 3.4028235e38f) e0 = (__builtin_amdgcn_frexp_expf(M) - 1) - 7;  // max -> [128, 256)
  e0 = e0 < -127 + 4 * (P - 1) ? -127 + 4 * (P - 1) : e0;
  float w[8];
#pragma unroll
  for (int i = 0; i < 8; i++) w[i] = v[i];
  const int g = (j8 & 7) >> 1;                            // lane group holding these K values
  const int off = 8 * (j8 & 1) + 16 * (j8 >> 3);          // byte offset inside the lane record
  const int kb = j8 >> 2;                                 // 32-value block
  uint8_t* dst = im.data + (size_t)(ktl * 4 + g) * CW * 32 + off;
  uint8_t* sdst = im.scale + (size_t)ktl * 4 * CW + kb * CW;
#pragma unroll
  for (int q = 0; q < P; q++) {
    const int e = e0 - 4 * q;
    const float sc = __builtin_ldexpf(1.0f, -e - cexp), us = __builtin_ldexpf(1.0f, e + cexp);
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
    *reinterpret_cast<uint2*>(dst + col * 32) = pk;
    if (j == 0) sdst[col] = (uint8_t)(e + 127);
  }
  float rep = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) rep += v[i] - w[i];         // represented value, exact
  rep = row16_sum(rep);
  if (j8 == 0) im.sum[(size_t)ktl * B + b] = rep;
}

// Batch row and column tile of chunk group t (= chunk index / 16) of a range
// of KL column tiles for BB <= 4 batch rows, without a division.
template <int BB>
__device__ __forceinline__ void chunk_pos(int t, int KL, int& b, int& ktl) {
  b = 0;
#pragma unroll
  for (int i = 1; i < BB; i++) b += t >= i * KL ? 1 : 0;
  ktl = t - b * KL;
}

// Rank-l envelope: internal batch row b (< 4) is input row b / env under
// scale row b % env, for env in 1..4 (without a division).
__device__ __forceinline__ void env_split(int b, int env, int& xr, int& sr) {
  xr = env == 1 ? b : (env == 2 ? b >> 1 : (env == 3 ? (b >= 3 ? 1 : 0) : 0));
  sr = b - xr * env;
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

// Loads the 16-byte word(s) holding elements [k, k+8) of p, k a multiple of 8.
// Every such word with k < end must be readable (a 16-byte aligned p whose
// allocation reaches the next 16-byte boundary past end); k >= end reads the
// first word instead.  Elements at or past `end` are garbage: the encoder masks
// them.  No branch, so that all loads of a pass are in flight together.
template <typename T>
__device__ __forceinline__ void raw_words(const T* __restrict__ p, int k, int end, Raw8<T>& r) {
  const uint4* q = reinterpret_cast<const uint4*>(p + (k < end ? k : 0));
#pragma unroll
  for (int i = 0; i < Raw8<T>::W; i++) r.w[i] = q[i];
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
template <typename XT, typename ST, int BB>
struct XPass {
  static constexpr int CPT = 4;
  Raw8<XT> rx[CPT];
  Raw8<ST> rs[CPT];

  // x rows start every xstride elements, 16-byte aligned, xstride a multiple
  // of 8; lanes past the last chunk load a copy of it.
  // With an envelope of env terms, batch row b reads x row b / env and s2 row
  // b % env (s2 rows s2_stride apart).
  __device__ __forceinline__ void load(const XT* __restrict__ x, int xstride, const ST* __restrict__ s2, int n,
                                       int kt0, int KL, int base, int env, int s2_stride) {
    const int total = BB * KL * 16, nt = blockDim.x;
#pragma unroll
    for (int c = 0; c < CPT; c++) {
      const int ci = base + c * nt + threadIdx.x;
      const int cc = ci < total ? ci : total - 1;
      int b, ktl, xr, sr;
      chunk_pos<BB>(cc >> 4, KL, b, ktl);
      env_split(b, env, xr, sr);
      const int k = (kt0 + ktl) * 128 + 8 * (cc & 15);
      raw_words(x + (size_t)xr * xstride, k, n, rx[c]);
      raw_words(s2 + (size_t)sr * s2_stride, k, n, rs[c]);
    }
  }

  __device__ __forceinline__ void encode(int n, int KL, int kt0, int CW, int base, Img li) {
    const int total = BB * KL * 16, nt = blockDim.x;
#pragma unroll
    for (int c = 0; c < CPT; c++) {
      const int ci = base + c * nt + threadIdx.x;
      if (ci < total) {  // whole 16-lane groups (total and nt are multiples of 16)
        const int j8 = ci & 15;
        int b, ktl;
        chunk_pos<BB>(ci >> 4, KL, b, ktl);
        const int k = (kt0 + ktl) * 128 + 8 * j8;
        float xv[8], sv[8], v[8];
        raw_to_f32(rx[c], xv);
        raw_to_f32(rs[c], sv);
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = xv[i] * sv[i];
        if (k + 8 > n) {  // the ragged end of the input
#pragma unroll
          for (int i = 0; i < 8; i++) v[i] = k + i < n ? v[i] : 0.0f;
        }
        encode_chunk(v, b, ktl, j8, CW, BB, li);
      }
    }
  }
};

// Encodes t' = g * (sum over the S1 <= SM stage-1 splits) for all KT column
// tiles into an LDS image, CPT chunks (all splits) per thread per pass; split
// into loads and encoding like XPass, and branch-free like it (split indices
// past S1 re-read split S1 - 1 and are left out of the sum).
template <typename ST, int SM, int BB, int CPTV = 2>
struct TPass {
  static constexpr int CPT = CPTV;
  float4 pv[CPT][SM][2];
  Raw8<ST> rg[CPT];

  __device__ __forceinline__ void load(const float* __restrict__ part, int S1, int Rpad,
                                       const ST* __restrict__ g, int r, int KT, int base) {
    const int total = BB * KT * 16, nt = blockDim.x;
#pragma unroll
    for (int c = 0; c < CPT; c++) {
      const int ci = base + c * nt + threadIdx.x;
      const int cc = ci < total ? ci : total - 1;
      int b, kt;
      chunk_pos<BB>(cc >> 4, KT, b, kt);
      const int k = kt * 128 + 8 * (cc & 15);
      // k < Rpad implies k + 8 <= Rpad (a multiple of 16); values past r are masked at encode
      const int kp = k < Rpad ? k : 0;
#pragma unroll
      for (int s = 0; s < SM; s++) {
        const int ss = s < S1 ? s : S1 - 1;
        const float4* pp = reinterpret_cast<const float4*>(part + ((size_t)ss * BB + b) * Rpad + kp);
        pv[c][s][0] = pp[0];
        pv[c][s][1] = pp[1];
      }
      raw_words(g, k, r, rg[c]);
    }
  }

  __device__ __forceinline__ void encode(int S1, int r, int KT, int CW, int base, Img li) {
    const int total = BB * KT * 16, nt = blockDim.x;
#pragma unroll
    for (int c = 0; c < CPT; c++) {
      const int ci = base + c * nt + threadIdx.x;
      if (ci < total) {
        const int j8 = ci & 15;
        int b, kt;
        chunk_pos<BB>(ci >> 4, KT, b, kt);
        const int k = kt * 128 + 8 * j8;
        float gv[8], v[8];
        raw_to_f32(rg[c], gv);
        float4 a0 = pv[c][0][0], a1 = pv[c][0][1];
#pragma unroll
        for (int s = 1; s < SM; s++) {
          if (s < S1) {
            a0.x += pv[c][s][0].x; a0.y += pv[c][s][0].y; a0.z += pv[c][s][0].z; a0.w += pv[c][s][0].w;
            a1.x += pv[c][s][1].x; a1.y += pv[c][s][1].y; a1.z += pv[c][s][1].z; a1.w += pv[c][s][1].w;
          }
        }
        const float t[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = t[i] * gv[i];
        if (k + 8 > r) {  // the ragged end of the rank
#pragma unroll
          for (int i = 0; i < 8; i++) v[i] = k + i < r ? v[i] : 0.0f;
        }
        encode_chunk(v, b, kt, j8, CW, BB, li);
      }
    }
  }
};

// x copied into rows of xstride (a multiple of 8) elements, zero-padded, for
// inputs whose rows are not 16-byte aligned.
template <typename XT>
__global__ void __launch_bounds__(256) dec_xpad_kernel(const XT* __restrict__ x, int n, int B, int xstride,
                                                       XT* __restrict__ xp) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= B * xstride) return;
  const int b = i / xstride, k = i - b * xstride;
  XT z;
  __builtin_memset(&z, 0, sizeof(XT));
  xp[i] = k < n ? x[(size_t)b * n + k] : z;
}

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
template <int RM, int QWT = 16 / RM>
struct WaveWork {
  static constexpr int QW = QWT;
  u4v w[RM][QW];
  int rt0, qa, qb, nfull;
};

// Issues the wave's RM x QW quad loads (16, or 20 for the two-row-tile waves
// of tall stages), always all of them and without a branch:
// a wave with no full quad re-reads the matrix's first 1 KiB (inside the blob
// for every shape) and ignores it.  With a fixed count the compiler waits for
// the prologue's loads (issued earlier) without waiting for these.
template <int RM, int QWT>
__device__ __forceinline__ void wave_load(const uint32_t* __restrict__ P, int KT, int RT, WaveWork<RM, QWT>& ww,
                                          int lane) {
  constexpr int QW = QWT;
  ww.nfull = full_quads(KT, ww.qa, ww.qb);
  const bool any = ww.nfull > 0;
  const int last = ww.qa + ww.nfull - 1;
#pragma unroll
  for (int r = 0; r < RM; r++) {
    const int rt = min(ww.rt0 + r, RT - 1);
    const u4v* qp = reinterpret_cast<const u4v*>(P + (any ? (size_t)rt * KT * 64 : 0)) + lane;
#pragma unroll
    for (int j = 0; j < QW; j++) {
      const int q = any ? (ww.qa + j < last ? ww.qa + j : last) : 0;
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

template <int CW, int RM, int QWT>
__device__ __forceinline__ void wave_mma(const uint32_t* __restrict__ P, int KT, int RT, const WaveWork<RM, QWT>& ww,
                                         const LaneImg<CW>& im, int ktbase, int lane, v4f (&acc)[RM]) {
  constexpr int QW = QWT;
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
  const void* x;       // B rows of activations, xstride apart, 16-byte aligned
  const void* s2;      // n input scales
  int n, xstride;
  int CW, B;
  float* part;
  int Rpad;
  int red_off;         // byte offset of the reduction buffer in LDS
  int env = 1;         // envelope terms: batch row b = input row b / env under s2 row b % env
  int s2_stride = 0;   // elements between s2 rows of an envelope
};

// The work of one stage-1 workgroup: row group `rowgroup` (RM row tiles) of
// column split `split`.
template <typename XT, typename ST, int BB, int RM>
__device__ __forceinline__ void s1_body(const S1Args& a, int rowgroup, int split, uint8_t* lds) {
  constexpr int CW = 4 * BB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kt0 = split * a.KL;
  const int kt1 = min(a.KT, kt0 + a.KL);
  const int KLr = kt1 - kt0;
  const int q0 = kt0 >> 2, q1 = (kt1 + 3) >> 2;
  WaveWork<RM> ww;
  ww.rt0 = rowgroup * RM;
  const int RG = min(RM, a.RT - ww.rt0);
  ww.qa = q0 + (int)(((long long)(q1 - q0) * wave) / a.KS);
  ww.qb = q0 + (int)(((long long)(q1 - q0) * (wave + 1)) / a.KS);
  const XT* x = reinterpret_cast<const XT*>(a.x);
  const ST* s2 = reinterpret_cast<const ST*>(a.s2);
  const Img li = img_at(lds, KLr, CW);
  const int per_pass = XPass<XT, ST, BB>::CPT * blockDim.x, total = BB * KLr * 16;
  XPass<XT, ST, BB> xp;
  // the prologue's loads go out first, then the weight stream; the encoder
  // waits for the prologue's loads only
  xp.load(x, a.xstride, s2, a.n, kt0, KLr, 0, a.env, a.s2_stride);
  wave_load<RM>(a.vt, a.KT, a.RT, ww, lane);
  xp.encode(a.n, KLr, kt0, CW, 0, li);
  for (int base = per_pass; base < total; base += per_pass) {
    xp.load(x, a.xstride, s2, a.n, kt0, KLr, base, a.env, a.s2_stride);
    xp.encode(a.n, KLr, kt0, CW, base, li);
  }
  __syncthreads();
  // the tile sums of this wave's range first: they need only LDS, and the
  // products below wait for the weights anyway
  float S[4];
  const int kta = 4 * ww.qa - kt0, ktb = min(kt1, 4 * ww.qb) - kt0;
  range_sums(li.sum + (size_t)kta * BB, ktb - kta, BB, lane, S);
  const LaneImg<CW> im(li, lane);
  v4f acc[RM];
#pragma unroll
  for (int r = 0; r < RM; r++) acc[r] = v4f{0.f, 0.f, 0.f, 0.f};
  wave_mma<CW, RM>(a.vt, a.KT, a.RT, ww, im, kt0, lane, acc);
  float z[RM][4];
#pragma unroll
  for (int r = 0; r < RM; r++) finish_acc(acc[r], S, lane, z[r]);
  float* red = reinterpret_cast<float*>(lds + a.red_off);
  reduce_parts<RM>(red, z, RG, a.KS, wave, lane, BB, [&](int r, int b, float4 t) {
    *reinterpret_cast<float4*>(a.part + ((size_t)split * BB + b) * a.Rpad + (ww.rt0 + r) * 16 + 4 * (lane >> 4)) = t;
  });
}

template <typename XT, typename ST, int BB, int RM>
__global__ void __launch_bounds__(512) dec_s1_kernel(S1Args a) {
  extern __shared__ __align__(16) uint8_t lds[];
  s1_body<XT, ST, BB, RM>(a, blockIdx.x, blockIdx.y, lds);
}

// Stage 1 of up to MAX_GROUP layers that share x, in one launch: workgroup
// blockIdx.x belongs to the layer whose range of row groups holds it.
constexpr int MAX_GROUP = GROUP_MAX;
struct S1Group {
  S1Args l[MAX_GROUP];
  int wg_end[MAX_GROUP];  // cumulative row groups (unused entries: INT_MAX)
};

template <typename XT, typename ST, int BB, int RM>
__global__ void __launch_bounds__(512) dec_s1_group_kernel(S1Group g) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int bx = blockIdx.x;
  int l = 0;
#pragma unroll
  for (int i = 0; i < MAX_GROUP - 1; i++) l += bx >= g.wg_end[i] ? 1 : 0;
  const int begin = l == 0 ? 0 : g.wg_end[l - 1];
  s1_body<XT, ST, BB, RM>(g.l[l], bx - begin, blockIdx.y, lds);
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
  int s1_off;  // byte offset of the staged output scales in LDS
  int env = 1;         // envelope terms summed into one output row (row-split kernel only)
  int s1_stride = 0;   // elements between s1 rows of an envelope
};

// The work of one stage-2 workgroup: row group `rowgroup` (RM row tiles).
template <typename ST, bool FUSED, int BB, int RM, int SM>
__device__ __forceinline__ void s2_body(const S2Args& a, int rowgroup, uint8_t* lds) {
  constexpr int CW = 4 * BB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nq = (a.KT + 3) >> 2;
  WaveWork<RM> ww;
  ww.rt0 = rowgroup * RM;
  const int RG = min(RM, a.RT - ww.rt0);
  ww.qa = (int)(((long long)nq * wave) / a.KS);
  ww.qb = (int)(((long long)nq * (wave + 1)) / a.KS);
  const Img li = img_at(lds, a.KT, CW);
  if (FUSED) {
    const ST* g = reinterpret_cast<const ST*>(a.g);
    const int per_pass = TPass<ST, SM, BB>::CPT * blockDim.x, total = BB * a.KT * 16;
    TPass<ST, SM, BB> tp;
    tp.load(a.part, a.S1, a.Rpad1, g, a.r, a.KT, 0);  // prologue loads first, then the weight stream
    wave_load<RM>(a.u, a.KT, a.RT, ww, lane);
    tp.encode(a.S1, a.r, a.KT, CW, 0, li);
    for (int base = per_pass; base < total; base += per_pass) {
      tp.load(a.part, a.S1, a.Rpad1, g, a.r, a.KT, base);
      tp.encode(a.S1, a.r, a.KT, CW, base, li);
    }
  } else {
    wave_load<RM>(a.u, a.KT, a.RT, ww, lane);
    copy_image(a.img, a.KT, 0, a.KT, CW, BB, lds);
  }
  // the output scales of the workgroup's RG * 16 <= 128 rows (two per thread,
  // clamped, no branch), loaded behind the weights and staged in LDS after the
  // products, so that the epilogue makes no memory round trip
  const ST* s1 = reinterpret_cast<const ST*>(a.s1);
  const int nrows = RG * 16;
  float s1v[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int t = min((int)threadIdx.x + i * (int)blockDim.x, nrows - 1);
    s1v[i] = ld_f32(s1, min(ww.rt0 * 16 + t, a.m - 1));
  }
  __syncthreads();
  float S[4];  // before the products, as in stage 1
  const int kta = 4 * ww.qa, ktb = min(a.KT, 4 * ww.qb);
  range_sums(li.sum + (size_t)kta * BB, ktb - kta, BB, lane, S);
  const LaneImg<CW> im(li, lane);
  v4f acc[RM];
#pragma unroll
  for (int r = 0; r < RM; r++) acc[r] = v4f{0.f, 0.f, 0.f, 0.f};
  wave_mma<CW, RM>(a.u, a.KT, a.RT, ww, im, 0, lane, acc);
  float* s1l = reinterpret_cast<float*>(lds + a.s1_off);
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int t = (int)threadIdx.x + i * (int)blockDim.x;
    if (t < nrows) s1l[t] = s1v[i];
  }
  __syncthreads();
  float z[RM][4];
#pragma unroll
  for (int r = 0; r < RM; r++) finish_acc(acc[r], S, lane, z[r]);
  float* red = reinterpret_cast<float*>(lds + a.red_off);
  reduce_parts<RM>(red, z, RG, a.KS, wave, lane, BB, [&](int r, int b, float4 t) {
    const float zz[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int v = 0; v < 4; v++) {
      const int row = (ww.rt0 + r) * 16 + 4 * (lane >> 4) + v;
      if (row < a.m) {
        const float yv = s1l[r * 16 + 4 * (lane >> 4) + v] * zz[v];
        const size_t yi = (size_t)b * a.m + row;
        if (a.ydt == 0) reinterpret_cast<float*>(a.y)[yi] = yv;
        else reinterpret_cast<uint16_t*>(a.y)[yi] = f32_to_bf16(yv);
      }
    }
  });
}

// Stage 2 with the waves of a workgroup on different rows: every wave takes
// RM row tiles over the whole rank (RM x quads <= 16), so no partial results
// cross waves and the workgroup of W waves shares one encoded t' among W x RM
// row tiles (fewer workgroups, so fewer copies of t' to read and encode).
// Row group `rowgroup` = row tiles [rowgroup * W * RM, + W * RM).
template <typename ST, int BB, int RM, int SM, int QW = 16 / RM, int CPT = 2>
__device__ __forceinline__ void s2_rows_body(const S2Args& a, int rowgroup, uint8_t* lds) {
  constexpr int CW = 4 * BB;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  WaveWork<RM, QW> ww;
  ww.rt0 = (rowgroup * W + wave) * RM;
  const int RG = min(RM, a.RT - ww.rt0);  // rows of this wave (<= 0: none; its loads are clamped)
  ww.qa = 0;
  ww.qb = (a.KT + 3) >> 2;
  const Img li = img_at(lds, a.KT, CW);
  const ST* g = reinterpret_cast<const ST*>(a.g);
  const ST* s1 = reinterpret_cast<const ST*>(a.s1);
  const int per_pass = TPass<ST, SM, BB, CPT>::CPT * blockDim.x, total = BB * a.KT * 16;
  TPass<ST, SM, BB, CPT> tp;
  tp.load(a.part, a.S1, a.Rpad1, g, a.r, a.KT, 0);  // prologue loads first, then the weight stream
  wave_load<RM, QW>(a.u, a.KT, a.RT, ww, lane);
  // output scales of this lane's four rows in each row tile (one word per tile,
  // clamped into the layer; used only for rows < m)
  Raw8<ST> s1w[RM];
  const int c = lane & 15, b = c >> 2;
  int ob, sr;  // output row and envelope term of this lane's batch column
  env_split(b < BB ? b : BB - 1, a.env, ob, sr);
  const ST* s1r = s1 + (size_t)sr * a.s1_stride;
#pragma unroll
  for (int r = 0; r < RM; r++) {
    const int rt = min(ww.rt0 + r, a.RT - 1);
    const int row4 = rt * 16 + 4 * (lane >> 4);
    if constexpr (sizeof(ST) == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(s1r + row4);
      s1w[r].w[0] = uint4{v.x, v.y, 0u, 0u};
    } else {
      s1w[r].w[0] = *reinterpret_cast<const uint4*>(s1r + row4);
    }
  }
  tp.encode(a.S1, a.r, a.KT, CW, 0, li);
  for (int base = per_pass; base < total; base += per_pass) {
    tp.load(a.part, a.S1, a.Rpad1, g, a.r, a.KT, base);
    tp.encode(a.S1, a.r, a.KT, CW, base, li);
  }
  __syncthreads();
  if (RG <= 0) return;
  float S[4];
  range_sums(li.sum, a.KT, BB, lane, S);
  const LaneImg<CW> im(li, lane);
  v4f acc[RM];
#pragma unroll
  for (int r = 0; r < RM; r++) acc[r] = v4f{0.f, 0.f, 0.f, 0.f};
  wave_mma<CW, RM, QW>(a.u, a.KT, a.RT, ww, im, 0, lane, acc);
  // columns 4b hold batch row b; with an envelope the env rows of one output
  // row are summed across lanes 4 and 8 apart (columns past the batch add 0)
  const bool valid = (c & 3) == 0 && b < BB && sr == 0;
#pragma unroll
  for (int r = 0; r < RM; r++) {
    float z[4];
    finish_acc(acc[r], S, lane, z);
    if (r < RG) {
      ST sc[4];
      __builtin_memcpy(sc, s1w[r].w, sizeof(sc));
      float yv[4];
#pragma unroll
      for (int v = 0; v < 4; v++) yv[v] = ld_f32(sc, v) * z[v];
      if (a.env > 1) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
          yv[v] = b < BB ? yv[v] : 0.0f;
          yv[v] += __shfl_xor(yv[v], 4);
          if (a.env > 2) yv[v] += __shfl_xor(yv[v], 8);
        }
      }
      if (valid) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
          const int row = (ww.rt0 + r) * 16 + 4 * (lane >> 4) + v;
          if (row < a.m) {
            const size_t yi = (size_t)ob * a.m + row;
            if (a.ydt == 0) reinterpret_cast<float*>(a.y)[yi] = yv[v];
            else reinterpret_cast<uint16_t*>(a.y)[yi] = f32_to_bf16(yv[v]);
          }
        }
      }
    }
  }
}

// BIG: more than 8 waves per workgroup (launch bound 1024 threads, so at most
// 128 VGPRs: only the shapes the plan allows it for fit without spilling).
template <typename ST, int BB, int RM, int SM, bool BIG, int QW = 16 / RM, int CPT = 2>
__global__ void __launch_bounds__(BIG ? 1024 : 512) dec_s2_rows_kernel(S2Args a) {
  extern __shared__ __align__(16) uint8_t lds[];
  s2_rows_body<ST, BB, RM, SM, QW, CPT>(a, blockIdx.x, lds);
}

template <typename ST, bool FUSED, int BB, int RM, int SM>
__global__ void __launch_bounds__(512) dec_s2_kernel(S2Args a) {
  extern __shared__ __align__(16) uint8_t lds[];
  s2_body<ST, FUSED, BB, RM, SM>(a, blockIdx.x, lds);
}

// Stage 2 of a group of layers (block-diagonal: each layer its own U, t and y).
struct S2Group {
  S2Args l[MAX_GROUP];
  int wg_end[MAX_GROUP];
};

template <typename ST, int BB, int RM, int SM>
__global__ void __launch_bounds__(512) dec_s2_group_kernel(S2Group g) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int bx = blockIdx.x;
  int l = 0;
#pragma unroll
  for (int i = 0; i < MAX_GROUP - 1; i++) l += bx >= g.wg_end[i] ? 1 : 0;
  const int begin = l == 0 ? 0 : g.wg_end[l - 1];
  s2_body<ST, true, BB, RM, SM>(g.l[l], bx - begin, lds);
}

template <typename ST, int BB, int RM, int SM, bool BIG, int QW = 16 / RM, int CPT = 2>
__global__ void __launch_bounds__(BIG ? 1024 : 512) dec_s2_rows_group_kernel(S2Group g) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int bx = blockIdx.x;
  int l = 0;
#pragma unroll
  for (int i = 0; i < MAX_GROUP - 1; i++) l += bx >= g.wg_end[i] ? 1 : 0;
  const int begin = l == 0 ? 0 : g.wg_end[l - 1];
  s2_rows_body<ST, BB, RM, SM, QW, CPT>(g.l[l], bx - begin, lds);
}

}  // namespace

// ------------------------------------------------------------------ plan
// Rows per workgroup (RM, a power of two <= 8) and column-part waves (KS <= 8)
// for a stage of RT row tiles, `splits` column splits, whose waves share
// `quads` quads.  The largest RM that still gives at least `minwg` workgroups
// (every workgroup encodes its own copy of its activation range, so fewer,
// taller workgroups encode less) and whose 16-quad buffer holds RM x
// ceil(quads/KS); KS as large as the quads allow (the prologue's parallelism)
// while the whole grid stays within WAVE_BUDGET resident waves, so that it
// runs in one round.  False if no shape fits.
static bool pick_shape(int RT, int splits, int quads, int minwg, int* RM, int* KS) {
  for (int rm = 8; rm >= 1; rm /= 2) {
    const int wgs = ceil_div(RT, rm) * splits;
    if (rm > 1 && wgs < minwg) continue;
    int ks = quads < 8 ? quads : 8;
    while (ks > 1 && wgs * ks > WAVE_BUDGET) ks--;
    const int qw = ceil_div(quads, ks);
    if (rm * qw > 16) continue;
    *RM = rm;
    *KS = ks;
    return true;
  }
  return false;
}

// Stage 2 with row-split waves (see s2_rows_body) when every row tile's quads
// fit one wave's 16-quad buffer: one row tile per wave (RM = 1), W waves per
// workgroup.  Only for stages of at least MIN_ROW_WAVES row tiles.  W is sized
// so that about 160 workgroups cover the rows and so that the prologue (2
// chunks per thread per pass) takes one pass; more than 8 waves only where the
// kernel fits 128 VGPRs (S1 <= 2 partials, B = 1, 2-byte scales).
static bool pick_rows(int RT, int quads, int chunks, int S1, int B, int scale_bytes, int min_waves, int* RM,
                      int* W) {
  if (quads > 16 || RT < min_waves) return false;  // few rows: the K-split keeps more waves busy
  // Tall stages (the 70B gate+up pair: 3584 row tiles) run 16 waves per CU
  // with one row tile per wave, and every wave reads the whole t' image from
  // LDS as its B operand: 2 KiB per MFMA per wave, 1.28 MB per CU, which
  // bounds the product phase by LDS bandwidth (measured 4.2 us of the
  // stage's 14 us).  Two row tiles per wave (a 20-quad buffer, 8 waves per
  // workgroup) read each B operand once for two MFMAs.
  if (scale_bytes == 2 && S1 <= 2 && RT >= TALL_ROW_TILES && quads <= RM2_QUADS &&
      chunks <= rm2_chunks_per_thread(B) * 64 * 8) {  // the prologue in one pass
    *RM = 2;
    *W = 8;
    return true;
  }
  // one row tile per wave: twice the waves and workgroups of two row tiles
  // per wave finish the products and the per-workgroup prologue sooner
  // (measured on the 70B chain: 2.6% less time per token)
  const int rm = 1;
  int w = ceil_div(RT, rm * 160);
  const int w_pass = ceil_div(chunks, 2 * 64);
  w = w > w_pass ? w : w_pass;
  const int wmax = (S1 <= 2 && B == 1 && scale_bytes == 2) ? 16 : 8;
  w = w < 1 ? 1 : (w > wmax ? wmax : w);
  *RM = rm;
  *W = w;
  return true;
}

static DecPlan dec_plan_cap(int m, int n, int r, int B, int scale_bytes, bool force_rows, size_t cap1, size_t cap2) {
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
  int klmax = (int)((cap1 - red_bytes) / tb) / 4 * 4;
  if (klmax < 4) return p;
  {
    int rm, ks;
    if (!pick_shape(p.RT1, 1, 4, MIN_WG, &rm, &ks)) return p;  // provisional row groups for the split count
    const int rowgroups = ceil_div(p.RT1, rm);
    // every stage-2 workgroup reads all S1 partial vectors of t: keep S1 small
    // where the rank is large (the reads are S1 x r x 4 bytes per workgroup)
    const int smax = r >= 2048 ? 2 : 4;
    int s = ceil_div(TARGET_WG, rowgroups);
    s = s > smax ? smax : s;
    s = s > quads1 ? quads1 : s;
    s = s < 1 ? 1 : s;
    // stage 2 folds the partial vectors into its prologue when S1 * B <= 4
    const int s_fold = 4 / B;
    s = s > s_fold ? s_fold : s;
    const int s_lds = ceil_div(p.KT1, klmax);
    if (s < s_lds) s = s_lds;
    if (s == 3) s = B == 1 ? 4 : 2;  // stage 2 reads 1, 2 or 4 partial vectors
    if (s < s_lds) s = s_lds;
    p.KL1 = 4 * ceil_div(ceil_div(p.KT1, s), 4);
    p.S1 = ceil_div(p.KT1, p.KL1);
    if (p.S1 == 3) {  // rounding KL1 to whole quads gave 3 splits: take 2 if they fit LDS
      const int kl2 = 4 * ceil_div(ceil_div(p.KT1, 2), 4);
      if (kl2 <= klmax) {
        p.KL1 = kl2;
        p.S1 = ceil_div(p.KT1, p.KL1);
      }
    }
    if (!pick_shape(p.RT1, p.S1, ceil_div(p.KL1, 4), MIN_WG, &p.RG1, &p.KS1)) return p;
  }
  p.QM1 = ceil_div(ceil_div(p.KL1, 4), p.KS1);
  p.Rpad1 = p.RT1 * 16;
  p.red1 = align_up((size_t)p.KL1 * tb, 16);
  p.lds1 = p.red1 + red_bytes;
  // stage 2: rows = outputs, columns = rank
  p.RT2 = ceil_div(m, 16);
  p.KT2 = ceil_div(r, 128);
  const int quads2 = ceil_div(p.KT2, 4);
  if (!pick_shape(p.RT2, 1, quads2, MIN_WG, &p.RG2, &p.KS2)) return p;
  {
    // the prologue encodes B x KT2 x 16 chunks, 2 per thread per pass: prefer
    // a shape that does it in one pass, if that keeps >= 3/4 of the CUs busy
    const int chunks = B * p.KT2 * 16;
    int rm, ks;
    if (chunks > 2 * 64 * p.KS2 && pick_shape(p.RT2, 1, quads2, MIN_WG * 3 / 4, &rm, &ks) &&
        chunks <= 2 * 64 * ks) {
      p.RG2 = rm;
      p.KS2 = ks;
    }
  }
  p.QM2 = ceil_div(quads2, p.KS2);
  p.red2 = align_up((size_t)p.KT2 * tb, 16);
  p.lds2 = p.red2 + red_bytes + S1_LDS_BYTES;
  if (p.lds2 > cap2) return p;
  p.fused_mid = p.S1 * B <= 4 && p.S1 != 3;
  p.rows2 = false;
  {
    int rm, w;
    if (p.fused_mid && pick_rows(p.RT2, quads2, B * p.KT2 * 16, p.S1, B, scale_bytes, force_rows ? 1 : MIN_ROW_WAVES, &rm, &w) && p.KT2 * tb <= cap2) {
      p.rows2 = true;
      p.RG2 = rm;
      p.KS2 = w;
      p.lds2 = p.KT2 * tb;
    }
  }
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  p.off_img1 = 0;
  p.off_part = take((size_t)p.S1 * B * p.Rpad1 * 4);
  p.off_img2 = take(p.fused_mid ? 0 : (size_t)p.KT2 * tb);
  p.off_xpad = take((size_t)B * align_up(n, 8) * 4);
  p.bytes = o;
  p.ok = true;
  return p;
}

DecPlan dec_plan(int m, int n, int r, int B, int scale_bytes, bool force_rows) {
  const DecPlan p = dec_plan_cap(m, n, r, B, scale_bytes, force_rows, LDS_S1, LDS_S2);
  return p.ok ? p : dec_plan_cap(m, n, r, B, scale_bytes, force_rows, LDS_MAX, LDS_MAX);
}

template <typename ST, bool FUSED, int BB, int SM>
static void launch_s2(int RG, dim3 g, dim3 b, size_t lds, hipStream_t st, const S2Args& k) {
  switch (RG) {
    case 8: hipLaunchKernelGGL((dec_s2_kernel<ST, FUSED, BB, 8, SM>), g, b, lds, st, k); break;
    case 4: hipLaunchKernelGGL((dec_s2_kernel<ST, FUSED, BB, 4, SM>), g, b, lds, st, k); break;
    case 2: hipLaunchKernelGGL((dec_s2_kernel<ST, FUSED, BB, 2, SM>), g, b, lds, st, k); break;
    default: hipLaunchKernelGGL((dec_s2_kernel<ST, FUSED, BB, 1, SM>), g, b, lds, st, k); break;
  }
}

template <typename ST, int BB, int SM, typename K>
static void launch_rows_t(int RM, bool big, dim3 g, dim3 b, size_t lds, hipStream_t st, const K& k) {
  constexpr bool GROUP = std::is_same<K, S2Group>::value;
#define NQ_ROWS(R, BIGV)                                                                                    \
  do {                                                                                                      \
    if constexpr (GROUP) hipLaunchKernelGGL((dec_s2_rows_group_kernel<ST, BB, R, SM, BIGV>), g, b, lds, st, k); \
    else hipLaunchKernelGGL((dec_s2_rows_kernel<ST, BB, R, SM, BIGV>), g, b, lds, st, k);                   \
  } while (0)
  if constexpr (SM <= 2 && sizeof(ST) == 2) {
    if (RM == 2) {  // tall stages: two row tiles per wave, 8 waves (see pick_rows)
      constexpr int CPT = rm2_chunks_per_thread(BB);  // the prologue in one pass of 512 threads
      if constexpr (GROUP) hipLaunchKernelGGL((dec_s2_rows_group_kernel<ST, BB, 2, SM, false, RM2_QUADS, CPT>), g, b, lds, st, k);
      else hipLaunchKernelGGL((dec_s2_rows_kernel<ST, BB, 2, SM, false, RM2_QUADS, CPT>), g, b, lds, st, k);
      return;
    }
  }
  if constexpr (BB == 1 && SM <= 2 && sizeof(ST) == 2) {
    if (big) {  // the shapes with more than 8 waves (see pick_rows)
      NQ_ROWS(1, true);
      return;
    }
  }
  NQ_ROWS(1, false);  // otherwise pick_rows gives every wave one row tile
#undef NQ_ROWS
}

template <typename ST, int BB, int SM>
static void launch_s2_rows(int RM, int W, dim3 g, dim3 b, size_t lds, hipStream_t st, const S2Args& k) {
  launch_rows_t<ST, BB, SM>(RM, W > 8, g, b, lds, st, k);
}

template <typename ST, int BB, int SM>
static void launch_s2_rows_group(int RM, int W, dim3 g, dim3 b, size_t lds, hipStream_t st, const S2Group& k) {
  launch_rows_t<ST, BB, SM>(RM, W > 8, g, b, lds, st, k);
}

template <typename ST, int BB, int SM>
static void launch_s2_group(int RG, dim3 g, dim3 b, size_t lds, hipStream_t st, const S2Group& k) {
  switch (RG) {
    case 8: hipLaunchKernelGGL((dec_s2_group_kernel<ST, BB, 8, SM>), g, b, lds, st, k); break;
    case 4: hipLaunchKernelGGL((dec_s2_group_kernel<ST, BB, 4, SM>), g, b, lds, st, k); break;
    case 2: hipLaunchKernelGGL((dec_s2_group_kernel<ST, BB, 2, SM>), g, b, lds, st, k); break;
    default: hipLaunchKernelGGL((dec_s2_group_kernel<ST, BB, 1, SM>), g, b, lds, st, k); break;
  }
}

template <typename XT, typename ST, int BB>
static hipError_t dec_forward_t(const FwdArgs& a, const DecPlan& p) {
  const int sb = sizeof(ST);
  BlobLayout L = blob_layout(a.m, a.n, a.r, sb);
  const uint32_t* U = reinterpret_cast<const uint32_t*>(a.blob + L.off_u);
  const uint32_t* Vt = reinterpret_cast<const uint32_t*>(a.blob + L.off_vt);
  // an envelope of env terms runs as env x B internal batch rows (B input and
  // output rows) with the scale vectors of each term from s1_env / s2_env
  const bool envl = a.env > 1;
  const ST* s1 = reinterpret_cast<const ST*>(envl ? a.s1_env : a.blob + L.off_s1);
  const ST* g = reinterpret_cast<const ST*>(a.blob + L.off_g);
  const ST* s2 = reinterpret_cast<const ST*>(envl ? a.s2_env : a.blob + L.off_s2);
  const int xrows = a.B / a.env;
  hipStream_t st = a.stream;
  float* part = reinterpret_cast<float*>(a.ws + p.off_part);
  uint8_t* img2 = a.ws + p.off_img2;
  const bool xvec = (a.n % 8 == 0) && (reinterpret_cast<uintptr_t>(a.x) % 16 == 0);
  const void* x = a.x;
  int xstride = a.n;
  if (!xvec) {  // rows not 16-byte aligned: an aligned, zero-padded copy first
    xstride = align_up(a.n, 8);
    XT* xp = reinterpret_cast<XT*>(a.ws + p.off_xpad);
    const int tot = xrows * xstride;
    mark(a, dim3(ceil_div(tot, 256)), dim3(256));
    hipLaunchKernelGGL((dec_xpad_kernel<XT>), dim3(ceil_div(tot, 256)), dim3(256), 0, st,
                       reinterpret_cast<const XT*>(a.x), a.n, xrows, xstride, xp);
    x = xp;
  }

  S1Args k1{Vt, p.RT1, p.KT1, p.KL1, p.RG1, p.KS1, x, s2, a.n, xstride, p.CW, a.B, part, p.Rpad1, (int)p.red1};
  k1.env = a.env;
  k1.s2_stride = envl ? a.s2_env_stride : 0;
  {
    dim3 g1(ceil_div(p.RT1, p.RG1), p.S1), b1(64 * p.KS1);
    mark(a, g1, b1);
    switch (p.RG1) {
      case 8: hipLaunchKernelGGL((dec_s1_kernel<XT, ST, BB, 8>), g1, b1, p.lds1, st, k1); break;
      case 4: hipLaunchKernelGGL((dec_s1_kernel<XT, ST, BB, 4>), g1, b1, p.lds1, st, k1); break;
      case 2: hipLaunchKernelGGL((dec_s1_kernel<XT, ST, BB, 2>), g1, b1, p.lds1, st, k1); break;
      default: hipLaunchKernelGGL((dec_s1_kernel<XT, ST, BB, 1>), g1, b1, p.lds1, st, k1); break;
    }
  }
  if (!p.fused_mid) {
    const int c2 = a.B * p.KT2 * 16;
    mark(a, dim3(ceil_div(c2, 256)), dim3(256));
    hipLaunchKernelGGL((dec_mid_kernel<ST>), dim3(ceil_div(c2, 256)), dim3(256), 0, st, part, p.S1, p.Rpad1, g,
                       a.r, a.B, p.KT2, p.CW, img2);
  }
  S2Args k2{U, p.RT2, p.KT2, p.RG2, p.KS2, p.fused_mid ? nullptr : img2, part, p.S1, p.Rpad1, a.r, g, p.CW, a.B,
            s1, a.scale_dtype, a.y, a.y_dtype == 0 ? 0 : 2, a.m, (int)p.red2, (int)(p.lds2 - S1_LDS_BYTES)};
  k2.env = a.env;
  k2.s1_stride = envl ? a.s1_env_stride : 0;
  dim3 g2(ceil_div(p.RT2, p.RG2 * (p.rows2 ? p.KS2 : 1))), b2(64 * p.KS2);
  mark(a, g2, b2);
  if (p.rows2) {
    if (p.S1 == 1) launch_s2_rows<ST, BB, 1>(p.RG2, p.KS2, g2, b2, p.lds2, st, k2);
    else if (p.S1 == 2) launch_s2_rows<ST, BB, (BB <= 2 ? 2 : 1)>(p.RG2, p.KS2, g2, b2, p.lds2, st, k2);
    else launch_s2_rows<ST, BB, (BB == 1 ? 4 : 1)>(p.RG2, p.KS2, g2, b2, p.lds2, st, k2);
  } else if (p.fused_mid) {
    // splits read by the prologue: 1, 2 or 4 (S1 * B <= 4)
    if (p.S1 == 1) launch_s2<ST, true, BB, 1>(p.RG2, g2, b2, p.lds2, st, k2);
    else if (p.S1 == 2) launch_s2<ST, true, BB, (BB <= 2 ? 2 : 1)>(p.RG2, g2, b2, p.lds2, st, k2);
    else launch_s2<ST, true, BB, (BB == 1 ? 4 : 1)>(p.RG2, g2, b2, p.lds2, st, k2);
  } else {
    launch_s2<ST, false, BB, 1>(p.RG2, g2, b2, p.lds2, st, k2);
  }
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

static GroupPlan group_plan_cap(const int* m, const int* r, int L, int n, int B, int scale_bytes, size_t cap1,
                                size_t cap2) {
  GroupPlan p{};
  p.ok = false;
  if (L < 1 || L > GROUP_MAX || B < 1 || B > DEC_MAX_B) return p;
  p.L = L;
  p.B = B;
  p.CW = B * P;
  const size_t tb = img_tile_bytes(p.CW, B);
  const size_t red_bytes = (size_t)8 * 8 * 16 * 16;
  p.KT1 = ceil_div(n, 128);
  int rt1_sum = 0, rt2_sum = 0, rmax = 0, kt2max = 0;
  for (int l = 0; l < L; l++) {
    p.RT1[l] = ceil_div(r[l], 16);
    p.Rpad1[l] = p.RT1[l] * 16;
    p.RT2[l] = ceil_div(m[l], 16);
    p.KT2[l] = ceil_div(r[l], 128);
    rt1_sum += p.RT1[l];
    rt2_sum += p.RT2[l];
    rmax = r[l] > rmax ? r[l] : rmax;
    kt2max = p.KT2[l] > kt2max ? p.KT2[l] : kt2max;
  }
  // stage 1: the rules of the single-layer plan, on the layers' rows together
  const int quads1 = ceil_div(p.KT1, 4);
  const int klmax = (int)((cap1 - red_bytes) / tb) / 4 * 4;
  if (klmax < 4) return p;
  {
    int rm, ks;
    if (!pick_shape(rt1_sum, 1, 4, MIN_WG, &rm, &ks)) return p;
    const int rowgroups = ceil_div(rt1_sum, rm);
    const int smax = rmax >= 2048 ? 2 : 4;
    int s = ceil_div(TARGET_WG, rowgroups);
    s = s > smax ? smax : s;
    s = s > quads1 ? quads1 : s;
    s = s > 4 / B ? 4 / B : s;  // stage 2 folds the S1 x B partial vectors (<= 4) into its prologue
    s = s < 1 ? 1 : s;
    const int s_lds = ceil_div(p.KT1, klmax);
    if (s < s_lds) s = s_lds;
    if (s == 3) s = 4;
    p.KL1 = 4 * ceil_div(ceil_div(p.KT1, s), 4);
    p.S1 = ceil_div(p.KT1, p.KL1);
    if (p.S1 == 3) {  // rounding KL1 to whole quads gave 3 splits: take 2 if they fit LDS
      const int kl2 = 4 * ceil_div(ceil_div(p.KT1, 2), 4);
      if (kl2 <= klmax) {
        p.KL1 = kl2;
        p.S1 = ceil_div(p.KT1, p.KL1);
      }
    }
    if (!pick_shape(rt1_sum, p.S1, ceil_div(p.KL1, 4), MIN_WG, &p.RG1, &p.KS1)) return p;
  }
  if (p.S1 * B > 4 || p.S1 == 3) return p;  // stage 2 folds the partial sums in its prologue
  p.red1 = align_up((size_t)p.KL1 * tb, 16);
  p.lds1 = p.red1 + red_bytes;
  // stage 2: one shape for all layers, sized for the longest rank
  const int quads2 = ceil_div(kt2max, 4);
  if (!pick_shape(rt2_sum, 1, quads2, MIN_WG, &p.RG2, &p.KS2)) return p;
  {
    const int chunks = B * kt2max * 16;
    int rm, ks;
    if (chunks > 2 * 64 * p.KS2 && pick_shape(rt2_sum, 1, quads2, MIN_WG * 3 / 4, &rm, &ks) &&
        chunks <= 2 * 64 * ks) {
      p.RG2 = rm;
      p.KS2 = ks;
    }
  }
  p.red2 = align_up((size_t)kt2max * tb, 16);
  p.lds2 = p.red2 + red_bytes + S1_LDS_BYTES;
  if (p.lds2 > cap2) return p;
  p.rows2 = false;
  {
    int rm, w;
    if (pick_rows(rt2_sum, quads2, B * kt2max * 16, p.S1, B, scale_bytes, MIN_ROW_WAVES, &rm, &w)) {
      p.rows2 = true;
      p.RG2 = rm;
      p.KS2 = w;
      p.lds2 = kt2max * tb;
    }
  }
  const int rows_per_wg2 = p.rows2 ? p.RG2 * p.KS2 : p.RG2;
  int e1 = 0, e2 = 0;
  for (int l = 0; l < GROUP_MAX; l++) {
    if (l < L) {
      e1 += ceil_div(p.RT1[l], p.RG1);
      e2 += ceil_div(p.RT2[l], rows_per_wg2);
      p.wg1_end[l] = e1;
      p.wg2_end[l] = e2;
    } else {
      p.wg1_end[l] = INT_MAX;
      p.wg2_end[l] = INT_MAX;
    }
  }
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  for (int l = 0; l < L; l++) p.off_part[l] = take((size_t)p.S1 * B * p.Rpad1[l] * 4);
  p.off_xpad = take((size_t)B * align_up(n, 8) * 4);
  p.bytes = o;
  p.ok = true;
  return p;
}

GroupPlan group_plan(const int* m, const int* r, int L, int n, int B, int scale_bytes) {
  const GroupPlan p = group_plan_cap(m, r, L, n, B, scale_bytes, LDS_S1, LDS_S2);
  return p.ok ? p : group_plan_cap(m, r, L, n, B, scale_bytes, LDS_MAX, LDS_MAX);
}

template <typename XT, typename ST, int BB>
static hipError_t group_forward_t(const GroupArgs& a, const GroupPlan& p) {
  hipStream_t st = a.stream;
  FwdArgs fa{};  // for the timing marks only
  fa.stream = st;
  fa.marks = a.marks;
  const bool xvec = (a.n % 8 == 0) && (reinterpret_cast<uintptr_t>(a.x) % 16 == 0);
  const void* x = a.x;
  int xstride = a.n;
  if (!xvec) {
    xstride = align_up(a.n, 8);
    XT* xp = reinterpret_cast<XT*>(a.ws + p.off_xpad);
    const int tot = a.B * xstride;
    mark(fa, dim3(ceil_div(tot, 256)), dim3(256));
    hipLaunchKernelGGL((dec_xpad_kernel<XT>), dim3(ceil_div(tot, 256)), dim3(256), 0, st,
                       reinterpret_cast<const XT*>(a.x), a.n, a.B, xstride, xp);
    x = xp;
  }
  S1Group g1{};
  S2Group g2{};
  const int sb = sizeof(ST);
  for (int l = 0; l < MAX_GROUP; l++) {
    g1.wg_end[l] = p.wg1_end[l];
    g2.wg_end[l] = p.wg2_end[l];
    if (l >= a.L) continue;
    const BlobLayout L = blob_layout(a.m[l], a.n, a.r[l], sb);
    const uint8_t* blob = a.blob[l];
    float* part = reinterpret_cast<float*>(a.ws + p.off_part[l]);
    g1.l[l] = S1Args{reinterpret_cast<const uint32_t*>(blob + L.off_vt), p.RT1[l], p.KT1, p.KL1, p.RG1, p.KS1, x,
                     blob + L.off_s2, a.n, xstride, p.CW, a.B, part, p.Rpad1[l], (int)p.red1};
    g2.l[l] = S2Args{reinterpret_cast<const uint32_t*>(blob + L.off_u), p.RT2[l], p.KT2[l], p.RG2, p.KS2, nullptr,
                     part, p.S1, p.Rpad1[l], a.r[l], blob + L.off_g, p.CW, a.B, blob + L.off_s1, a.scale_dtype,
                     a.y[l], a.y_dtype == 0 ? 0 : 2, a.m[l], (int)p.red2, (int)(p.lds2 - S1_LDS_BYTES)};
  }
  const dim3 grid1(p.wg1_end[a.L - 1], p.S1), b1(64 * p.KS1);
  mark(fa, grid1, b1);
  switch (p.RG1) {
    case 8: hipLaunchKernelGGL((dec_s1_group_kernel<XT, ST, BB, 8>), grid1, b1, p.lds1, st, g1); break;
    case 4: hipLaunchKernelGGL((dec_s1_group_kernel<XT, ST, BB, 4>), grid1, b1, p.lds1, st, g1); break;
    case 2: hipLaunchKernelGGL((dec_s1_group_kernel<XT, ST, BB, 2>), grid1, b1, p.lds1, st, g1); break;
    default: hipLaunchKernelGGL((dec_s1_group_kernel<XT, ST, BB, 1>), grid1, b1, p.lds1, st, g1); break;
  }
  const dim3 grid2(p.wg2_end[a.L - 1]), b2(64 * p.KS2);
  mark(fa, grid2, b2);
  // splits folded by the prologue: 1, 2 or 4 (S1 * B <= 4)
  if (p.rows2) {
    if (p.S1 == 1) launch_s2_rows_group<ST, BB, 1>(p.RG2, p.KS2, grid2, b2, p.lds2, st, g2);
    else if (p.S1 == 2) launch_s2_rows_group<ST, BB, (BB <= 2 ? 2 : 1)>(p.RG2, p.KS2, grid2, b2, p.lds2, st, g2);
    else launch_s2_rows_group<ST, BB, (BB == 1 ? 4 : 1)>(p.RG2, p.KS2, grid2, b2, p.lds2, st, g2);
  } else if (p.S1 == 1) launch_s2_group<ST, BB, 1>(p.RG2, grid2, b2, p.lds2, st, g2);
  else if (p.S1 == 2) launch_s2_group<ST, BB, (BB <= 2 ? 2 : 1)>(p.RG2, grid2, b2, p.lds2, st, g2);
  else launch_s2_group<ST, BB, (BB == 1 ? 4 : 1)>(p.RG2, grid2, b2, p.lds2, st, g2);
  mark(fa);
  return hipGetLastError();
}

template <typename XT, typename ST>
static hipError_t group_forward_b(const GroupArgs& a, const GroupPlan& p) {
  switch (a.B) {
    case 1: return group_forward_t<XT, ST, 1>(a, p);
    case 2: return group_forward_t<XT, ST, 2>(a, p);
    case 3: return group_forward_t<XT, ST, 3>(a, p);
    default: return group_forward_t<XT, ST, 4>(a, p);
  }
}

hipError_t group_forward(const GroupArgs& a, const GroupPlan& p) {
  if (a.x_dtype == 2) {
    return a.scale_dtype == 1 ? group_forward_b<uint16_t, _Float16>(a, p) : group_forward_b<uint16_t, float>(a, p);
  }
  return a.scale_dtype == 1 ? group_forward_b<float, _Float16>(a, p) : group_forward_b<float, float>(a, p);
}

hipError_t dec_forward(const FwdArgs& a, const DecPlan& p) {
  if (a.x_dtype == 2) {
    return a.scale_dtype == 1 ? dec_forward_b<uint16_t, _Float16>(a, p) : dec_forward_b<uint16_t, float>(a, p);
  }
  return a.scale_dtype == 1 ? dec_forward_b<float, _Float16>(a, p) : dec_forward_b<float, float>(a, p);
}

}  // namespace nq
