// Shared definitions of libnq: the packed sign-bit layout, the blob layout, the
// fp8 "piece" encoding of activations, and small device helpers.
//
// The operation is y = s1 * (U (g * (V^T (s2 * x)))) with U, V sign matrices
// (NanoQuant pages: hardwired.dev article, section "Jak NanoQuant funguje";
// rapidrecap.app summary, "Quantization Technique").  Both sign-matrix products
// are the same primitive: out[row] = sum_col P[row][col] * v[col], P in {-1,+1},
// evaluated as 2 * sum_{bit=1} v - sum v.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace nq {

// ---------------------------------------------------------------------------
// Packed sign-bit layout ("tile layout").
//
// A sign matrix P with R rows (output index) and C columns (contraction index)
// is stored as tiles of 16 rows x 128 columns; one tile is 64 lanes x 32 bits,
// which is exactly one wavefront's fp4 A operand of the 16x16x128 scaled MFMA
// when the bits are spread over nibbles (see the gemv kernels):
//   lane L of tile (rt, kt) holds row 16*rt + (L & 15) and the 32 columns
//   128*kt + 32*(L >> 4) + [0, 32);
//   bit (4*p + j) of that 32-bit word is column 128*kt + 32*(L >> 4) + 8*j + p,
//   p in [0, 8), j in [0, 4); bit value 1 means +1, 0 means -1.
// Row tiles are stored one after the other; inside a row tile, column tiles are
// grouped by four ("quads") and a quad stores its 4 (or, for the last quad,
// f < 4) words per lane contiguously, so that one 16-byte load per lane reads
// four column tiles of one row tile (1 KiB per wavefront, eight full 128-byte
// lines).  Bits of rows >= R or columns >= C are 0.
// ---------------------------------------------------------------------------
constexpr int TILE_ROWS = 16;
constexpr int TILE_COLS = 128;
constexpr int TILE_WORDS = 64;  // 32-bit words per tile

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct PackedDims {
  int R, C;    // logical rows / columns
  int RT, KT;  // row tiles, column tiles
  __host__ __device__ size_t words() const { return (size_t)RT * KT * TILE_WORDS; }
  __host__ __device__ size_t bytes() const { return words() * 4; }
};

__host__ __device__ inline PackedDims packed_dims(int R, int C) {
  PackedDims d;
  d.R = R;
  d.C = C;
  d.RT = ceil_div(R, TILE_ROWS);
  d.KT = ceil_div(C, TILE_COLS);
  return d;
}

// Index (in 32-bit words) of lane L's word of tile (rt, kt).
__host__ __device__ inline size_t packed_word_index(int rt, int kt, int lane, int KT) {
  int q = kt >> 2;
  int f = KT - 4 * q;
  f = f < 4 ? f : 4;
  return (size_t)rt * KT * TILE_WORDS + (size_t)q * 4 * TILE_WORDS + (size_t)lane * f + (kt & 3);
}

// Column offset (inside the 128-column tile) of bit b of lane L's word.
__host__ __device__ inline int packed_bit_col(int lane, int b) {
  return 32 * (lane >> 4) + 8 * (b & 3) + (b >> 2);
}

// ---------------------------------------------------------------------------
// Blob layout: header | packed U (rows = m, cols = r) | packed V^T (rows = r,
// cols = n) | s1 (m) | g (r) | s2 (n), each section 256-byte aligned.
// ---------------------------------------------------------------------------
constexpr uint32_t BLOB_MAGIC = 0x3142514eu;  // "NQB1"
constexpr uint32_t BLOB_VERSION = 1;
constexpr size_t HEADER_BYTES = 256;

struct BlobHeader {
  uint32_t magic, version;
  int32_t m, n, r, scale_dtype;
  int32_t bad_sign_count;  // written by the pack kernels: entries that are not +-1
  int32_t reserved0;
  uint64_t off_u, off_vt, off_s1, off_g, off_s2, total;
};

struct BlobLayout {
  PackedDims u, vt;
  size_t off_u, off_vt, off_s1, off_g, off_s2, total;
  int scale_bytes;
};

__host__ __device__ inline BlobLayout blob_layout(int m, int n, int r, int scale_bytes) {
  BlobLayout b;
  b.scale_bytes = scale_bytes;
  b.u = packed_dims(m, r);
  b.vt = packed_dims(r, n);
  b.off_u = HEADER_BYTES;
  b.off_vt = align_up(b.off_u + b.u.bytes(), 256);
  b.off_s1 = align_up(b.off_vt + b.vt.bytes(), 256);
  b.off_g = align_up(b.off_s1 + (size_t)m * scale_bytes, 256);
  b.off_s2 = align_up(b.off_g + (size_t)r * scale_bytes, 256);
  b.total = align_up(b.off_s2 + (size_t)n * scale_bytes, 256);
  return b;
}

// ---------------------------------------------------------------------------
// Activation operand of the 16x16x128 scaled MFMA ("B image").
//
// A vector v of length C (KT column tiles) is written, per column tile, as the
// exact register image of the fp8 B operand.  Each value is split into P fp8
// E4M3 "pieces" v ~= sum_q piece_q * 2^e_q, each with its own power-of-two
// scale per block of 32 columns (the MFMA's e8m0 block scale).  Batch row b and
// piece q occupy MFMA column c = (b % TPG) * P + q of column group G = b / TPG,
// TPG = 16 / P rows per group.
//
// Operand geometry of v_mfma_scale_f32_16x16x128_f8f6f4 (checked on gfx950):
//   fp8 operand: lane L holds column L & 15 and the 32 K values
//       16*(L>>4) + [0,16) in bytes 0..15 and 64 + 16*(L>>4) + [0,16) in bytes 16..31;
//   fp4 operand: lane L holds row L & 15 and K values 32*(L>>4) + [0,32),
//       value i in nibble i%8 (low nibble first) of dword i/8;
//   block scale of (row or column c, K block kb = K/32) is byte 0 of lane c + 16*kb;
//   result: lane L holds D[4*(L>>4) + v][L & 15], v in [0,4).
// Because the sign bits are spread over fp4 nibbles by bit-plane (plane j of the
// packed word becomes dword j with nibble value 0.5, 1, 2, 2 for j = 0..3; see
// the gemv kernel), each value is divided by that plane factor before it is
// split: c_j = {0.5, 1, 2, 2} for j = (K % 32) / 8.
//
// Image layout, per column tile kt and column group G (NG groups):
//   data  : 64 lanes x 32 bytes  at xq  + ((kt*NG + G)*64 + L)*32
//   scale : 64 lanes x 4 bytes   at xs  + ((kt*NG + G)*64 + L)   (e8m0 in byte 0)
//   sum   : B floats             at xsum + b*KT + kt  (sum of the represented values)
// Lanes whose column is unused are never read.
// ---------------------------------------------------------------------------
constexpr int IMG_LANE_BYTES = 32;
constexpr int IMG_TILE_BYTES = 64 * IMG_LANE_BYTES;  // per (kt, G)

__host__ __device__ inline int pieces_for_batch(int B) { return B <= 4 ? 4 : 3; }
__host__ __device__ inline int rows_per_group(int P) { return 16 / P; }
__host__ __device__ inline int groups_for_batch(int B) {
  int P = pieces_for_batch(B);
  return ceil_div(B, rows_per_group(P));
}

// Lane and byte of the fp8 image that hold K offset k (0..127) for MFMA column c.
__host__ __device__ inline void img_slot(int k, int c, int* lane, int* byte) {
  int G, i;
  if (k < 64) {
    G = k >> 4;
    i = k & 15;
  } else {
    G = (k - 64) >> 4;
    i = 16 + ((k - 64) & 15);
  }
  *lane = c + 16 * G;
  *byte = i;
}

// Plane factor c_j by which the fp4 operand scales the sign bit of column k.
__host__ __device__ inline float plane_factor(int k) {
  int j = (k & 31) >> 3;
  return j == 0 ? 0.5f : (j == 1 ? 1.0f : 2.0f);
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ inline int floor_log2(float a) {  // a > 0, finite
  return __builtin_amdgcn_frexp_expf(a) - 1;
}

// Round a (|a| < 512) to the nearest fp8 E4M3 value, ties to even.  Exact
// arithmetic: the quantum is a power of two.
__device__ inline float round_e4m3(float a) {
  float ax = fabsf(a);
  if (!(ax > 0.0f)) return 0.0f;
  int E = __builtin_amdgcn_frexp_expf(ax) - 1;
  int qe = (E < -6 ? -6 : E) - 3;
  float r = rintf(ldexpf(ax, -qe));
  return copysignf(ldexpf(r, qe), a);
}

// Bit pattern of an fp8 E4M3 value that is exactly representable and finite.
__device__ inline uint32_t encode_e4m3(float p) {
  uint32_t s = p < 0.0f ? 0x80u : 0u;
  float ap = fabsf(p);
  if (!(ap > 0.0f)) return 0u;
  int E = __builtin_amdgcn_frexp_expf(ap) - 1;
  if (E < -6) return s | (uint32_t)(int)ldexpf(ap, 9);
  uint32_t man = (uint32_t)(int)ldexpf(ap, 3 - E) - 8u;
  return s | ((uint32_t)(E + 7) << 3) | man;
}

template <typename T> __device__ inline float to_f32(T v);
template <> __device__ inline float to_f32<float>(float v) { return v; }
template <> __device__ inline float to_f32<_Float16>(_Float16 v) { return (float)v; }
template <> __device__ inline float to_f32<uint16_t>(uint16_t v) {  // bf16 bits
  return __uint_as_float((uint32_t)v << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace nq
