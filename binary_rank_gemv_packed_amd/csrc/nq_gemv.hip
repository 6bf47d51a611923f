// Batch 1..16 forward ("gemv" path): sign bits fed to the gfx950 scaled MFMA as
// fp4 operands, activations as fp8 pieces with e8m0 block scales.
//
// Each sign-matrix product out[row] = sum_col P[row][col] v[col] is evaluated as
//     2 * sum_{col: bit = 1} v[col] - sum_col v[col]
// (the packed bit is 1 for +1 and 0 for -1).  The masked sum is what the MFMA
// computes when the A operand holds the bit itself as an fp4 number: plane j of
// a packed 32-bit word, (word & (0x11111111 << j)), is eight fp4 nibbles whose
// value is 0 or 2^(j-1) -- one AND turns eight sign bits into eight MFMA
// operands.  Plane 3 would land on the fp4 sign bit, so it is shifted down one
// place first (nibble value 0 or 2).  The activation side carries the inverse
// plane factor, so the MFMA sum is exactly sum_{bit=1} v.
//
// Per forward: prep (s2 * x -> image) ; stage 1 (t = V^T image, split over
// column ranges) ; mid (t' = g * sum of splits -> image) ; stage 2 (y = s1 * (U
// image), optionally split + finish).
#include "nq_common.h"
#include "nq_internal.h"

namespace nq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int TARGET_WAVES = 2048;  // 256 CUs x 8 waves
constexpr int NO_SPLIT_ROW_TILES = 1024;

StagePlan stage_plan(int R, int C) {
  StagePlan s;
  s.RT = ceil_div(R, TILE_ROWS);
  s.KT = ceil_div(C, TILE_COLS);
  int quads = ceil_div(s.KT, 4);
  int want = s.RT >= NO_SPLIT_ROW_TILES ? 1 : ceil_div(TARGET_WAVES, s.RT);
  if (want < 1) want = 1;
  if (want > quads) want = quads;
  int qps = ceil_div(quads, want);
  s.kt_per_split = 4 * qps;
  s.nsplit = ceil_div(s.KT, s.kt_per_split);
  return s;
}

GemvPlan gemv_plan(int m, int n, int r, int B) {
  GemvPlan p;
  p.P = pieces_for_batch(B);
  p.TPG = rows_per_group(p.P);
  p.NG = ceil_div(B, p.TPG);
  p.s1 = stage_plan(r, n);  // V^T: rows = rank, columns = inputs
  p.s2 = stage_plan(m, r);  // U:   rows = outputs, columns = rank
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  p.off_img1 = take((size_t)p.s1.KT * p.NG * IMG_TILE_BYTES);
  p.off_xs1 = take((size_t)p.s1.KT * p.NG * 64 * 4);
  p.off_sum1 = take((size_t)B * p.s1.KT * 4);
  p.off_part1 = take((size_t)p.s1.nsplit * B * p.s1.RT * TILE_ROWS * 4);
  p.off_img2 = take((size_t)p.s2.KT * p.NG * IMG_TILE_BYTES);
  p.off_xs2 = take((size_t)p.s2.KT * p.NG * 64 * 4);
  p.off_sum2 = take((size_t)B * p.s2.KT * 4);
  p.off_part2 = take(p.s2.nsplit > 1 ? (size_t)p.s2.nsplit * B * p.s2.RT * TILE_ROWS * 4 : 0);
  p.bytes = o;
  return p;
}

// ------------------------------------------------------------------ images
struct ImgOut {
  uint8_t* xq;
  uint32_t* xs;
  float* xsum;
  int P, TPG, NG, KT;
};

__device__ inline float block128_sum(float s, float* red) {
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  float t = red[0] + red[1];
  __syncthreads();
  return t;
}

// Called by all 128 threads of a block, thread k holding value v of column
// 128*kt + k of batch row b.  Splits v (divided by its plane factor) into P
// fp8 pieces with one power-of-two scale per block of 32 columns and writes
// them into the MFMA image; writes the sum of the represented values.
__device__ void build_tile_image(float v, int kt, int b, const ImgOut& o, float* red) {
  const int k = threadIdx.x;
  const int G = b / o.TPG, tb = b % o.TPG;
  const float c = plane_factor(k);
  // a non-finite value gets no pieces; it reaches the output through the sum term
  const bool fin = __builtin_isfinite(v);
  float res = fin ? v / c : 0.0f;
  float recon = 0.0f;
  const size_t tbase = (size_t)(kt * o.NG + G) * 64;
  for (int q = 0; q < o.P; q++) {
    float M = fabsf(res);
    for (int s = 16; s > 0; s >>= 1) M = fmaxf(M, __shfl_xor(M, s));  // max over the 32-column block
    int e = 0;
    if (M > 0.0f) {
      e = floor_log2(M) - 7;  // block max lands in [128, 256)
      e = e < -127 ? -127 : e;
    }
    float p = round_e4m3(ldexpf(res, -e));
    float pv = ldexpf(p, e);
    res -= pv;
    recon += pv;
    int col = tb * o.P + q, lane, byte;
    img_slot(k, col, &lane, &byte);
    o.xq[(tbase + lane) * IMG_LANE_BYTES + byte] = (uint8_t)encode_e4m3(p);
    if ((k & 31) == 0) o.xs[tbase + col + 16 * (k >> 5)] = (uint32_t)(e + 127);
  }
  float s = block128_sum(fin ? recon * c : v, red);
  if (k == 0) o.xsum[(size_t)b * o.KT + kt] = s;
}

// Image of v = s2 * x, one block per column tile.
template <typename XT, typename ST>
__global__ void __launch_bounds__(128) prep_x_kernel(const XT* __restrict__ x, const ST* __restrict__ s2, int n,
                                                     int B, ImgOut o) {
  __shared__ float red[2];
  const int kt = blockIdx.x;
  const int col = kt * TILE_COLS + threadIdx.x;
  const float sv = col < n ? to_f32(s2[col]) : 0.0f;
  for (int b = 0; b < B; b++) {
    float v = col < n ? to_f32(x[(size_t)b * n + col]) * sv : 0.0f;
    build_tile_image(v, kt, b, o, red);
  }
}

// Image of t' = g * (sum over splits of the stage-1 partial results).
template <typename ST>
__global__ void __launch_bounds__(128) mid_kernel(const float* __restrict__ part, int nsplit, int Rpad,
                                                  const ST* __restrict__ g, int r, int B, ImgOut o) {
  __shared__ float red[2];
  const int kt = blockIdx.x;
  const int row = kt * TILE_COLS + threadIdx.x;
  const float gv = row < r ? to_f32(g[row]) : 0.0f;
  for (int b = 0; b < B; b++) {
    float t = 0.0f;
    if (row < r)
      for (int s = 0; s < nsplit; s++) t += part[((size_t)s * B + b) * Rpad + row];
    build_tile_image(t * gv, kt, b, o, red);
  }
}

// ------------------------------------------------------------------ MFMA stage
enum { EPI_PART = 0, EPI_OUT = 1 };

struct StageK {
  const uint32_t* packed;
  int R, RT, KT, nsplit, kt_per_split;
  const uint8_t* xq;
  const uint32_t* xs;
  const float* xsum;
  int P, TPG, NG, B;
  float* part;  // EPI_PART: part[(split*B + b)*Rpad + row]
  int Rpad;
  void* y;  // EPI_OUT: y[b*R + row] = s1[row] * z
  const void* s1;
  int ydt, sdt;
};

template <int NGC, int EPI>
__global__ void __launch_bounds__(256) stage_kernel(StageK a) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.RT * a.nsplit) return;
  const int rt = wid % a.RT, split = wid / a.RT;
  const int kt0 = split * a.kt_per_split;
  const int kt1 = min(a.KT, kt0 + a.kt_per_split);
  const int c = lane & 15;

  bool act[NGC];
#pragma unroll
  for (int G = 0; G < NGC; G++) {
    int rows = min(a.TPG, a.B - G * a.TPG);
    act[G] = G < a.NG && c < rows * a.P;
  }
  v4f acc[NGC];
#pragma unroll
  for (int G = 0; G < NGC; G++) acc[G] = v4f{0.f, 0.f, 0.f, 0.f};

  const uint32_t* rowbase = a.packed + (size_t)rt * a.KT * TILE_WORDS;
  for (int q = kt0 >> 2; 4 * q < kt1; q++) {
    const int f = min(4, a.KT - 4 * q);
    const uint32_t* qb = rowbase + (size_t)q * 4 * TILE_WORDS;
    uint32_t w[4];
    if (f == 4) {
      uint4 t = *reinterpret_cast<const uint4*>(qb + lane * 4);
      w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++) w[i] = i < f ? qb[lane * f + i] : 0u;
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if (i < f) {
        const int kt = 4 * q + i;
        const uint32_t word = w[i];
        v8i A = {(int)(word & 0x11111111u), (int)(word & 0x22222222u), (int)(word & 0x44444444u),
                 (int)((word >> 1) & 0x44444444u), 0, 0, 0, 0};
#pragma unroll
        for (int G = 0; G < NGC; G++) {
          if (G < a.NG) {
            const size_t tb = (size_t)(kt * a.NG + G) * 64 + lane;
            v8i Bv = {0, 0, 0, 0, 0, 0, 0, 0};
            int sb = 127;
            if (act[G]) {
              Bv = *reinterpret_cast<const v8i*>(a.xq + tb * IMG_LANE_BYTES);
              sb = (int)a.xs[tb];
            }
            acc[G] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bv, acc[G], 4, 0, 0, 127, 0, sb);
          }
        }
      }
    }
  }

  // Epilogue: lane c = tb*P + q holds piece q of batch row G*TPG + tb; rows
  // 4*(lane>>4) + v of the tile.
  const int tbi = c / a.P, qi = c % a.P;
#pragma unroll
  for (int G = 0; G < NGC; G++) {
    if (G >= a.NG) break;
    const int b = G * a.TPG + tbi;
    const bool valid = qi == 0 && tbi < a.TPG && b < a.B;
    float S = 0.0f;
    if (valid)
      for (int kt = kt0; kt < kt1; kt++) S += a.xsum[(size_t)b * a.KT + kt];
    float z[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
      float t = acc[G][v];
      float s = t;
#pragma unroll
      for (int dq = 1; dq < 4; dq++) {
        float o = __shfl_down(t, dq);
        if (dq < a.P) s += o;
      }
      z[v] = 2.0f * s - S;
    }
    if (valid) {
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int row = rt * TILE_ROWS + 4 * (lane >> 4) + v;
        if (row < a.R) {
          if (EPI == EPI_PART) {
            a.part[((size_t)split * a.B + b) * a.Rpad + row] = z[v];
          } else {
            float sc = a.sdt == 0 ? reinterpret_cast<const float*>(a.s1)[row]
                                  : (float)reinterpret_cast<const _Float16*>(a.s1)[row];
            float yv = sc * z[v];
            size_t yi = (size_t)b * a.R + row;
            if (a.ydt == 0) reinterpret_cast<float*>(a.y)[yi] = yv;
            else reinterpret_cast<uint16_t*>(a.y)[yi] = f32_to_bf16(yv);
          }
        }
      }
    }
  }
}

// y = s1 * (sum of stage-2 splits), one thread per output.
__global__ void __launch_bounds__(256) finish_kernel(const float* __restrict__ part, int nsplit, int Rpad, int m,
                                                     int B, const void* s1, int sdt, void* y, int ydt) {
  long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)B * m) return;
  int b = (int)(idx / m), i = (int)(idx % m);
  float z = 0.0f;
  for (int s = 0; s < nsplit; s++) z += part[((size_t)s * B + b) * Rpad + i];
  float sc = sdt == 0 ? reinterpret_cast<const float*>(s1)[i] : (float)reinterpret_cast<const _Float16*>(s1)[i];
  float yv = sc * z;
  if (ydt == 0) reinterpret_cast<float*>(y)[idx] = yv;
  else reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16(yv);
}

void launch_finish(const float* part, int nsplit, int Rpad, int m, int B, const void* s1, int sdt, void* y, int ydt,
                   hipStream_t st) {
  long long total = (long long)B * m;
  hipLaunchKernelGGL(finish_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, part, nsplit, Rpad, m, B,
                     s1, sdt, y, ydt);
}

// ------------------------------------------------------------------ host side
template <int EPI>
static void launch_stage(const StageK& k, hipStream_t s) {
  int waves = k.RT * k.nsplit;
  dim3 grid(ceil_div(waves, 4)), block(256);
  switch (k.NG) {
    case 1: hipLaunchKernelGGL((stage_kernel<1, EPI>), grid, block, 0, s, k); break;
    case 2: hipLaunchKernelGGL((stage_kernel<2, EPI>), grid, block, 0, s, k); break;
    case 3: hipLaunchKernelGGL((stage_kernel<3, EPI>), grid, block, 0, s, k); break;
    default: hipLaunchKernelGGL((stage_kernel<4, EPI>), grid, block, 0, s, k); break;
  }
}

hipError_t gemv_forward(const FwdArgs& a, const GemvPlan& p) {
  const int sb = a.scale_dtype == 0 ? 4 : 2;
  BlobLayout L = blob_layout(a.m, a.n, a.r, sb);
  const uint32_t* U = reinterpret_cast<const uint32_t*>(a.blob + L.off_u);
  const uint32_t* Vt = reinterpret_cast<const uint32_t*>(a.blob + L.off_vt);
  const void* s1 = a.blob + L.off_s1;
  const void* g = a.blob + L.off_g;
  const void* s2 = a.blob + L.off_s2;
  uint8_t* ws = a.ws;
  hipStream_t st = a.stream;

  ImgOut o1{ws + p.off_img1, reinterpret_cast<uint32_t*>(ws + p.off_xs1), reinterpret_cast<float*>(ws + p.off_sum1),
            p.P, p.TPG, p.NG, p.s1.KT};
  dim3 g1(p.s1.KT), b128(128);
  if (a.x_dtype == 2) {
    if (a.scale_dtype == 1)
      hipLaunchKernelGGL((prep_x_kernel<uint16_t, _Float16>), g1, b128, 0, st, (const uint16_t*)a.x,
                         (const _Float16*)s2, a.n, a.B, o1);
    else
      hipLaunchKernelGGL((prep_x_kernel<uint16_t, float>), g1, b128, 0, st, (const uint16_t*)a.x, (const float*)s2,
                         a.n, a.B, o1);
  } else {
    if (a.scale_dtype == 1)
      hipLaunchKernelGGL((prep_x_kernel<float, _Float16>), g1, b128, 0, st, (const float*)a.x, (const _Float16*)s2,
                         a.n, a.B, o1);
    else
      hipLaunchKernelGGL((prep_x_kernel<float, float>), g1, b128, 0, st, (const float*)a.x, (const float*)s2, a.n,
                         a.B, o1);
  }

  StageK k1{};
  k1.packed = Vt;
  k1.R = a.r;
  k1.RT = p.s1.RT;
  k1.KT = p.s1.KT;
  k1.nsplit = p.s1.nsplit;
  k1.kt_per_split = p.s1.kt_per_split;
  k1.xq = o1.xq;
  k1.xs = o1.xs;
  k1.xsum = o1.xsum;
  k1.P = p.P;
  k1.TPG = p.TPG;
  k1.NG = p.NG;
  k1.B = a.B;
  k1.part = reinterpret_cast<float*>(ws + p.off_part1);
  k1.Rpad = p.s1.RT * TILE_ROWS;
  launch_stage<EPI_PART>(k1, st);

  ImgOut o2{ws + p.off_img2, reinterpret_cast<uint32_t*>(ws + p.off_xs2), reinterpret_cast<float*>(ws + p.off_sum2),
            p.P, p.TPG, p.NG, p.s2.KT};
  dim3 g2(p.s2.KT);
  if (a.scale_dtype == 1)
    hipLaunchKernelGGL((mid_kernel<_Float16>), g2, b128, 0, st, k1.part, p.s1.nsplit, k1.Rpad, (const _Float16*)g,
                       a.r, a.B, o2);
  else
    hipLaunchKernelGGL((mid_kernel<float>), g2, b128, 0, st, k1.part, p.s1.nsplit, k1.Rpad, (const float*)g, a.r,
                       a.B, o2);

  StageK k2{};
  k2.packed = U;
  k2.R = a.m;
  k2.RT = p.s2.RT;
  k2.KT = p.s2.KT;
  k2.nsplit = p.s2.nsplit;
  k2.kt_per_split = p.s2.kt_per_split;
  k2.xq = o2.xq;
  k2.xs = o2.xs;
  k2.xsum = o2.xsum;
  k2.P = p.P;
  k2.TPG = p.TPG;
  k2.NG = p.NG;
  k2.B = a.B;
  k2.y = a.y;
  k2.s1 = s1;
  k2.ydt = a.y_dtype == 0 ? 0 : 2;
  k2.sdt = a.scale_dtype;
  if (p.s2.nsplit == 1) {
    launch_stage<EPI_OUT>(k2, st);
  } else {
    k2.part = reinterpret_cast<float*>(ws + p.off_part2);
    k2.Rpad = p.s2.RT * TILE_ROWS;
    launch_stage<EPI_PART>(k2, st);
    launch_finish(k2.part, p.s2.nsplit, k2.Rpad, a.m, a.B, s1, a.scale_dtype, a.y, k2.ydt, st);
  }
  return hipGetLastError();
}

}  // namespace nq
