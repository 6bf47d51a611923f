// Batch-1 forward on the vector ALU only: each sign bit selects whether its
// activation is added, t = 2 * sum_{bit=1} v - sum v, with the four lanes that
// share a row combined by cross-lane shuffles.  Kept as the plain baseline
// against which the MFMA path is measured; it reads the same packed layout.
#include "nq_common.h"
#include "nq_internal.h"

namespace nq {

ValuPlan valu_plan(int m, int n, int r) {
  ValuPlan p;
  p.s1 = stage_plan(r, n);
  p.s2 = stage_plan(m, r);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  p.off_v1 = take((size_t)p.s1.KT * TILE_COLS * 4);
  p.off_part1 = take((size_t)p.s1.nsplit * p.s1.RT * TILE_ROWS * 4);
  p.off_v2 = take((size_t)p.s2.KT * TILE_COLS * 4);
  p.off_part2 = take(p.s2.nsplit > 1 ? (size_t)p.s2.nsplit * p.s2.RT * TILE_ROWS * 4 : 0);
  p.off_sums = take(256);
  p.bytes = o;
  return p;
}

// v[col] = s2[col] * x[col] (zero past n), for the padded length.
template <typename XT, typename ST>
__global__ void __launch_bounds__(256) valu_prep_kernel(const XT* __restrict__ x, const ST* __restrict__ s2, int n,
                                                        int npad, float* __restrict__ v) {
  int col = blockIdx.x * blockDim.x + threadIdx.x;
  if (col < npad) v[col] = col < n ? to_f32(x[col]) * to_f32(s2[col]) : 0.0f;
}

// v[k] = g[k] * sum_s part[s*Rpad + k] (zero past r).
template <typename ST>
__global__ void __launch_bounds__(256) valu_mid_kernel(const float* __restrict__ part, int nsplit, int Rpad,
                                                       const ST* __restrict__ g, int r, int kpad, float* __restrict__ v) {
  int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= kpad) return;
  float t = 0.0f;
  if (k < r) {
    for (int s = 0; s < nsplit; s++) t += part[(size_t)s * Rpad + k];
    t *= to_f32(g[k]);
  }
  v[k] = t;
}

enum { VEPI_PART = 0, VEPI_OUT = 1 };

template <int EPI>
__global__ void __launch_bounds__(256) valu_stage_kernel(const uint32_t* __restrict__ packed, int R, int RT, int KT,
                                                         int nsplit, int kt_per_split, const float* __restrict__ v,
                                                         float* __restrict__ part, int Rpad, void* y, const void* s1,
                                                         int ydt, int sdt) {
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= RT * nsplit) return;
  const int rt = wid % RT, split = wid / RT;
  const int kt0 = split * kt_per_split, kt1 = min(KT, kt0 + kt_per_split);
  float sel = 0.0f, all = 0.0f;
  for (int kt = kt0; kt < kt1; kt++) {
    const uint32_t word = packed[packed_word_index(rt, kt, lane, KT)];
    const float4* vb = reinterpret_cast<const float4*>(v + kt * TILE_COLS + 32 * (lane >> 4));
    float vv[32];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      float4 t = vb[i];
      vv[4 * i] = t.x; vv[4 * i + 1] = t.y; vv[4 * i + 2] = t.z; vv[4 * i + 3] = t.w;
    }
#pragma unroll
    for (int b = 0; b < 32; b++) {
      const float val = vv[8 * (b & 3) + (b >> 2)];
      sel += ((word >> b) & 1u) ? val : 0.0f;
      all += val;
    }
  }
  float z = 2.0f * sel - all;
  z += __shfl_xor(z, 16);
  z += __shfl_xor(z, 32);
  const int row = rt * TILE_ROWS + (lane & 15);
  if (lane < 16 && row < R) {
    if (EPI == VEPI_PART) {
      part[(size_t)split * Rpad + row] = z;
    } else {
      float sc = sdt == 0 ? reinterpret_cast<const float*>(s1)[row] : (float)reinterpret_cast<const _Float16*>(s1)[row];
      float yv = sc * z;
      if (ydt == 0) reinterpret_cast<float*>(y)[row] = yv;
      else reinterpret_cast<uint16_t*>(y)[row] = f32_to_bf16(yv);
    }
  }
}

hipError_t valu_forward(const FwdArgs& a, const ValuPlan& p) {
  const int sb = a.scale_dtype == 0 ? 4 : 2;
  BlobLayout L = blob_layout(a.m, a.n, a.r, sb);
  const uint32_t* U = reinterpret_cast<const uint32_t*>(a.blob + L.off_u);
  const uint32_t* Vt = reinterpret_cast<const uint32_t*>(a.blob + L.off_vt);
  const void* s1 = a.blob + L.off_s1;
  const void* g = a.blob + L.off_g;
  const void* s2 = a.blob + L.off_s2;
  hipStream_t st = a.stream;
  float* v1 = reinterpret_cast<float*>(a.ws + p.off_v1);
  float* part1 = reinterpret_cast<float*>(a.ws + p.off_part1);
  float* v2 = reinterpret_cast<float*>(a.ws + p.off_v2);
  float* part2 = reinterpret_cast<float*>(a.ws + p.off_part2);
  const int npad = p.s1.KT * TILE_COLS, kpad = p.s2.KT * TILE_COLS;

  dim3 b256(256);
  if (a.x_dtype == 2) {
    if (a.scale_dtype == 1)
      hipLaunchKernelGGL((valu_prep_kernel<uint16_t, _Float16>), dim3(ceil_div(npad, 256)), b256, 0, st,
                         (const uint16_t*)a.x, (const _Float16*)s2, a.n, npad, v1);
    else
      hipLaunchKernelGGL((valu_prep_kernel<uint16_t, float>), dim3(ceil_div(npad, 256)), b256, 0, st,
                         (const uint16_t*)a.x, (const float*)s2, a.n, npad, v1);
  } else {
    if (a.scale_dtype == 1)
      hipLaunchKernelGGL((valu_prep_kernel<float, _Float16>), dim3(ceil_div(npad, 256)), b256, 0, st, (const float*)a.x,
                         (const _Float16*)s2, a.n, npad, v1);
    else
      hipLaunchKernelGGL((valu_prep_kernel<float, float>), dim3(ceil_div(npad, 256)), b256, 0, st, (const float*)a.x,
                         (const float*)s2, a.n, npad, v1);
  }
  const int Rpad1 = p.s1.RT * TILE_ROWS, Rpad2 = p.s2.RT * TILE_ROWS;
  hipLaunchKernelGGL((valu_stage_kernel<VEPI_PART>), dim3(ceil_div(p.s1.RT * p.s1.nsplit, 4)), b256, 0, st, Vt, a.r,
                     p.s1.RT, p.s1.KT, p.s1.nsplit, p.s1.kt_per_split, v1, part1, Rpad1, nullptr, nullptr, 0, 0);
  if (a.scale_dtype == 1)
    hipLaunchKernelGGL((valu_mid_kernel<_Float16>), dim3(ceil_div(kpad, 256)), b256, 0, st, part1, p.s1.nsplit, Rpad1,
                       (const _Float16*)g, a.r, kpad, v2);
  else
    hipLaunchKernelGGL((valu_mid_kernel<float>), dim3(ceil_div(kpad, 256)), b256, 0, st, part1, p.s1.nsplit, Rpad1,
                       (const float*)g, a.r, kpad, v2);
  const int ydt = a.y_dtype == 0 ? 0 : 2;
  if (p.s2.nsplit == 1) {
    hipLaunchKernelGGL((valu_stage_kernel<VEPI_OUT>), dim3(ceil_div(p.s2.RT, 4)), b256, 0, st, U, a.m, p.s2.RT,
                       p.s2.KT, 1, p.s2.kt_per_split, v2, nullptr, 0, a.y, s1, ydt, a.scale_dtype);
  } else {
    hipLaunchKernelGGL((valu_stage_kernel<VEPI_PART>), dim3(ceil_div(p.s2.RT * p.s2.nsplit, 4)), b256, 0, st, U, a.m,
                       p.s2.RT, p.s2.KT, p.s2.nsplit, p.s2.kt_per_split, v2, part2, Rpad2, nullptr, nullptr, 0, 0);
    launch_finish(part2, p.s2.nsplit, Rpad2, a.m, 1, s1, a.scale_dtype, a.y, ydt, st);
  }
  return hipGetLastError();
}

}  // namespace nq
