// Internal launchers and launch plans of libnq (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace nq {

hipError_t launch_pack(const int8_t* M, int R, int C, long long ld_row, long long ld_col, uint32_t* out,
                       int* bad_count, hipStream_t s);
hipError_t launch_unpack(const uint32_t* in, int R, int C, long long ld_row, long long ld_col, int8_t* M,
                         hipStream_t s);

// dtype codes match nq_dtype: 0 = f32, 1 = f16, 2 = bf16.
struct FwdArgs {
  int m, n, r, B;
  int scale_dtype, x_dtype, y_dtype;
  const uint8_t* blob;
  const void* x;
  void* y;
  uint8_t* ws;
  size_t ws_bytes;
  hipStream_t stream;
};

// Work split of one sign-matrix product over wavefronts: each wave handles one
// 16-row tile and kt_per_split column tiles (a multiple of 4).
struct StagePlan {
  int RT, KT;
  int nsplit, kt_per_split;
};

StagePlan stage_plan(int R, int C);
// y = s1 * (sum over nsplit partial results part[(s*B + b)*Rpad + i]).
void launch_finish(const float* part, int nsplit, int Rpad, int m, int B, const void* s1, int sdt, void* y, int ydt,
                   hipStream_t st);

struct GemvPlan {
  int P, TPG, NG;
  StagePlan s1, s2;
  size_t off_img1, off_xs1, off_sum1, off_part1;
  size_t off_img2, off_xs2, off_sum2, off_part2;
  size_t bytes;
};
GemvPlan gemv_plan(int m, int n, int r, int B);
hipError_t gemv_forward(const FwdArgs& a, const GemvPlan& p);

struct ValuPlan {
  StagePlan s1, s2;
  size_t off_v1, off_part1, off_v2, off_part2, off_sums;
  size_t bytes;
};
ValuPlan valu_plan(int m, int n, int r);
hipError_t valu_forward(const FwdArgs& a, const ValuPlan& p);

struct GemmPlan {
  int Bpad, KT1, KT2, RT1, RT2;
  size_t off_x16, off_xexp, off_t32, off_t16, off_texp;
  size_t bytes;
};
GemmPlan gemm_plan(int m, int n, int r, int B);
hipError_t gemm_forward(const FwdArgs& a, const GemmPlan& p);

}  // namespace nq
