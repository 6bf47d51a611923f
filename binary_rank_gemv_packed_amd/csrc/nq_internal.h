// Internal launchers and launch plans of libnq (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace nq {

hipError_t launch_pack(const int8_t* M, int R, int C, long long ld_row, long long ld_col, uint32_t* out,
                       int* bad_count, hipStream_t s);
hipError_t launch_transpose(const uint32_t* src, int R, int C, uint32_t* dst, hipStream_t s);
hipError_t launch_unpack(const uint32_t* in, int R, int C, long long ld_row, long long ld_col, int8_t* M,
                         hipStream_t s);

// dtype codes match nq_dtype: 0 = f32, 1 = f16, 2 = bf16.
// Optional timing marks: event k is recorded on the stream just before the
// k-th kernel launch of a forward, and one more after the last launch.
struct LaunchMarks {
  hipEvent_t* ev = nullptr;
  int32_t* dims = nullptr;  // per launch: workgroups, threads per workgroup
  int n = 0;
  int k = 0;
  void mark(hipStream_t s, dim3 grid, dim3 block) {
    if (ev && k < n) hipEventRecord(ev[k], s);
    if (dims && k < n - 1) {
      dims[2 * k] = (int32_t)(grid.x * grid.y * grid.z);
      dims[2 * k + 1] = (int32_t)(block.x * block.y * block.z);
    }
    k++;
  }
};

struct FwdArgs {
  int m, n, r, B;
  int scale_dtype, x_dtype, y_dtype;
  const uint8_t* blob;
  const void* x;
  void* y;
  uint8_t* ws;
  size_t ws_bytes;
  hipStream_t stream;
  LaunchMarks* marks = nullptr;  // null: no timing marks
  // rank-l envelope (decode path, row-split stage 2 only): B counts env x the
  // input rows; the env scale-vector pairs are s1_env (env x m), s2_env (env x n)
  int env = 1;
  const void* s1_env = nullptr;
  const void* s2_env = nullptr;
  int s1_env_stride = 0, s2_env_stride = 0;  // elements between rows; a row may be read
                                             // in whole words up to 16 (s1) / 8 (s2) past its end
};

// Before each launch (with its grid and block) and once after the last one
// (no arguments).
inline void mark(const FwdArgs& a, dim3 grid = dim3(0, 0, 0), dim3 block = dim3(0, 0, 0)) {
  if (a.marks) a.marks->mark(a.stream, grid, block);
}

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

// Batch 1..4 decode path (nq_dec.hip).  Stage 1 runs on S1 column splits of
// KL1 tiles with RG1 row tiles per workgroup; stage 2 on RG2 row tiles x KS2
// column parts per workgroup.  fused_mid: stage 2 builds the image of t' itself.
struct DecPlan {
  bool ok, fused_mid;
  bool rows2;  // stage 2 with row-split waves: RG2 row tiles per wave, KS2 waves per workgroup
  int B, CW;
  int RT1, KT1, RG1, KL1, S1, KS1, Rpad1;
  int RT2, KT2, RG2, KS2;
  int QM1, QM2;  // most quads one wave of stage 1 / stage 2 streams per row tile
  size_t lds1, lds2, red1, red2;
  size_t off_img1, off_part, off_img2, off_xpad;
  size_t bytes;
};
// scale_bytes: 2 (fp16) or 4; force_rows: row-split stage 2 whenever it fits (the envelope needs it)
DecPlan dec_plan(int m, int n, int r, int B, int scale_bytes, bool force_rows = false);
hipError_t dec_forward(const FwdArgs& a, const DecPlan& p);

// Several layers that share x (same n, scale dtype, batch <= 4) in two
// launches: stage 1 over all their V^T row tiles, stage 2 block-diagonal.
constexpr int GROUP_MAX = 4;
struct GroupPlan {
  bool ok;
  int L, B, CW;
  int KT1, KL1, S1, RG1, KS1;   // stage 1, common to the layers
  int RG2, KS2;                 // stage 2, common to the layers
  bool rows2;                   // stage 2 with row-split waves (RG2 rows per wave, KS2 waves)
  int RT1[GROUP_MAX], Rpad1[GROUP_MAX], RT2[GROUP_MAX], KT2[GROUP_MAX];
  int wg1_end[GROUP_MAX], wg2_end[GROUP_MAX];  // cumulative workgroups per layer
  size_t lds1, lds2, red1, red2;
  size_t off_part[GROUP_MAX], off_xpad;
  size_t bytes;
};
GroupPlan group_plan(const int* m, const int* r, int L, int n, int B, int scale_bytes);

struct GroupArgs {
  int L, n, B;
  int m[GROUP_MAX], r[GROUP_MAX];
  int scale_dtype, x_dtype, y_dtype;
  const uint8_t* blob[GROUP_MAX];
  const void* x;
  void* y[GROUP_MAX];
  uint8_t* ws;
  hipStream_t stream;
  LaunchMarks* marks = nullptr;
};
hipError_t group_forward(const GroupArgs& a, const GroupPlan& p);

struct ValuPlan {
  StagePlan s1, s2;
  size_t off_v1, off_part1, off_v2, off_part2, off_sums;
  size_t bytes;
};
ValuPlan valu_plan(int m, int n, int r);
hipError_t valu_forward(const FwdArgs& a, const ValuPlan& p);

struct GemmPlan {
  int Bpad, KT1, KT2, RT1, RT2;
  int S1;  // K splits of the first GEMM (partials summed by the mid kernel)
  size_t off_x16, off_xexp, off_t32, off_t16, off_texp;
  size_t bytes;
};
GemmPlan gemm_plan(int m, int n, int r, int B);
hipError_t gemm_forward(const FwdArgs& a, const GemmPlan& p);

// Read-rate probe (nq_probe.hip): reads `bytes` (a multiple of
// PROBE_BATCH_BYTES) once, XORs the words into *sink; *grid receives the grid.
constexpr size_t PROBE_BATCH_BYTES = 16384;
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s, dim3* grid);

// Initialiser (nq_admm.hip): `iters` ADMM steps with a sign projection from
// the latent factors A0 (m x r), B0 (n x r) for W (m x n), all fp32 row-major
// on the device; writes U (m x r), V (n x r) int8 +-1, s1 (m), g (r), s2 (n)
// fp32 and, when err is not null, iters + 1 relative squared errors.
struct AdmmArgs {
  const float* W;
  int m, n, r;
  const float* A0;
  const float* B0;
  float rho;
  int iters, power_iters;
  int8_t* U;
  int8_t* V;
  float* s1;
  float* g;
  float* s2;
  float* err;
  uint8_t* ws;
  hipStream_t stream;
};
size_t admm_workspace_bytes(int m, int n, int r);
hipError_t admm_run(const AdmmArgs& a);
hipError_t launch_balance(float* s1, float* g, float* s2, int m, int n, int r, hipStream_t st);

}  // namespace nq

