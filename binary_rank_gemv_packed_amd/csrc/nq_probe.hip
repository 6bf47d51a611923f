// HBM read-rate probe: reads a device buffer once with the access pattern of
// the decode kernels' weight stream (each wave issues sixteen 1 KiB loads, one
// 16-byte word per lane, all in flight before it consumes any) and folds the
// words into one XOR so that no load can be dropped.  It computes nothing of
// the layer; it measures what a kernel of this shape can read per second.
#include <hip/hip_runtime.h>

#include "nq_internal.h"

namespace nq {

typedef unsigned int probe_u4 __attribute__((ext_vector_type(4)));

constexpr int PROBE_WAVES_PER_WG = 4;
constexpr int PROBE_MAX_WAVES = 256 * 16;  // 16 resident waves per CU

__global__ void __launch_bounds__(64 * PROBE_WAVES_PER_WG)
read_probe_kernel(const probe_u4* __restrict__ p, long long batches, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const long long wave = (long long)blockIdx.x * PROBE_WAVES_PER_WG + (threadIdx.x >> 6);
  const long long nwaves = (long long)gridDim.x * PROBE_WAVES_PER_WG;
  uint32_t acc = 0;
  for (long long b = wave; b < batches; b += nwaves) {
    const probe_u4* q = p + b * (PROBE_BATCH_BYTES / 16) + lane;
    probe_u4 v[16];
#pragma unroll
    for (int k = 0; k < 16; k++) v[k] = __builtin_nontemporal_load(q + 64 * k);
#pragma unroll
    for (int k = 0; k < 16; k++) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (lane == 0 && acc) atomicXor(sink, acc);
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s, dim3* grid) {
  const long long batches = (long long)(bytes / PROBE_BATCH_BYTES);
  const long long waves = batches < PROBE_MAX_WAVES ? batches : PROBE_MAX_WAVES;
  const dim3 g((unsigned)((waves + PROBE_WAVES_PER_WG - 1) / PROBE_WAVES_PER_WG)), b(64 * PROBE_WAVES_PER_WG);
  if (grid) *grid = g;
  read_probe_kernel<<<g, b, 0, s>>>(static_cast<const probe_u4*>(buf), batches, sink);
  return hipGetLastError();
}

}  // namespace nq
