// Pack / unpack of sign matrices into the tile layout described in nq_common.h.
//
// The binary factors hold only +1 and -1 (hardwired.dev NanoQuant article,
// section "Jak NanoQuant funguje"); a stored bit encodes that sign (bit 1 = +1).
#include "nq_common.h"
#include "nq_internal.h"

namespace nq {

// One thread per 32-bit word of the packed matrix.  Element (row, col) of the
// source int8 matrix is at M[row * ld_row + col * ld_col].
__global__ void __launch_bounds__(256) pack_kernel(const int8_t* __restrict__ M, int R, int C,
                                                   long long ld_row, long long ld_col,
                                                   uint32_t* __restrict__ out, int RT, int KT,
                                                   int* __restrict__ bad_count) {
  long long wid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long total = (long long)RT * KT * TILE_WORDS;
  if (wid >= total) return;
  int lane = (int)(wid % TILE_WORDS);
  long long t = wid / TILE_WORDS;
  int kt = (int)(t % KT);
  int rt = (int)(t / KT);
  int row = rt * TILE_ROWS + (lane & 15);
  uint32_t word = 0;
  int bad = 0;
  if (row < R) {
    const int8_t* base = M + (long long)row * ld_row;
    for (int b = 0; b < 32; b++) {
      int col = kt * TILE_COLS + packed_bit_col(lane, b);
      if (col < C) {
        int v = base[(long long)col * ld_col];
        if (v == 1) word |= 1u << b;
        else if (v != -1) bad++;
      }
    }
  }
  out[packed_word_index(rt, kt, lane, KT)] = word;
  if (bad) atomicAdd(bad_count, bad);
}

__global__ void __launch_bounds__(256) unpack_kernel(const uint32_t* __restrict__ in, int R, int C,
                                                     long long ld_row, long long ld_col, int RT, int KT,
                                                     int8_t* __restrict__ M) {
  long long wid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long total = (long long)RT * KT * TILE_WORDS;
  if (wid >= total) return;
  int lane = (int)(wid % TILE_WORDS);
  long long t = wid / TILE_WORDS;
  int kt = (int)(t % KT);
  int rt = (int)(t / KT);
  int row = rt * TILE_ROWS + (lane & 15);
  if (row >= R) return;
  uint32_t word = in[packed_word_index(rt, kt, lane, KT)];
  int8_t* base = M + (long long)row * ld_row;
  for (int b = 0; b < 32; b++) {
    int col = kt * TILE_COLS + packed_bit_col(lane, b);
    if (col < C) base[(long long)col * ld_col] = ((word >> b) & 1u) ? (int8_t)1 : (int8_t)-1;
  }
}

// Transpose of a packed sign matrix: src is R x C, dst (C x R) gets
// dst(i, c) = src(c, i).  One thread per dst word; its 32 bits come from 32
// consecutive src rows at one src column, i.e. one fixed bit position of 32
// src words (two row tiles' lanes), which neighbouring threads share through
// the caches.  Padding bits of dst are zero, as pack_kernel writes them.
__global__ void __launch_bounds__(256) transpose_kernel(const uint32_t* __restrict__ src, int R, int C, int KTs,
                                                        uint32_t* __restrict__ dst, int RTd, int KTd) {
  long long wid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long total = (long long)RTd * KTd * TILE_WORDS;
  if (wid >= total) return;
  const int lane = (int)(wid % TILE_WORDS);
  const long long t = wid / TILE_WORDS;
  const int kt = (int)(t % KTd);
  const int rt = (int)(t / KTd);
  const int c = rt * TILE_ROWS + (lane & 15);  // dst row = src column
  uint32_t word = 0;
  if (c < C) {
    const int ktc = c / TILE_COLS, cc = c % TILE_COLS;
    const int sgrp = cc >> 5, c32 = cc & 31;
    const int sbit = 4 * (c32 & 7) + (c32 >> 3);  // bit of column c32 in a word: packed_bit_col inverted
    for (int b = 0; b < 32; b++) {
      const int sr = kt * TILE_COLS + packed_bit_col(lane, b);  // dst column = src row
      if (sr < R) {
        const int slane = (sr & 15) + 16 * sgrp;
        const uint32_t w = src[packed_word_index(sr / TILE_ROWS, ktc, slane, KTs)];
        word |= ((w >> sbit) & 1u) << b;
      }
    }
  }
  dst[packed_word_index(rt, kt, lane, KTd)] = word;
}

hipError_t launch_transpose(const uint32_t* src, int R, int C, uint32_t* dst, hipStream_t s) {
  const PackedDims ds = packed_dims(R, C), dd = packed_dims(C, R);
  const long long total = (long long)dd.RT * dd.KT * TILE_WORDS;
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(transpose_kernel, dim3(blocks), dim3(256), 0, s, src, R, C, ds.KT, dst, dd.RT, dd.KT);
  return hipGetLastError();
}

hipError_t launch_pack(const int8_t* M, int R, int C, long long ld_row, long long ld_col, uint32_t* out,
                       int* bad_count, hipStream_t s) {
  PackedDims d = packed_dims(R, C);
  long long total = (long long)d.RT * d.KT * TILE_WORDS;
  int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, s, M, R, C, ld_row, ld_col, out, d.RT, d.KT,
                     bad_count);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* in, int R, int C, long long ld_row, long long ld_col, int8_t* M,
                         hipStream_t s) {
  PackedDims d = packed_dims(R, C);
  long long total = (long long)d.RT * d.KT * TILE_WORDS;
  int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(unpack_kernel, dim3(blocks), dim3(256), 0, s, in, R, C, ld_row, ld_col, d.RT, d.KT, M);
  return hipGetLastError();
}

}  // namespace nq
