// Fine-grained activation quantisation (the architecture article, section
// 4.2: fp8 GEMM inputs, quantised block by block): every run of 128
// consecutive bf16 values of a row gets one fp32 scale, its largest
// magnitude / 448, and each value becomes the e4m3 code of value / scale.
//
// HBM-bound: 2 bytes read, 1 byte + 4/128 bytes written per element. Sixteen
// lanes hold one block (16 bytes of bf16 each); the block maximum is a
// four-step DPP reduction inside the 16-lane row, so no LDS is used; each
// lane writes its 8 codes as one 8-byte store (a block's codes are 128
// contiguous bytes).
#include "moe_internal.hpp"

namespace moe {

namespace {
constexpr int kThreads = 256;
constexpr int kBlocksPerWG = kThreads / 16;

__global__ __launch_bounds__(kThreads) void quant_e4m3_kernel(const uint16_t* __restrict__ x, size_t nblk,
                                                              uint8_t* __restrict__ q, float* __restrict__ scale) {
  const size_t b = (size_t)blockIdx.x * kBlocksPerWG + (threadIdx.x >> 4);  // block index = row * (cols/128) + j
  const int part = threadIdx.x & 15;
  // whole 16-lane rows are in or out, so the DPP steps below read live lanes
  if (b >= nblk) return;
  const uint4 raw = *reinterpret_cast<const uint4*>(x + b * kActBlock + part * 8);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __uint_as_float(dpp_u32<0xB1>(__float_as_uint(amax))));
  amax = fmaxf(amax, __uint_as_float(dpp_u32<0x4E>(__float_as_uint(amax))));
  amax = fmaxf(amax, __uint_as_float(dpp_u32<0x141>(__float_as_uint(amax))));
  amax = fmaxf(amax, __uint_as_float(dpp_u32<0x140>(__float_as_uint(amax))));
  const float s = e4m3_block_scale(amax);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= e4m3_code(v[i] / s) << (8 * i);
    hi |= e4m3_code(v[4 + i] / s) << (8 * i);
  }
  *reinterpret_cast<uint2*>(q + b * kActBlock + part * 8) = make_uint2(lo, hi);
  if (part == 0) scale[b] = s;
}
}  // namespace

hipError_t launch_quant_e4m3(const uint16_t* x, int rows, int cols, uint8_t* q, float* scale, hipStream_t s) {
  const size_t nblk = (size_t)rows * (cols / kActBlock);
  if (nblk == 0) return hipSuccess;
  const size_t wgs = (nblk + kBlocksPerWG - 1) / kBlocksPerWG;
  hipLaunchKernelGGL(quant_e4m3_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, s, x, nblk, q, scale);
  return hipGetLastError();
}

}  // namespace moe
