// Roofline calibration kernels of libtree_attn (gfx950): the attainable
// bf16 matrix-core rate and the attainable HBM read rate on the GPU at hand,
// measured beside the attention kernels so that their fractions can be read
// against what the chip delivers under load as well as against its
// published peaks.
//
//   calib_mfma_kernel   every wave issues back-to-back
//                       v_mfma_f32_32x32x16_bf16 on eight independent
//                       accumulators (no memory traffic in the loop): 32,768
//                       FLOP per instruction
//   calib_read_kernel   grid-stride 16-byte non-temporal loads over a buffer,
//                       four in flight per thread, folded by XOR so that no
//                       load is dead; one 4-byte word written per workgroup
#include "ta_device.h"

namespace ta {
namespace {

constexpr int kCalibThreads = 256;
constexpr int kCalibAcc = 8;

__global__ __launch_bounds__(kCalibThreads) void calib_mfma_kernel(int32_t iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1e-3f * float(lane + e));
    b[e] = static_cast<__bf16>(1e-3f * float(64 - lane + e));
  }
  f32x16 acc[kCalibAcc];
#pragma unroll
  for (int j = 0; j < kCalibAcc; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kCalibAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kCalibAcc; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  if (lane == 0) sink[int64_t(blockIdx.x) * (kCalibThreads / 64) + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(kCalibThreads) void calib_read_kernel(const u32x4* src, int64_t n16, uint32_t* sink) {
  constexpr int kUnroll = 4;
  const int64_t stride = int64_t(gridDim.x) * kCalibThreads;
  uint32_t x = 0;
  int64_t i = int64_t(blockIdx.x) * kCalibThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) x ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ uint32_t red[kCalibThreads / 64];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= uint32_t(__shfl_xor(int(x), o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
#pragma unroll
    for (int w = 0; w < kCalibThreads / 64; ++w) y ^= red[w];
    sink[blockIdx.x] = y;
  }
}

}  // namespace

hipError_t launch_calib_mfma(int32_t blocks, int32_t iters, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(unsigned(blocks)), dim3(kCalibThreads), 0, st, iters, sink);
  return hipGetLastError();
}

hipError_t launch_calib_read(const void* src, int64_t bytes, int32_t blocks, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(calib_read_kernel, dim3(unsigned(blocks)), dim3(kCalibThreads), 0, st,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

int64_t calib_mfma_flops(int32_t blocks, int32_t iters) {
  return int64_t(blocks) * (kCalibThreads / 64) * int64_t(iters) * kCalibAcc * (2 * 32 * 32 * 16);
}

}  // namespace ta
