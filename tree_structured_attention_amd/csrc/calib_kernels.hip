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
//   calib_tile_kernel   a model of the forward's 64-key tile loop at bf16,
//                       head_dim 128: per wave and iteration the 16 S MFMAs,
//                       the softmax of 32 scores (fma, exp2, pack, dot2 row
//                       sums, the 2^16 test gating the PV step) and the 16 PV
//                       MFMAs, with a workgroup barrier per iteration, like
//                       the kernel.  Variant 0 keeps the K and V operands in
//                       registers; variant 1 reads them from an LDS tile in
//                       the kernel's layout and order; variant 2 also copies
//                       the next tile from memory into a second LDS stage per
//                       iteration, as the kernel does.  The rates bound what
//                       the tile loop can reach with and without each of the
//                       kernel's memory steps.
// The matrix-core loops take a seed: 0 keeps one fixed, slowly varying
// operand pattern (few bits change from one instruction to the next); any
// other seed fills the operands with pseudo-random bf16 values, so that
// consecutive instructions see unrelated bits as the attention kernels do on
// real data.  The chip draws more power on the second kind and lowers its
// clock under the power limit, so the two rates differ.
#include <algorithm>

#include "ta_device.h"

namespace ta {
namespace {

constexpr int kCalibThreads = 256;
constexpr int kCalibAcc = 8;

// MurmurHash3's 32-bit finalizer (Appleby): a counter-based source of
// well-mixed bits.
__device__ __forceinline__ uint32_t fmix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}
// A pseudo-random bf16 of element `i` under `seed`: random sign and
// mantissa, magnitude in [2^-4, 1).
__device__ __forceinline__ __bf16 rand_bf16(uint32_t seed, uint32_t i) {
  const uint32_t h = fmix32(fmix32(seed) ^ (i * 0x9e3779b9u));
  return __builtin_bit_cast(__bf16, uint16_t((h & 0x807fu) | ((123u + ((h >> 8) & 3u)) << 7)));
}
__device__ __forceinline__ uint32_t thread_id() { return blockIdx.x * blockDim.x + threadIdx.x; }

__global__ __launch_bounds__(kCalibThreads) void calib_mfma_kernel(int32_t iters, uint32_t seed, float* sink) {
  const int lane = threadIdx.x & 63;
  // seed 0: one operand pair for every instruction; otherwise a random pair
  // per accumulator, so consecutive instructions differ in every operand
  bf16x8 a[kCalibAcc], b[kCalibAcc];
#pragma unroll
  for (int j = 0; j < kCalibAcc; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t i = (thread_id() * kCalibAcc + j) * 16 + e;
      a[j][e] = seed ? rand_bf16(seed, i) : static_cast<__bf16>(1e-3f * float(lane + e));
      b[j][e] = seed ? rand_bf16(seed, i + 8) : static_cast<__bf16>(1e-3f * float(64 - lane + e));
    }
  f32x16 acc[kCalibAcc];
#pragma unroll
  for (int j = 0; j < kCalibAcc; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int32_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kCalibAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[j], 0, 0, 0);
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

constexpr int kTileD = 128;
constexpr int64_t kTileRowStride = 8 * kTileD * 2;  // 8 KV heads of bf16 per key row

template <int VAR>
__global__ __launch_bounds__(256, 2) void calib_tile_kernel(int32_t iters, uint32_t seed, float* sink,
                                                            const unsigned char* src, int32_t n_tiles) {
  using G = TileGeom<__bf16, kTileD>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[VAR == 0 ? 16 : (VAR == 1 ? 1 : 2) * G::kStageBytes];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int n = lane & 31, h = lane >> 5;
  bf16x8 qf[8], kf[8], kg[8], vf[4];
  const uint32_t r0 = thread_id() * 224;  // 224 register operands per lane
#pragma unroll
  for (int st = 0; st < 8; ++st)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t i = r0 + 8 * st + e;
      qf[st][e] = seed ? rand_bf16(seed, i) : static_cast<__bf16>(0.01f * float((lane * 7 + st + 2 * e) & 15));
      kf[st][e] = seed ? rand_bf16(seed, i + 64) : static_cast<__bf16>(0.01f * float((lane + 3 * st + e) & 15));
      kg[st][e] = seed ? rand_bf16(seed, i + 128) : static_cast<__bf16>(0.01f * float((lane + 5 * st + 3 * e) & 15));
    }
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vf[m][e] = seed ? rand_bf16(seed, r0 + 192 + 8 * m + e) : static_cast<__bf16>(0.001f * float((lane + m + e) & 31));
  // the kernel's LDS operand offsets (permuted K rows, transposing V reads)
  int koff[8], voff[8];
  {
    const int krow0 = key_perm(n);
#pragma unroll
    for (int st = 0; st < 8; ++st) koff[st] = G::at(krow0, kTileD * h + 16 * st);
    const int m16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int md = 0; md < 4; ++md)
        voff[r * 4 + md] = G::at(8 * (grp >> 1) + 4 * r + (m16 >> 2), 2 * (32 * md + 16 * (grp & 1) + 4 * (m16 & 3)));
  }
  TileLoader<__bf16, kTileD, 4> loader;
  loader.init(lane, wave, kTileRowStride);
  const int kvh = int(blockIdx.x % 8u), tile0 = int(blockIdx.x / 8u);
  const unsigned char* kbase = src + kvh * kTileD * 2;
  const unsigned char* vbase = kbase + int64_t(n_tiles) * kKeyTile * kTileRowStride;
  if constexpr (VAR == 1) {
    for (int i = int(threadIdx.x); i < G::kStageBytes / 4; i += 256) {
      const uint32_t lo = __builtin_bit_cast(uint16_t, rand_bf16(seed, 2 * i));
      const uint32_t hi = __builtin_bit_cast(uint16_t, rand_bf16(seed, 2 * i + 1));
      reinterpret_cast<uint32_t*>(lds)[i] = seed ? lo | (hi << 16) : 0x3c003c00u ^ uint32_t(i & 0xff);
    }
  }
  if constexpr (VAR == 2) {
    const int64_t off = int64_t(tile0 % n_tiles) * kKeyTile * kTileRowStride;
    loader.issue(lds, kbase + off, vbase + off, 0, kKeyTile, kTileRowStride, wave);
  }

  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;
  float l_run = 0.f, mb = 0.5f;
  const float c = 0.1275f;
  const bf16x2v ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  for (int it = 0; it < iters; ++it) {
    const unsigned char* tile = lds + (VAR == 2 ? (it & 1) * G::kStageBytes : 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if constexpr (VAR == 2) {
      if (it + 1 < iters) {
        const int64_t off = int64_t((it + 1 + tile0) % n_tiles) * kKeyTile * kTileRowStride;
        loader.issue(lds + ((it + 1) & 1) * G::kStageBytes, kbase + off, vbase + off, 0, kKeyTile, kTileRowStride,
                     wave);
      }
    }
    if constexpr (VAR == 0) {
      // register operands: an empty asm marks one fragment as changed so the
      // S products are not hoisted out of the loop
      asm volatile("" : "+v"(kf[0]));
      asm volatile("" : "+v"(kg[0]));
    }
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[b][i] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        bf16x8 a = b ? kg[st] : kf[st];
        if constexpr (VAR != 0) a = *reinterpret_cast<const bf16x8*>(tile + koff[st] + 32 * b * G::kRowBytes);
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[b], 0, 0, 0);
      }
    if constexpr (VAR != 0) sched_ld_mfma<0, 16, 1, 4>();
    u32x4 pw[2][2];
    float ls[2] = {0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t pk = pack_bf16x2(fast_exp2(fmaf(s[b][2 * j], c, -mb)), fast_exp2(fmaf(s[b][2 * j + 1], c, -mb)));
        pw[b][j >> 2][j & 3] = pk;
        ls[j & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, pk), ones, ls[j & 1], false);
      }
    const float l = ls[0] + ls[1];
    if (__ballot(l > 65536.f)) {  // never taken for these operands; the PV step waits for the test
      mb += 1.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          pw[b][j >> 2][j & 3] = pack_bf16x2(fast_exp2(fmaf(s[b][2 * j], c, -mb)), fast_exp2(fmaf(s[b][2 * j + 1], c, -mb)));
    }
    l_run += l;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[b][c2]);
        const unsigned char* vb = tile + G::kTileBytes + (32 * b + 16 * c2) * G::kRowBytes;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          bf16x8 a = vf[m];
          if constexpr (VAR != 0) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vb + voff[m]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vb + voff[4 + m]));
            const s16x4 both[2] = {lo, hi};
            a = __builtin_bit_cast(bf16x8, both);
          }
          acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[m], 0, 0, 0);
        }
      }
    if constexpr (VAR != 0) sched_ld_mfma<0, 16, 2, 8>();
  }
  float t = l_run;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) t += acc[m][i];
  if (lane == 0) sink[int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)] = t;
}

}  // namespace

hipError_t launch_calib_tile(int32_t variant, int32_t blocks, int32_t iters, uint32_t seed, const void* src,
                             int64_t src_bytes, float* sink, hipStream_t st) {
  const unsigned char* s8 = static_cast<const unsigned char*>(src);
  const int32_t n_tiles = int32_t(std::min<int64_t>(src_bytes / (2 * kKeyTile * kTileRowStride), 1 << 20));
  if (variant == 0)
    hipLaunchKernelGGL(calib_tile_kernel<0>, dim3(unsigned(blocks)), dim3(256), 0, st, iters, seed, sink, s8, 1);
  else if (variant == 1)
    hipLaunchKernelGGL(calib_tile_kernel<1>, dim3(unsigned(blocks)), dim3(256), 0, st, iters, seed, sink, s8, 1);
  else
    hipLaunchKernelGGL(calib_tile_kernel<2>, dim3(unsigned(blocks)), dim3(256), 0, st, iters, seed, sink, s8,
                       n_tiles);
  return hipGetLastError();
}

int64_t calib_tile_flops(int32_t blocks, int32_t iters) {
  return int64_t(blocks) * 4 * int64_t(iters) * 32 * (2 * 32 * 32 * 16);
}

int64_t calib_tile_min_bytes() { return 2 * kKeyTile * kTileRowStride; }

hipError_t launch_calib_mfma(int32_t blocks, int32_t iters, uint32_t seed, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(unsigned(blocks)), dim3(kCalibThreads), 0, st, iters, seed, sink);
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
