// Calibration kernels: what the matrix cores, the transcendental unit and the memory
// system of this part sustain when nothing else competes, at the clock the chip runs
// under that load.
//
// The forward kernels are judged against the published dense MFMA peak (256 CUs x
// 2.4 GHz x 4096 bf16 FLOP per clock); under full MFMA load the engine clock drops below
// 2.4 GHz, so these loops measure the attainable rate on the same launch shape the
// attention kernels use (one workgroup of 8 waves per CU, two waves per SIMD). The
// softmax's exponentials are the main non-MFMA cost ("8.3 FlashAttention-3", section 1:
// the exponential unit is far slower than the matrix units), so the second loop measures
// v_exp_f32 throughput, the secondary bound of the forward pass.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kCalWaves = 8;
constexpr int kChains = 8;   // independent accumulators per wave: no MFMA waits on its predecessor

// Each wave: iters x kChains independent 32x32x16 bf16 MFMAs (32768 FLOPs each). The
// operands come from the inputs so that nothing folds; each lane writes one sum.
__global__ __launch_bounds__(kCalWaves * 64, 1) void calib_mfma_kernel(const uint32_t* __restrict__ seed, float* out,
                                                                       int iters) {
  const int lane = threadIdx.x % 64;
  const u32x4 a = {seed[lane % 4], seed[(lane + 1) % 4], seed[(lane + 2) % 4], seed[(lane + 3) % 4]};
  const u32x4 b = {seed[(lane + 3) % 4], seed[(lane + 2) % 4], seed[(lane + 1) % 4], seed[lane % 4]};
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = mfma32(Bf16Tag{}, a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Each lane: iters x 16 independent chains of x <- 2^-x (v_exp_f32 with a negated
// source, which the instruction encodes for free; the values stay in [1/2, 1]).
__global__ __launch_bounds__(kCalWaves * 64, 1) void calib_exp_kernel(const uint32_t* __restrict__ seed, float* out,
                                                                      int iters) {
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = 0.5f + (float)((seed[j % 4] >> j) & 7) * 0.01f + 0.001f * (float)(threadIdx.x % 64);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = fast_exp2(-x[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// MFMA loop with other work between the MFMAs, to price what the attention kernels put
// there: after every 32x32x16 bf16 MFMA, NF fp32 FMAs, NE exponentials and NA adds on
// registers independent of the MFMAs, and one 16-byte LDS read (ds_read_b128) every
// 16/ND MFMAs that feeds the next MFMA's A operand (ND = 0: none). WV waves per
// workgroup (8: two per SIMD, 4: one per SIMD; the 128 KiB of LDS keep one workgroup per
// CU). Each wave runs iters x 16 MFMAs over four accumulators.
template <int NF, int NE, int NA, int ND, int WV>
__global__ __launch_bounds__(WV * 64, 1) void calib_mix_kernel(const uint32_t* __restrict__ seed, float* out,
                                                               int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[131072];
  const int lane = threadIdx.x % 64;
  for (int i = threadIdx.x; i < 131072 / 4; i += WV * 64) ((uint32_t*)lds)[i] = seed[i % 4];
  __syncthreads();
  const u32x4 a = {seed[lane % 4], seed[(lane + 1) % 4], seed[(lane + 2) % 4], seed[(lane + 3) % 4]};
  const u32x4 b = a;
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
  float x[16], y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    x[j] = 0.5f + 0.001f * lane + j * 0.01f;
    y[j] = 0.25f + j * 0.02f;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      u32x4 aa = a;
      // lane * 16 + m * 1024 + (it % 4) * 16384 + 16 <= 131072: inside the array
      if (ND > 0 && m % (16 / ND) == 0) aa = *(const u32x4*)(lds + lane * 16 + m * 1024 + (it & 3) * 16384);
      acc[m % 4] = mfma32(Bf16Tag{}, aa, b, acc[m % 4]);
#pragma unroll
      for (int f = 0; f < NF; ++f) x[(m * 3 + f) % 16] = __builtin_fmaf(x[(m * 3 + f) % 16], 0.999f, y[f % 16]);
#pragma unroll
      for (int e = 0; e < NE; ++e) y[(m * 5 + e) % 16] = fast_exp2(-y[(m * 5 + e) % 16]);
#pragma unroll
      for (int d = 0; d < NA; ++d) x[(m * 7 + d + 1) % 16] += y[(m + d) % 16];
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[c][r];
#pragma unroll
  for (int j = 0; j < 16; ++j) sum += x[j] + y[j];
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = sum;
}

// Streaming reads (kind 6): what the memory system delivers to a kernel that only reads,
// the attainable rate of the HBM-bound kernels beside the published 8 TB/s. Each of the
// grid's threads loads one 16-byte element per iteration; iteration i of the grid covers
// the consecutive elements [i * G, (i + 1) * G) (G = threads of the grid), so the whole
// grid sweeps the buffer once, front to back.
constexpr int kReadThreads = 256;
__global__ __launch_bounds__(kReadThreads) void calib_read_kernel(const u32x4* __restrict__ src, float* out,
                                                                   int iters) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it, i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(int64_t)blockIdx.x * kReadThreads + threadIdx.x] = (float)acc;
}

// LDS read rate (kinds 7, 8): 8 waves per workgroup (the 128 KiB of LDS keep one
// workgroup per CU), each lane reading 16 bytes (ds_read_b128, TR
// false) or 8 bytes (ds_read_b64_tr_b16, TR true: the transpose reads that give the
// attention kernels their V^T and Q^T / dO^T operands) per instruction, 16 instructions per
// iteration, from addresses that put the 64 lanes on distinct banks. The values are
// XOR-accumulated, so that no read is dead, and the result is written as a small integer
// (a finite float).
template <bool TR>
__global__ __launch_bounds__(kCalWaves * 64, 1) void calib_lds_kernel(const uint32_t* __restrict__ seed, float* out,
                                                                     int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[131072];
  for (int i = threadIdx.x; i < 131072 / 4; i += kCalWaves * 64) ((uint32_t*)lds)[i] = seed[i % 4] + i;
  __syncthreads();
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      // lane * 16 + 15 * 1024 + 7 * 16384 + 16 <= 131072: inside the array
      const uint8_t* p = lds + lane * 16 + ((m + wave) % 16) * 1024 + (it & 7) * 16384;
      if constexpr (TR) {
        const u32x2 v = lds_read_tr16((const uint16_t*)p);
        acc ^= v[0] ^ v[1];
      } else {
        const u32x4 v = *(const u32x4*)p;
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    }
  }
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = (float)(acc & 0xFFFFu);
}

// kinds 2..5 of attn_calibrate: the mixes above
struct Mix {
  int waves;
};
constexpr Mix kMix[4] = {{8}, {8}, {4}, {8}};

}  // namespace

hipError_t launch_calib(int kind, const uint32_t* seed, float* out, int64_t workgroups, int iters,
                        hipStream_t stream) {
  const dim3 grid((unsigned)workgroups);
  switch (kind) {
    case 0: hipLaunchKernelGGL(calib_mfma_kernel, grid, dim3(kCalWaves * 64), 0, stream, seed, out, iters); break;
    case 1: hipLaunchKernelGGL(calib_exp_kernel, grid, dim3(kCalWaves * 64), 0, stream, seed, out, iters); break;
    case 2: hipLaunchKernelGGL((calib_mix_kernel<1, 1, 1, 16, 8>), grid, dim3(8 * 64), 0, stream, seed, out, iters); break;
    case 3: hipLaunchKernelGGL((calib_mix_kernel<1, 1, 1, 8, 8>), grid, dim3(8 * 64), 0, stream, seed, out, iters); break;
    case 4: hipLaunchKernelGGL((calib_mix_kernel<1, 1, 1, 8, 4>), grid, dim3(4 * 64), 0, stream, seed, out, iters); break;
    case 5: hipLaunchKernelGGL((calib_mix_kernel<1, 1, 1, 0, 8>), grid, dim3(8 * 64), 0, stream, seed, out, iters); break;
    case 7: hipLaunchKernelGGL(calib_lds_kernel<false>, grid, dim3(kCalWaves * 64), 0, stream, seed, out, iters); break;
    case 8: hipLaunchKernelGGL(calib_lds_kernel<true>, grid, dim3(kCalWaves * 64), 0, stream, seed, out, iters); break;
    default:
      hipLaunchKernelGGL(calib_read_kernel, grid, dim3(kReadThreads), 0, stream, (const u32x4*)seed, out, iters);
      break;
  }
  return hipGetLastError();
}

int64_t calib_ops_per_workgroup(int kind, int iters) {
  // MFMA kinds: FLOPs; exp: exponentials
  if (kind == 0) return (int64_t)kCalWaves * iters * kChains * 32768;
  if (kind == 1) return (int64_t)kCalWaves * 64 * iters * 16;
  if (kind == 6) return (int64_t)kReadThreads * iters * 16;   // bytes read
  if (kind == 7 || kind == 8) return (int64_t)kCalWaves * 64 * iters * 16 * (kind == 7 ? 16 : 8);   // LDS bytes read
  return (int64_t)kMix[kind - 2].waves * iters * 16 * 32768;
}

}  // namespace attn
