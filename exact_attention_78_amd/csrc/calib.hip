// Calibration kernels: what the matrix cores and the transcendental unit of this part
// sustain when nothing else competes, at the clock the chip runs under that load.
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

}  // namespace

hipError_t launch_calib(int kind, const uint32_t* seed, float* out, int64_t workgroups, int iters,
                        hipStream_t stream) {
  if (kind == 0)
    hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)workgroups), dim3(kCalWaves * 64), 0, stream, seed, out,
                       iters);
  else
    hipLaunchKernelGGL(calib_exp_kernel, dim3((unsigned)workgroups), dim3(kCalWaves * 64), 0, stream, seed, out,
                       iters);
  return hipGetLastError();
}

int64_t calib_ops_per_workgroup(int kind, int iters) {
  // MFMA: FLOPs; exp: exponentials
  return kind == 0 ? (int64_t)kCalWaves * iters * kChains * 32768 : (int64_t)kCalWaves * 64 * iters * 16;
}

}  // namespace attn
