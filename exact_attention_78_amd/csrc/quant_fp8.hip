// fp8 input preparation on gfx950: optional Hadamard rotation of each row, then
// per-128-row-block E4M3 quantisation ("8.3 FlashAttention-3", sections 5.1 and 5.2).
//
// One workgroup owns one (batch*head, 128-row block). Each lane holds 16-byte chunks
// (8 consecutive elements) of the block, so a row of d elements spans d/8 neighbouring
// lanes. The fast Walsh-Hadamard butterfly runs in fp32: the spans 1, 2, 4 combine
// elements inside a lane, the spans 8 .. d/2 combine a lane with the lane whose chunk
// index differs in one bit, fetched with DPP lane moves. Every butterfly output is one
// rounded fp32 add or subtract of the same two operands at every stage, so the result
// does not depend on how the stages are scheduled. The scale of a block is
// fp32(amax / 448) (1 for an all-zero block); each element becomes the nearest E4M3FN
// code to clamp(fp32(x / scale), -448, 448) via v_cvt_pk_fp8_f32 (round to nearest
// even on gfx950; out-of-range inputs would give NaN, hence the clamp).
//
// The kernel is bound by HBM: it reads 2 bytes and writes 1 byte per element.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kRowsPerBlock = 128;
constexpr int kThreads = 256;

// DPP lane moves within 16-lane rows (controls: quad_perm, row_shl, row_shr).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Value held by the lane whose index differs in bit b (b = 0..3), same slot.
template <int B>
__device__ __forceinline__ float xor_lane(float x, int lane) {
  if constexpr (B == 0) return dpp<0xB1>(x);                          // quad_perm [1,0,3,2]
  else if constexpr (B == 1) return dpp<0x4E>(x);                     // quad_perm [2,3,0,1]
  else if constexpr (B == 2) {
    const float up = dpp<0x104>(x);                                   // row_shl:4 -> lane+4
    const float dn = dpp<0x114>(x);                                   // row_shr:4 -> lane-4
    return (lane & 4) ? dn : up;
  } else {
    const float up = dpp<0x108>(x);                                   // row_shl:8 -> lane+8
    const float dn = dpp<0x118>(x);                                   // row_shr:8 -> lane-8
    return (lane & 8) ? dn : up;
  }
}

// One cross-lane butterfly stage over all 8 slots of a chunk: chunk-index bit B.
template <int B>
__device__ __forceinline__ void cross_stage(float (&x)[8], int lane) {
  const bool upper = (lane >> B) & 1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = xor_lane<B>(x[e], lane);
    x[e] = upper ? (p - x[e]) : (x[e] + p);
  }
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

template <int D, bool ROTATE>
__global__ __launch_bounds__(kThreads) void quant_fp8_kernel(const uint16_t* __restrict__ X, uint8_t* __restrict__ X8,
                                                             float* __restrict__ scales,
                                                             const float* __restrict__ signs, int N, int nblk,
                                                             float inv_sqrt_d) {
  constexpr int NCH = D / 8;                                   // chunks per row
  constexpr int CPT = kRowsPerBlock * NCH / kThreads;          // chunks per thread
  __shared__ float wave_max[kThreads / 64];

  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int tid = threadIdx.x, lane = tid % 64;
  const int c = tid % NCH;                                     // this lane's chunk within a row
  const int64_t base = ((int64_t)bh * N + (int64_t)blk * kRowsPerBlock) * D;

  float sg[8];
  if constexpr (ROTATE) {
    const f32x4 s0 = *(const f32x4*)(signs + c * 8), s1 = *(const f32x4*)(signs + c * 8 + 4);
    sg[0] = s0[0]; sg[1] = s0[1]; sg[2] = s0[2]; sg[3] = s0[3];
    sg[4] = s1[0]; sg[5] = s1[1]; sg[6] = s1[2]; sg[7] = s1[3];
  }

  float x[CPT][8];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < CPT; ++p) {
    const int idx = tid + p * kThreads;
    const int row = idx / NCH;
    const bool valid = blk * kRowsPerBlock + row < N;
    u32x4 raw = valid ? *(const u32x4*)(X + base + (int64_t)row * D + c * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[p][2 * e] = bf16_to_f32(raw[e] & 0xFFFFu);
      x[p][2 * e + 1] = bf16_to_f32(raw[e] >> 16);
    }
    if constexpr (ROTATE) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[p][e] *= sg[e];
      // spans 1, 2, 4: inside the lane
#pragma unroll
      for (int h = 1; h < 8; h *= 2)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!(e & h)) {
            const float a = x[p][e], b = x[p][e + h];
            x[p][e] = a + b;
            x[p][e + h] = a - b;
          }
      // spans 8 .. D/2: across lanes
      cross_stage<0>(x[p], lane);
      cross_stage<1>(x[p], lane);
      cross_stage<2>(x[p], lane);
      if constexpr (D == 128) cross_stage<3>(x[p], lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[p][e] *= inv_sqrt_d;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[p][e]));
  }

  // block amax: wave reduction, then across the 4 waves
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (lane == 0) wave_max[tid / 64] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;

#pragma unroll
  for (int p = 0; p < CPT; ++p) {
    const int idx = tid + p * kThreads;
    const int row = idx / NCH;
    if (blk * kRowsPerBlock + row >= N) continue;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(x[p][e] / s, -448.0f), 448.0f);
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
    *(u32x2*)(X8 + base + (int64_t)row * D + c * 8) = u32x2{(uint32_t)w0, (uint32_t)w1};
  }
  if (tid == 0) scales[(int64_t)bh * nblk + blk] = s;
}

template <int D>
hipError_t launch(const void* x, uint8_t* x8, float* sc, const float* signs, int64_t BH, int64_t N,
                  hipStream_t stream) {
  const int nblk = (int)((N + kRowsPerBlock - 1) / kRowsPerBlock);
  const float inv_sqrt_d = (float)(1.0 / __builtin_sqrt((double)D));
  const dim3 grid((unsigned)(BH * nblk));
  if (signs)
    hipLaunchKernelGGL((quant_fp8_kernel<D, true>), grid, dim3(kThreads), 0, stream, (const uint16_t*)x, x8, sc, signs,
                       (int)N, nblk, inv_sqrt_d);
  else
    hipLaunchKernelGGL((quant_fp8_kernel<D, false>), grid, dim3(kThreads), 0, stream, (const uint16_t*)x, x8, sc,
                       signs, (int)N, nblk, inv_sqrt_d);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_fp8(const void* x, uint8_t* x8, float* scales, const float* signs, int64_t BH, int64_t N,
                            int64_t d, hipStream_t stream) {
  return d == 128 ? launch<128>(x, x8, scales, signs, BH, N, stream) : launch<64>(x, x8, scales, signs, BH, N, stream);
}

int64_t max_workgroups_quant(int64_t BH, int64_t N) { return BH * ((N + kRowsPerBlock - 1) / kRowsPerBlock); }

}  // namespace attn
