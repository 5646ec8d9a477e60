// fp8 input preparation on gfx950: optional Hadamard rotation of each row, then
// per-128-row-block E4M3 quantisation ("8.3 FlashAttention-3", sections 5.1 and 5.2).
//
// One workgroup owns one (batch*head, 128-row block). Each lane holds a 32-element
// segment of a row (64 contiguous bytes), so a row of d elements spans d/32 neighbouring
// lanes. The fast Walsh-Hadamard butterfly runs in fp32 with its stages in the usual
// order (spans 1, 2, 4, ..., d/2): the spans 1..16 combine elements inside a lane, the
// spans 32 and 64 combine a lane with its neighbour (lane xor 1, xor 2) through a DPP
// quad permutation. Every butterfly output is one rounded fp32 add or subtract of the
// same two operands as in the textbook network, so the result does not depend on how
// the elements are laid out. The scale of a block is fp32(amax / 448) (1 for an
// all-zero block); each element becomes the nearest E4M3FN code to
// clamp(fp32(x / scale), -448, 448) via v_cvt_pk_fp8_f32 (round to nearest even on
// gfx950; out-of-range inputs would give NaN, hence the clamp).
//
// The kernel reads 2 bytes and writes 1 byte per element.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kRowsPerBlock = 128;
constexpr int kThreads = 256;

// Value held by lane (this lane xor 1) or (xor 2): DPP quad permutations.
template <int B>
__device__ __forceinline__ float xor_lane(float x) {
  constexpr int ctrl = B == 0 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xF, 0xF, true));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

// One (batch*head, 128-row block) of one tensor: workgroup `wg` of a grid over BH * nblk.
template <int D, bool ROTATE>
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ X, uint8_t* __restrict__ X8,
                                            float* __restrict__ scales, const float* __restrict__ signs, int N,
                                            int nblk, float inv_sqrt_d, int wg, float* wave_max) {
  constexpr int EPL = 32;                                      // elements per lane segment
  constexpr int LPR = D / EPL;                                 // lanes per row (4 or 2)
  constexpr int RPP = kThreads / LPR;                          // rows per pass
  constexpr int PASSES = kRowsPerBlock / RPP;                  // 2 or 1

  const int bh = wg / nblk, blk = wg % nblk;
  const int tid = threadIdx.x, lane = tid % 64;
  const int seg = tid % LPR;                                   // this lane's segment of a row
  const int64_t base = ((int64_t)bh * N + (int64_t)blk * kRowsPerBlock) * D;

  float sg[EPL];
  if constexpr (ROTATE) {
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) {
      const f32x4 v = *(const f32x4*)(signs + seg * EPL + i * 4);
      sg[4 * i] = v[0]; sg[4 * i + 1] = v[1]; sg[4 * i + 2] = v[2]; sg[4 * i + 3] = v[3];
    }
  }
  // +1 for the lower, -1 for the upper lane of a cross-lane pair: out = partner + sign * own
  float lane_sign[2];
  lane_sign[0] = (seg & 1) ? -1.f : 1.f;
  lane_sign[1] = (seg & 2) ? -1.f : 1.f;

  float x[PASSES][EPL];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = tid / LPR + p * RPP;
    const bool valid = blk * kRowsPerBlock + row < N;
    const uint16_t* src = X + base + (int64_t)row * D + seg * EPL;
#pragma unroll
    for (int i = 0; i < EPL / 8; ++i) {
      const u32x4 raw = valid ? *(const u32x4*)(src + i * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[p][i * 8 + 2 * e] = bf16_to_f32(raw[e] & 0xFFFFu);
        x[p][i * 8 + 2 * e + 1] = bf16_to_f32(raw[e] >> 16);
      }
    }
    if constexpr (ROTATE) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[p][e] *= sg[e];          // exact (+-1)
      // spans 1 .. 16: inside the lane
#pragma unroll
      for (int h = 1; h < EPL; h *= 2)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          if (!(e & h)) {
            const float a = x[p][e], b = x[p][e + h];
            x[p][e] = a + b;
            x[p][e + h] = a - b;
          }
      // spans 32, 64: across lanes; the upper lane of a pair gets partner - own, the
      // lower own + partner, each one rounded fp32 operation (fma with a +-1 factor)
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[p][e] = __builtin_fmaf(lane_sign[0], x[p][e], xor_lane<0>(x[p][e]));
      if constexpr (LPR == 4) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[p][e] = __builtin_fmaf(lane_sign[1], x[p][e], xor_lane<1>(x[p][e]));
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[p][e] *= inv_sqrt_d;
    }
#pragma unroll
    for (int e = 0; e < EPL; e += 2)
      amax = __builtin_elementwise_maximum(amax, __builtin_elementwise_maximum(__builtin_fabsf(x[p][e]),
                                                                                __builtin_fabsf(x[p][e + 1])));
  }

  // block amax: wave reduction, then across the 4 waves
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (lane == 0) wave_max[tid / 64] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  // x / s, correctly rounded, from the correctly rounded reciprocal y = 1/s (one IEEE
  // division per thread) and one FMA correction per element (Markstein's division
  // theorem: with y within half an ulp of 1/s and q0 = RN(x*y) close to x/s, the residual
  // r = x - s*q0 is exact and RN(q0 + r*y) is the correctly rounded quotient; checked
  // against exact rational arithmetic on the CPU and bit-exactly against the oracle).
  // The theorem needs 1/s finite and r clear of the subnormal range. For a block of tiny
  // values (s < 2^-64, s possibly subnormal) both x and s are first multiplied by 2^64:
  // the products are exact, so the quotient is the same, and with the scaled divisor
  // s' >= 2^-78 every quotient that can reach a nonzero code keeps r normal.
  float sd = s;
  if (s < 0x1p-64f) {                                          // block-uniform, rare
    sd = s * 0x1p64f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[p][e] *= 0x1p64f;
  }
  const float y_rcp = 1.0f / sd;

#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = tid / LPR + p * RPP;
    if (blk * kRowsPerBlock + row >= N) continue;
    int w[EPL / 4];
#pragma unroll
    for (int e = 0; e < EPL; e += 2) {
      float y[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float xv = x[p][e + k];
        const float q0 = xv * y_rcp;
        // (copysign keeps the sign of a zero input: -0 / s is -0, but the correction sums +0 and -0)
        const float q = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, sd, xv), y_rcp, q0), xv);
        y[k] = fminf(fmaxf(q, -448.0f), 448.0f);
      }
      if (e % 4 == 0) w[e / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      else w[e / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], w[e / 4], true);
    }
    uint8_t* dst = X8 + base + (int64_t)row * D + seg * EPL;
    *(u32x4*)dst = u32x4{(uint32_t)w[0], (uint32_t)w[1], (uint32_t)w[2], (uint32_t)w[3]};
    *(u32x4*)(dst + 16) = u32x4{(uint32_t)w[4], (uint32_t)w[5], (uint32_t)w[6], (uint32_t)w[7]};
  }
  if (tid == 0) scales[(int64_t)bh * nblk + blk] = s;
}

template <int D, bool ROTATE>
__global__ __launch_bounds__(kThreads) void quant_fp8_kernel(const uint16_t* __restrict__ X, uint8_t* __restrict__ X8,
                                                             float* __restrict__ scales,
                                                             const float* __restrict__ signs, int N, int nblk,
                                                             float inv_sqrt_d) {
  __shared__ float wave_max[kThreads / 64];
  quant_block<D, ROTATE>(X, X8, scales, signs, N, nblk, inv_sqrt_d, blockIdx.x, wave_max);
}

// Q (rotated, when nq = 1), K (rotated) and V (unrotated) of one attention call in one
// launch: in blocks of n_wg = BH * nblk workgroups, Q's blocks first (nq = 1), then K's,
// then V's.
template <int D>
__global__ __launch_bounds__(kThreads) void quant_fp8_qkv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint8_t* __restrict__ Q8, uint8_t* __restrict__ K8, uint8_t* __restrict__ V8, float* __restrict__ sq,
    float* __restrict__ sk, float* __restrict__ sv, const float* __restrict__ signs, int N, int nblk, int n_wg, int nq,
    float inv_sqrt_d) {
  __shared__ float wave_max[kThreads / 64];
  const int wg = blockIdx.x, t = wg / n_wg + (nq ? 0 : 1);   // 0 Q (only when nq = 1), 1 K, 2 V
  if (t == 0)
    quant_block<D, true>(Q, Q8, sq, signs, N, nblk, inv_sqrt_d, wg % n_wg, wave_max);
  else if (t == 1)
    quant_block<D, true>(K, K8, sk, signs, N, nblk, inv_sqrt_d, wg % n_wg, wave_max);
  else
    quant_block<D, false>(V, V8, sv, nullptr, N, nblk, inv_sqrt_d, wg % n_wg, wave_max);
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

template <int D>
hipError_t launch_qkv(const void* q, const void* k, const void* v, uint8_t* q8, uint8_t* k8, uint8_t* v8, float* sq,
                      float* sk, float* sv, const float* signs, int64_t BH, int64_t N, hipStream_t stream) {
  const int nblk = (int)((N + kRowsPerBlock - 1) / kRowsPerBlock);
  const float inv_sqrt_d = (float)(1.0 / __builtin_sqrt((double)D));
  const int64_t n_wg = BH * nblk;
  const int nq = q != nullptr ? 1 : 0;
  hipLaunchKernelGGL((quant_fp8_qkv_kernel<D>), dim3((unsigned)((2 + nq) * n_wg)), dim3(kThreads), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, q8, k8, v8, sq, sk, sv, signs, (int)N,
                     nblk, (int)n_wg, nq, inv_sqrt_d);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_fp8_qkv(const void* q, const void* k, const void* v, uint8_t* q8, uint8_t* k8, uint8_t* v8,
                                float* q_scales, float* k_scales, float* v_scales, const float* signs, int64_t BH,
                                int64_t N, int64_t d, hipStream_t stream) {
  return d == 128 ? launch_qkv<128>(q, k, v, q8, k8, v8, q_scales, k_scales, v_scales, signs, BH, N, stream)
                  : launch_qkv<64>(q, k, v, q8, k8, v8, q_scales, k_scales, v_scales, signs, BH, N, stream);
}

hipError_t launch_quant_fp8(const void* x, uint8_t* x8, float* scales, const float* signs, int64_t BH, int64_t N,
                            int64_t d, hipStream_t stream) {
  return d == 128 ? launch<128>(x, x8, scales, signs, BH, N, stream) : launch<64>(x, x8, scales, signs, BH, N, stream);
}

int64_t max_workgroups_quant(int64_t BH, int64_t N) { return BH * ((N + kRowsPerBlock - 1) / kRowsPerBlock); }

}  // namespace attn
