// Exact attention forward with fp32 inputs and outputs on gfx950.
//
// Same algorithm as the 16-bit kernel (FlashAttention-2 digest, framework-overview
// flowchart: K/V tiles streamed through an online softmax, one final rescale, O and
// LSE stored; split-Q over waves; causal tiles above the diagonal skipped), but every
// quantity stays in fp32: both contractions use v_mfma_f32_32x32x2_f32 and P is never
// rounded to a narrower type. This path serves small fp32 problems; it keeps the
// S^T = K Q^T orientation (one query row per lane) and single-buffers K/V in LDS.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 32;
constexpr int kThreads = 256;

// 32x32x2 fp32 MFMA: lane l holds A[l%32][l/32] and B[l/32][l%32].
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_f32_kernel(const float* __restrict__ Q,
                                                                   const float* __restrict__ K,
                                                                   const float* __restrict__ V, float* __restrict__ O,
                                                                   float* __restrict__ LSE, int N, int n_mtiles,
                                                                   int total_wg, float scale, float c) {
  constexpr int NDB = D / 32;
  constexpr int PAD = 1;                       // row padding (floats) against bank conflicts
  constexpr int LD = D + PAD;
  __shared__ float Ks[kBN * LD];
  __shared__ float Vs[kBN * LD];

  int bh, mt;
  xcd_query_tile(blockIdx.x, total_wg, n_mtiles, CAUSAL, bh, mt);

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int half = lane / 32, l32 = lane % 32;
  const int64_t head_off = (int64_t)bh * N * D;
  const int q0 = mt * kBM + wave * 32;
  const int qrow = q0 + l32;

  float qreg[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qreg[s] = qrow < N ? Q[head_off + (int64_t)qrow * D + s * 2 + half] : 0.f;

  const int n_ktiles = (N + kBN - 1) / kBN;
  int kt_end = n_ktiles;
  if (CAUSAL) kt_end = min(n_ktiles, ((mt + 1) * kBM + kBN - 1) / kBN);
  const int wave_kt_end = CAUSAL ? min(kt_end, (q0 + 31) / kBN + 1) : kt_end;
  const bool wave_live = q0 < N;

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;

  for (int kt = 0; kt < kt_end; ++kt) {
    __syncthreads();
    for (int idx = tid; idx < kBN * D; idx += kThreads) {
      const int r = idx / D, col = idx % D;
      const int key = kt * kBN + r;
      Ks[r * LD + col] = key < N ? K[head_off + (int64_t)key * D + col] : 0.f;
      Vs[r * LD + col] = key < N ? V[head_off + (int64_t)key * D + col] : 0.f;
    }
    __syncthreads();
    if (!wave_live || kt >= wave_kt_end) continue;

    f32x16 s = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 2; ++st) s = mfma32_f32(Ks[l32 * LD + st * 2 + half], qreg[st], s);

    const int key0 = kt * kBN;
    if ((CAUSAL && key0 + kBN - 1 > q0) || key0 + kBN > N) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + (r / 4) * 8 + half * 4 + (r % 4);
        if ((CAUSAL && key > qrow) || key >= N) s[r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx);
    const float mc = m_new * c;
    const float alpha = fast_exp2(m_run * c - mc);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = fast_exp2(__builtin_fmaf(s[r], c, -mc));
      lsum += s[r];
    }
    l_part = l_part * alpha + lsum;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      oacc[db] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r / 4) * 8 + half * 4 + (r % 4);
        oacc[db] = mfma32_f32(Vs[key * LD + db * 32 + l32], s[r], oacc[db]);
      }
    }
  }

  if (!wave_live || qrow >= N) return;
  const float l_tot = add_halves(l_part);
  const float inv = 1.0f / l_tot;
  float* Orow = O + head_off + (int64_t)qrow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + half * 4;
      const f32x16 a = oacc[db];
      *(f32x4*)(Orow + d) = f32x4{a[g * 4] * inv, a[g * 4 + 1] * inv, a[g * 4 + 2] * inv, a[g * 4 + 3] * inv};
    }
  if (half == 0) LSE[(int64_t)bh * N + qrow] = m_run * scale + __builtin_log2f(l_tot) * kLn2;
}

template <int D, bool CAUSAL>
hipError_t launch(const float* q, const float* k, const float* v, float* o, float* lse, int64_t BH, int64_t N,
                  float scale, hipStream_t stream) {
  const int n_mtiles = (int)((N + kBM - 1) / kBM);
  const int64_t total = BH * n_mtiles;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)total), dim3(kThreads), 0, stream, q, k, v, o,
                     lse, (int)N, n_mtiles, (int)total, scale, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int64_t BH, int64_t N,
                          int64_t d, bool causal, float scale, hipStream_t stream) {
  if (d == 128)
    return causal ? launch<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch<128, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch<64, false>(q, k, v, o, lse, BH, N, scale, stream);
}

int64_t max_workgroups_fwd32(int64_t BH, int64_t N) { return BH * ((N + kBM - 1) / kBM); }

}  // namespace attn
