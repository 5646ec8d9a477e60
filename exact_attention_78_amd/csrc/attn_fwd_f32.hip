// Exact attention forward with fp32 inputs and outputs on gfx950.
//
// Same algorithm as the 16-bit kernel (FlashAttention-2 digest, framework-overview
// flowchart: K/V tiles streamed through an online softmax, one final rescale, O and
// LSE stored; causal tiles above the diagonal skipped), but every quantity stays in fp32:
// both contractions use v_mfma_f32_32x32x2_f32 and P is never rounded to a narrower type.
// This path serves small fp32 problems, where one wave's chain of key tiles would be the
// whole time: the key tiles of a 32-row query block are split over the workgroup's waves,
// whose partial results are merged at the end. It keeps the S^T = K Q^T orientation (one
// query row per lane).
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kBM = 32;      // query rows per workgroup
constexpr int kBN = 32;      // keys per tile
constexpr int kW = 4;        // waves per workgroup: the key tiles are split over them
constexpr int kThreads = kW * 64;

// 32x32x2 fp32 MFMA: lane l holds A[l%32][l/32] and B[l/32][l%32].
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// One workgroup per (batch*head, 32-row query block); its 4 waves take the key tiles w,
// w + 4, w + 8, ... (split over keys, so that a short sequence is not one wave's serial
// chain of tiles), each with its own K/V tile buffer in LDS and its own running max, row
// sum and O partial, which the waves then merge through LDS as the split-KV decoding
// step does: m = max of the waves' maxima, each wave's sum and O weighted by
// 2^((m_w - m) * scale * log2 e).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_f32_kernel(const float* __restrict__ Q,
                                                                   const float* __restrict__ K,
                                                                   const float* __restrict__ V, float* __restrict__ O,
                                                                   float* __restrict__ LSE, int N, int n_mtiles,
                                                                   int total_wg, float scale, float c) {
  constexpr int NDB = D / 32;
  constexpr int PAD = 1;                       // row padding (floats) against bank conflicts
  constexpr int LD = D + PAD;
  constexpr int TILE = kBN * LD;               // floats of one K (or V) tile
  constexpr int NV = 16 * NDB;                 // O values per lane
  __shared__ float lds[kW * 2 * TILE];         // per wave: K tile, V tile; then the merge
  static_assert(kW * (2 + NV) * 64 <= kW * 2 * TILE, "the merge fits the tiles' LDS");

  int bh, mt;
  xcd_query_tile(blockIdx.x, total_wg, n_mtiles, CAUSAL, bh, mt);

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  const int half = lane / 32, l32 = lane % 32;
  const int64_t head_off = (int64_t)bh * N * D;
  const int q0 = mt * kBM;
  const int qrow = q0 + l32;

  float qreg[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qreg[s] = qrow < N ? Q[head_off + (int64_t)qrow * D + s * 2 + half] : 0.f;

  const int n_ktiles = (N + kBN - 1) / kBN;
  const int kt_end = CAUSAL ? min(n_ktiles, q0 / kBN + 1) : n_ktiles;   // kBM == kBN: tile mt is the diagonal
  static_assert(kBM == kBN, "the causal bound takes the diagonal tile as the query block's own");
  float* Ks = lds + wave * 2 * TILE;
  float* Vs = Ks + TILE;

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_part = 0.f;

  for (int kt = wave; kt < kt_end; kt += kW) {
    // this wave's tile into its own buffer; the wave's LDS operations complete in order,
    // so its reads below see all of it, and its next tile's writes follow these reads
    for (int idx = lane; idx < kBN * D; idx += 64) {
      const int r = idx / D, col = idx % D;
      const int key = kt * kBN + r;
      Ks[r * LD + col] = key < N ? K[head_off + (int64_t)key * D + col] : 0.f;
      Vs[r * LD + col] = key < N ? V[head_off + (int64_t)key * D + col] : 0.f;
    }

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
    // (every tile a wave takes has an unmasked key for each row below N: key 0 of the
    // tile, or for the diagonal tile the row's own key, so m_new is finite)
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

  // Merge: each wave publishes its row max, row sum and O partial (lane-major), wave 0
  // combines them. A wave without tiles for these rows publishes m = -inf, sum 0 and O 0,
  // which get the weight 2^-inf = 0 (wave 0 always has tile 0, so m is finite).
  const float l_tot = add_halves(l_part);
  __syncthreads();                             // every wave is done with its tile buffer
  float* mm = lds;                             // [wave][lane]
  float* ll = lds + kW * 64;                   // [wave][lane]
  float* oo = lds + 2 * kW * 64;               // [wave][value][lane]
  mm[wave * 64 + lane] = m_run;
  ll[wave * 64 + lane] = l_tot;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oo[(wave * NV + db * 16 + r) * 64 + lane] = oacc[db][r];
  __syncthreads();
  if (wave != 0 || qrow >= N) return;
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < kW; ++w) m = fmaxf(m, mm[w * 64 + lane]);
  float f[kW], l = 0.f;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    f[w] = fast_exp2((mm[w * 64 + lane] - m) * c);
    l = __builtin_fmaf(f[w], ll[w * 64 + lane], l);
  }
  const float inv = 1.0f / l;
  float* Orow = O + head_off + (int64_t)qrow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float o4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kW; ++w) acc = __builtin_fmaf(f[w], oo[(w * NV + db * 16 + g * 4 + e) * 64 + lane], acc);
        o4[e] = acc * inv;
      }
      *(f32x4*)(Orow + db * 32 + g * 8 + half * 4) = f32x4{o4[0], o4[1], o4[2], o4[3]};
    }
  if (half == 0) LSE[(int64_t)bh * N + qrow] = m * scale + __builtin_log2f(l) * kLn2;
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
