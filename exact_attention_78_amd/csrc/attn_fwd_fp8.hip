// fp8 (E4M3FN) exact attention forward on gfx950, head dim 128.
//
// Inputs are E4M3 codes with one fp32 scale per 128-row block of each (batch, head)
// ("8.3 FlashAttention-3", section 5.1: block quantisation; section 5: fp8 operands,
// fp32 accumulation). The tiling is the one of the 16-bit kernel (FlashAttention-2
// digest, framework-overview flowchart: online softmax over streamed K/V tiles, one
// final rescale, O and LSE written; split-Q waves; causal tiles above the diagonal
// skipped, masks only on diagonal / tail tiles).
//
// Per tile of 64 keys (inside one 128-row scale block of K and V):
//   S^T = K Q^T with v_mfma_f32_32x32x64_f8f6f4 on the raw codes; the block scales and
//   scale*log2(e) are one per-tile factor c_t = scale*log2e*sq*sk applied inside the
//   exp2 argument (the running max is kept in these log2 units).
//   P is produced as 2^8 * P, so that the row's largest probability (1) is exactly 256
//   in E4M3 and the smallest ones stay clear of the subnormal range; it is rounded to
//   E4M3 (v_cvt_pk_fp8_f32) and fed to the P.V MFMA against the raw V codes. The V block
//   scale is applied in fp32: the accumulator is kept in units of the current tile's V
//   scale, so moving to a tile with another scale multiplies it by the old/new ratio,
//   folded into the online-softmax rescale factor. The row sum l is accumulated from the
//   unrounded fp32 probabilities; the epilogue multiplies by the last V scale and
//   divides by l once.
//   V^T is gathered with ds_read_b64_tr_b8 (8-bit LDS transpose reads) in the key order
//   the S^T accumulators give P.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;
constexpr int kScaleRows = 128;
constexpr float kPShift = 8.0f;   // P enters the P.V MFMA as 2^8 * P

typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format 0 = E4M3 for both operands; E8M0 scale 127 = 2^0 (no block scaling in the MFMA)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 8-bit LDS transpose read: within a 16-lane group, lane i receives byte (i % 8) of the
// 8-byte segments addressed by lanes i/8 + 2j, j = 0..7 (result byte j).
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(p));
}

// 16-byte chunk c (of 8 per 128-byte row) of tile row r lives at chunk c ^ swz(r).
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_v(int r) { return (r >> 1) & 7; }

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ SQ, const float* __restrict__ SK, const float* __restrict__ SV,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_mtiles, int nblk, int total_wg, float c_base) {
  constexpr int NCH = kD / 16;                                  // 16-byte chunks per row (8)
  constexpr int TILE = kBN * kD;                                // bytes per K (or V) tile
  constexpr int CPT = kBN * NCH / kThreads;                     // chunks per thread per tile (2)
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][TILE];

  const int logical = xcd_logical_id(blockIdx.x, total_wg);
  const int bh = logical / n_mtiles;
  int mt = logical % n_mtiles;
  if (CAUSAL) mt = n_mtiles - 1 - mt;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int half = lane / 32, l32 = lane % 32;
  const int64_t head_off = (int64_t)bh * N * kD;
  const uint8_t* Qh = Q + head_off;
  const uint8_t* Kh = K + head_off;
  const uint8_t* Vh = V + head_off;
  const float* sk = SK + (int64_t)bh * nblk;
  const float* sv = SV + (int64_t)bh * nblk;

  const int q0 = mt * kBM + wave * 32;
  const int qrow = q0 + l32;
  const float cq = c_base * SQ[(int64_t)bh * nblk + mt];       // BM = 128: the tile is one Q scale block

  // Q^T as the B operand: for MFMA m (head-dim half), bytes [m*64 + half*32, +32) of the row.
  i32x8 qreg[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (qrow < N) {
      const i32x4 a = *(const i32x4*)(Qh + (int64_t)qrow * kD + m * 64 + half * 32);
      const i32x4 b = *(const i32x4*)(Qh + (int64_t)qrow * kD + m * 64 + half * 32 + 16);
      qreg[m] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
      qreg[m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  const int n_ktiles = (N + kBN - 1) / kBN;
  int kt_end = n_ktiles;
  if (CAUSAL) kt_end = min(n_ktiles, ((mt + 1) * kBM + kBN - 1) / kBN);
  const int wave_kt_end = CAUSAL ? min(kt_end, (q0 + 31) / kBN + 1) : kt_end;
  const bool wave_live = q0 < N;

  i32x4 kst[CPT], vst[CPT];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + i * kThreads;
      const int r = idx / NCH, ch = idx % NCH;
      const int key = kt * kBN + r;
      if (key < N) {
        kst[i] = *(const i32x4*)(Kh + (int64_t)key * kD + ch * 16);
        vst[i] = *(const i32x4*)(Vh + (int64_t)key * kD + ch * 16);
      } else {
        kst[i] = i32x4{0, 0, 0, 0};
        vst[i] = i32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int idx = tid + i * kThreads;
      const int r = idx / NCH, ch = idx % NCH;
      *(i32x4*)(&smem[buf][0][r * kD + ((ch ^ swz_k(r)) * 16)]) = kst[i];
      *(i32x4*)(&smem[buf][1][r * kD + ((ch ^ swz_v(r)) * 16)]) = vst[i];
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;   // running max in log2 units (score * scale * log2e)
  float l_part = 0.f;        // sum of 2^8 * P over this lane's half of the keys
  float sv_cur = 1.f;        // V scale whose units oacc is kept in

  // lane roles in the V transpose reads
  const int g16 = lane / 16, i16 = lane % 16;
  const int tr_h = g16 / 2;                       // key set (which half of the k-slots)
  const int tr_col = 16 * (g16 % 2) + 8 * (i16 & 1);
  const int tr_j = i16 >> 1;                      // slot j this lane addresses as a source

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < kt_end; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < kt_end) load_tile(kt + 1);

    if (wave_live && kt < wave_kt_end) {
      const uint8_t* Ks = smem[buf][0];
      const uint8_t* Vs = smem[buf][1];
      const int kblk = (kt * kBN) / kScaleRows;
      const float ct = cq * sk[kblk];
      const float svt = sv[kblk];

      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        const int r = kb * 32 + l32;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int c0 = m * 4 + half * 2;
          const i32x4 a0 = *(const i32x4*)(Ks + r * kD + ((c0 ^ swz_k(r)) * 16));
          const i32x4 a1 = *(const i32x4*)(Ks + r * kD + (((c0 + 1) ^ swz_k(r)) * 16));
          sacc[kb] = mfma_fp8(i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]}, qreg[m], sacc[kb]);
        }
      }
      const int key0 = kt * kBN;
      if ((CAUSAL && key0 + kBN - 1 > q0) || (key0 + kBN > N)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
            if ((CAUSAL && key > qrow) || key >= N) sacc[kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = max_halves(mx) * ct;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      const float oscale = alpha * (sv_cur / svt);
      sv_cur = svt;
      m_run = m_new;
      const float bias = m_new - kPShift;           // exp2 yields 2^8 * P
      float lsum = 0.f;
      int pb[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = fast_exp2(__builtin_fmaf(sacc[kb][q4 * 4 + e], ct, -bias));
            lsum += p[e];
          }
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
          pb[kb * 4 + q4] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
        }
      l_part = l_part * alpha + lsum;
      const i32x8 pop = i32x8{pb[0], pb[1], pb[2], pb[3], pb[4], pb[5], pb[6], pb[7]};
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        oacc[db] *= oscale;
        int av[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // slot 8m + j  <->  key (m/2)*32 + ((m%2)*2 + j/4)*8 + h*4 + j%4
          const int j = tr_j;
          const int row = (m / 2) * 32 + ((m % 2) * 2 + j / 4) * 8 + tr_h * 4 + (j % 4);
          const int col = db * 32 + tr_col;
          const i32x2 t = lds_read_tr8(Vs + row * kD + (((col >> 4) ^ swz_v(row)) << 4) + (col & 15));
          av[2 * m] = t[0];
          av[2 * m + 1] = t[1];
        }
        oacc[db] = mfma_fp8(i32x8{av[0], av[1], av[2], av[3], av[4], av[5], av[6], av[7]}, pop, oacc[db]);
      }
    }

    if (kt + 1 < kt_end) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_live || qrow >= N) return;
  const float l_tot = add_halves(l_part);
  const float inv = sv_cur / l_tot;
  uint16_t* Orow = O + head_off + (int64_t)qrow * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + half * 4;
      const f32x16 a = oacc[db];
      u32x2 w = {pack2(Bf16Tag{}, a[g * 4 + 0] * inv, a[g * 4 + 1] * inv),
                 pack2(Bf16Tag{}, a[g * 4 + 2] * inv, a[g * 4 + 3] * inv)};
      *(u32x2*)(Orow + d) = w;
    }
  if (half == 0) LSE[(int64_t)bh * N + qrow] = (m_run + __builtin_log2f(l_tot) - kPShift) * kLn2;
}

template <bool CAUSAL>
hipError_t launch(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* sq, const float* sk,
                  const float* sv, void* o, float* lse, int64_t BH, int64_t N, float scale, hipStream_t stream) {
  const int n_mtiles = (int)((N + kBM - 1) / kBM);
  const int nblk = (int)((N + kScaleRows - 1) / kScaleRows);
  const int64_t total = BH * n_mtiles;
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<CAUSAL>), dim3((unsigned)total), dim3(kThreads), 0, stream, q8, k8, v8, sq,
                     sk, sv, (uint16_t*)o, lse, (int)N, n_mtiles, nblk, (int)total, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* sq, const float* sk,
                          const float* sv, void* o, float* lse, int64_t BH, int64_t N, int64_t /*d*/, bool causal,
                          float scale, hipStream_t stream) {
  return causal ? launch<true>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, stream)
                : launch<false>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, stream);
}

int64_t max_workgroups_fwd8(int64_t BH, int64_t N) { return BH * ((N + kBM - 1) / kBM); }

}  // namespace attn
