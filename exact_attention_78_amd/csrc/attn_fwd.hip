// Exact attention forward for bf16 / fp16 on gfx950 (MI355X).
//
// Algorithm: FlashAttention-2 digest (irregular6612.github.io), framework-overview
// flowchart and key-components list — a workgroup per (batch*head, query tile); the
// query tile stays on chip while K/V tiles stream through an online softmax (running
// row max m and sum l); the 1/l rescale happens once at the end; O and one
// log-sum-exp per row are written. Work is split by query rows between waves (split-Q:
// every wave owns 32 query rows and reads the shared K/V tile, so waves never reduce
// across each other). Causal: key tiles wholly above the diagonal are never loaded;
// only tiles that cross the diagonal (or the end of the sequence) apply a mask.
// exp2-based softmax and fp32 accumulation follow "Triton 07: Flash Attention v3",
// Method. The 1D grid over (batch*head, m-tile) with neighbouring ids on the same head
// follows the same page's item 4, remapped so that each of the 8 XCDs walks its own
// contiguous range of heads (their K/V stay in that XCD's L2).
//
// gfx950 mapping (per wave, 32 query rows, key tile of BN = 64):
//   S^T = K Q^T   32x32x16 MFMAs: A = K rows from LDS (ds_read_b128), B = Q^T kept in
//                 VGPRs for the whole kernel. The result puts one query row per lane
//                 (lane l and l^32 share a row, each holding half of the keys), so the
//                 row max / row sum are in-lane plus one v_permlane32_swap.
//   O^T += V^T P^T  A = V^T via ds_read_b64_tr_b16 (LDS transpose read of row-major V),
//                 B = P rounded to 16 bits straight from the S^T accumulators. The key
//                 order inside each MFMA is permuted identically on both sides.
//   K/V tiles are double-buffered in LDS (2 x 32 KiB at d = 128) and the next tile's
//   global loads are in flight while the current tile is computed.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kBM = 128;      // query rows per workgroup
constexpr int kBN = 64;       // keys per tile
constexpr int kWaves = 4;     // 32 query rows per wave
constexpr int kThreads = kWaves * 64;
constexpr float kTau = 8.0f;  // lazy-rescale threshold for the running max, in log2 units

// LDS swizzles: 16-byte chunk c of tile row r is stored at chunk c ^ swz(r).
// K is read 32 rows x one chunk per instruction; V is read as 8 rows x 4 chunks
// (transpose reads), so the two tiles use different swizzles.
template <int D> struct Swz;
template <> struct Swz<128> {
  static __device__ __forceinline__ int k(int r) { return r & 15; }
  static __device__ __forceinline__ int v(int r) { return (r & 3) << 2; }
};
template <> struct Swz<64> {
  static __device__ __forceinline__ int k(int r) { return (r >> 1) & 7; }
  static __device__ __forceinline__ int v(int r) { return ((r >> 1) & 1) << 2; }
};

template <typename Tag, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_mtiles, int total_wg, float scale,
    float c /* scale * log2(e) */) {
  constexpr int NCH = D / 8;                        // 16-byte chunks per row
  constexpr int TILE = kBN * D;                     // elements per K (or V) tile
  constexpr int NSTEP = D / 16;                     // MFMA k-steps over the head dim
  constexpr int NKB = kBN / 32;                     // 32-key blocks per tile
  constexpr int NDB = D / 32;                       // 32-wide head-dim blocks of O
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][TILE];   // [buffer][K,V]

  const int logical = xcd_logical_id(blockIdx.x, total_wg);
  const int bh = logical / n_mtiles;
  int mt = logical % n_mtiles;
  if (CAUSAL) mt = n_mtiles - 1 - mt;               // longest query tiles first

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int half = lane / 32, l32 = lane % 32;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* Qh = Q + head_off;
  const uint16_t* Kh = K + head_off;
  const uint16_t* Vh = V + head_off;

  const int q0 = mt * kBM + wave * 32;              // first query row of this wave
  const int qrow = q0 + l32;                        // the query row this lane holds

  // Q^T as the B operand, resident for the whole kernel.
  u32x4 qreg[NSTEP];
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    if (qrow < N)
      qreg[s] = *(const u32x4*)(Qh + (int64_t)qrow * D + s * 16 + half * 8);
    else
      qreg[s] = u32x4{0, 0, 0, 0};
  }

  const int n_ktiles = (N + kBN - 1) / kBN;
  int kt_end = n_ktiles;
  if (CAUSAL) kt_end = min(n_ktiles, ((mt + 1) * kBM + kBN - 1) / kBN);
  // last key tile this wave needs (causal: its last row's diagonal)
  const int wave_kt_end = CAUSAL ? min(kt_end, (q0 + 31) / kBN + 1) : kt_end;
  const bool wave_live = q0 < N;

  // Direct global -> LDS loads of one K/V tile (global_load_lds_dwordx4: no VGPR staging).
  // Each wave instruction fills 1 KiB of LDS, 16 bytes per lane at consecutive addresses;
  // the lane therefore fetches the global chunk that the swizzle places at its slot.
  // Rows past the end of the sequence re-read the last row: their scores are masked and
  // their probabilities are zero, so any finite data will do.
  constexpr int ROW_BYTES = D * 2;
  constexpr int LOADS_PER_WAVE = TILE * 2 / 1024 / kWaves;
  auto issue_tile_loads = [&](int kt, int buf) {
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      const int slot = (wave * LOADS_PER_WAVE + i) * 1024 + lane * 16;   // byte offset in the tile
      const int r = slot / ROW_BYTES, phys = (slot % ROW_BYTES) / 16;
      const int key = min(kt * kBN + r, N - 1);
      const int64_t goff = (int64_t)key * D;
      const uint16_t* gk = Kh + goff + ((phys ^ Swz<D>::k(r)) * 8);
      const uint16_t* gv = Vh + goff + ((phys ^ Swz<D>::v(r)) * 8);
      uint16_t* lk = &smem[buf][0][(wave * LOADS_PER_WAVE + i) * 512];
      uint16_t* lv = &smem[buf][1][(wave * LOADS_PER_WAVE + i) * 512];
      __builtin_amdgcn_global_load_lds((const void*)gk, (__attribute__((address_space(3))) void*)lk, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)gv, (__attribute__((address_space(3))) void*)lv, 16, 0, 0);
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  // Running max in log2 units (score * scale * log2 e). It is raised only when a tile's
  // max exceeds it by more than kTau, so most tiles skip the O rescale; probabilities are
  // then bounded by 2^kTau, which bf16/fp16 P and the fp32 sums hold exactly as well.
  float M = -INFINITY;
  float l_part = 0.f;        // running sum over this lane's half of the keys

  // Lane roles in the V transpose reads.
  const int g16 = lane / 16, i16 = lane % 16;
  const int tr_row = (g16 / 2) * 4 + i16 / 4;          // + kb*32 + t*16 (+8)
  const int tr_col = 16 * (g16 % 2) + 4 * (i16 % 4);   // + db*32

  issue_tile_loads(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int kt = 0; kt < kt_end; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < kt_end) issue_tile_loads(kt + 1, buf ^ 1);

    if (wave_live && kt < wave_kt_end) {
      const uint16_t* Ks = smem[buf][0];
      const uint16_t* Vs = smem[buf][1];
      // ---- S^T = K Q^T
      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sacc[kb] = f32x16{};
        const int r = kb * 32 + l32;
#pragma unroll
        for (int s = 0; s < NSTEP; ++s) {
          const int ch = s * 2 + half;
          const u32x4 a = *(const u32x4*)(Ks + r * D + ((ch ^ Swz<D>::k(r)) * 8));
          sacc[kb] = mfma32(Tag{}, a, qreg[s], sacc[kb]);
        }
      }
      // ---- mask (diagonal tiles and the sequence tail only)
      const int key0 = kt * kBN;
      const bool need_mask = (CAUSAL && key0 + kBN - 1 > q0) || (key0 + kBN > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
            const bool masked = (CAUSAL && key > qrow) || key >= N;
            if (masked) sacc[kb][r] = -INFINITY;
          }
      }
      // ---- online softmax (exp2, lazily raised running max, deferred normalisation)
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = max_halves(mx) * c;
      if (__builtin_amdgcn_ballot_w64(mx > M + kTau) != 0) {
        const float M_new = fmaxf(M, mx);
        const float alpha = fast_exp2(M - M_new);
        M = M_new;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      }
      float lsum = 0.f;
      u32x4 pk[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(__builtin_fmaf(sacc[kb][r], c, -M));
          lsum += p[r];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
          pk[kb][t] = u32x4{pack2(Tag{}, p[t * 8 + 0], p[t * 8 + 1]), pack2(Tag{}, p[t * 8 + 2], p[t * 8 + 3]),
                            pack2(Tag{}, p[t * 8 + 4], p[t * 8 + 5]), pack2(Tag{}, p[t * 8 + 6], p[t * 8 + 7])};
      }
      l_part += lsum;
      // ---- O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int row1 = kb * 32 + t * 16 + tr_row;
            const int row2 = row1 + 8;
            const int col = db * 32 + tr_col;
            const u32x2 v1 = lds_read_tr16(Vs + row1 * D + (((col >> 3) ^ Swz<D>::v(row1)) << 3) + (col & 7));
            const u32x2 v2 = lds_read_tr16(Vs + row2 * D + (((col >> 3) ^ Swz<D>::v(row2)) << 3) + (col & 7));
            const u32x4 a = u32x4{v1[0], v1[1], v2[0], v2[1]};
            oacc[db] = mfma32(Tag{}, a, pk[kb][t], oacc[db]);
          }
        }
      }
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  if (!wave_live || qrow >= N) return;
  // ---- epilogue: one division per row, O and LSE
  const float l_tot = add_halves(l_part);
  const float inv = 1.0f / l_tot;
  uint16_t* Orow = O + head_off + (int64_t)qrow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + half * 4;
      const f32x16 a = oacc[db];
      u32x2 w = {pack2(Tag{}, a[g * 4 + 0] * inv, a[g * 4 + 1] * inv), pack2(Tag{}, a[g * 4 + 2] * inv, a[g * 4 + 3] * inv)};
      *(u32x2*)(Orow + d) = w;
    }
  if (half == 0) LSE[(int64_t)bh * N + qrow] = (M + __builtin_log2f(l_tot)) * kLn2;
}

template <typename Tag, int D, bool CAUSAL>
hipError_t launch_one(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                      float scale, hipStream_t stream) {
  const int n_mtiles = (int)((N + kBM - 1) / kBM);
  const int64_t total = BH * n_mtiles;
  hipLaunchKernelGGL((attn_fwd_kernel<Tag, D, CAUSAL>), dim3((unsigned)total), dim3(kThreads), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, (int)N, n_mtiles,
                     (int)total, scale, scale * kLog2e);
  return hipGetLastError();
}

template <typename Tag>
hipError_t launch_16bit(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                        int64_t d, bool causal, float scale, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_one<Tag, 128, true>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch_one<Tag, 128, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch_one<Tag, 64, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch_one<Tag, 64, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                           int64_t d, bool causal, float scale, hipStream_t stream) {
  return launch_16bit<Bf16Tag>(q, k, v, o, lse, BH, N, d, causal, scale, stream);
}

hipError_t launch_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                          int64_t d, bool causal, float scale, hipStream_t stream) {
  return launch_16bit<F16Tag>(q, k, v, o, lse, BH, N, d, causal, scale, stream);
}

int64_t max_workgroups_fwd16(int64_t BH, int64_t N) { return BH * ((N + kBM - 1) / kBM); }

}  // namespace attn
