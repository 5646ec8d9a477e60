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
#include <type_traits>

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
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_mtiles, int total_wg, float c /* scale*log2 e */) {
  constexpr int NSTEP = D / 16;                     // MFMA k-steps over the head dim
  constexpr int NKB = kBN / 32;                     // 32-key blocks per tile
  constexpr int NDB = D / 32;                       // 32-wide head-dim blocks of O
  constexpr int ROW = D * 2;                        // bytes per K/V row
  constexpr int TB = kBN * ROW;                     // bytes per K (or V) tile
  constexpr int LPW = TB / 1024 / kWaves;           // 1 KiB direct loads per wave per tile
  // LDS: two K and two V tiles, as four separate objects so that the compiler can tell
  // the direct loads into one buffer from the reads of another (no needless vmcnt waits).
  __shared__ __attribute__((aligned(16))) uint8_t lds_k0[TB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_k1[TB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v0[TB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v1[TB];

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
  for (int s = 0; s < NSTEP; ++s)
    qreg[s] = qrow < N ? *(const u32x4*)(Qh + (int64_t)qrow * D + s * 16 + half * 8) : u32x4{0, 0, 0, 0};

  const int n_ktiles = (N + kBN - 1) / kBN;
  const int T = CAUSAL ? min(n_ktiles, ((mt + 1) * kBM + kBN - 1) / kBN) : n_ktiles;

  // ---- per-lane LDS byte addresses (buffer and row-block offsets are immediates)
  uint32_t kaddr[NSTEP];
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) kaddr[s] = l32 * ROW + (((2 * s + half) ^ Swz<D>::k(l32)) << 4);
  const int g16 = lane / 16, i16 = lane % 16;
  const int tr_row = (g16 / 2) * 4 + i16 / 4;          // + kb*32 + t*16 (+8)
  const int tr_col = 16 * (g16 % 2) + 4 * (i16 % 4);   // + db*32
  uint32_t vaddr[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int col = db * 32 + tr_col;
    vaddr[db] = tr_row * ROW + ((((col >> 3) ^ Swz<D>::v(tr_row))) << 4) + ((col & 7) << 1);
  }

  // ---- direct global -> LDS loads (global_load_lds_dwordx4, no VGPR staging). Each wave
  // instruction fills 1 KiB of LDS, 16 bytes per lane at consecutive addresses, so a lane
  // fetches the global chunk the swizzle places at its slot. Rows past the end of the
  // sequence re-read the last row: their scores are masked and their probabilities are 0.
  int ld_row[LPW], ld_kch[LPW], ld_vch[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int slot = (wave * LPW + i) * 1024 + lane * 16;
    const int r = slot / ROW, phys = (slot % ROW) / 16;
    ld_row[i] = r;
    ld_kch[i] = (phys ^ Swz<D>::k(r)) * 8;
    ld_vch[i] = (phys ^ Swz<D>::v(r)) * 8;
  }
  auto buf = [&](auto IDX) -> uint8_t* {
    constexpr int i = decltype(IDX)::value;
    if constexpr (i == 0) return lds_k0;
    else if constexpr (i == 1) return lds_k1;
    else if constexpr (i == 2) return lds_v0;
    else return lds_v1;
  };
  auto load_k = [&](int kt, auto OFF) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int key = min(kt * kBN + ld_row[i], N - 1);
      __builtin_amdgcn_global_load_lds((const void*)(Kh + (int64_t)key * D + ld_kch[i]),
                                       (__attribute__((address_space(3))) void*)(buf(OFF) + (wave * LPW + i) * 1024),
                                       16, 0, 0);
    }
  };
  auto load_v = [&](int kt, auto OFF) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int key = min(kt * kBN + ld_row[i], N - 1);
      __builtin_amdgcn_global_load_lds((const void*)(Vh + (int64_t)key * D + ld_vch[i]),
                                       (__attribute__((address_space(3))) void*)(buf(OFF) + (wave * LPW + i) * 1024),
                                       16, 0, 0);
    }
  };

  // ---- S^T = K Q^T from the K tile at byte offset OFF
  auto qk = [&](auto OFF, f32x16 (&sacc)[NKB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        const u32x4 a = *(const u32x4*)(buf(OFF) + kb * 32 * ROW + kaddr[s]);
        sacc[kb] = mfma32(Tag{}, a, qreg[s], sacc[kb]);
      }
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

  // ---- one pipelined step: softmax + P.V of tile t (held in S, V tile at VOFF) while the
  // MFMAs of S^T for tile t+1 (K tile at KNEXT) are issued; loads for tiles t+2 (K, into
  // KLOAD) and t+1 (V, into VLOAD) are in flight.
  f32x16 Sa[NKB], Sb[NKB];
  auto step = [&](int t, f32x16 (&S)[NKB], f32x16 (&Sn)[NKB], auto KNEXT, auto KLOAD, auto VOFF, auto VLOAD) {
    if (t + 2 < T) load_k(t + 2, KLOAD);
    if (t + 1 < T) load_v(t + 1, VLOAD);
    const int key0 = t * kBN;
    if ((CAUSAL && key0 + kBN - 1 > q0) || key0 + kBN > N) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
          if ((CAUSAL && key > qrow) || key >= N) S[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
    mx = max_halves(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mx > M + kTau) != 0) {
      const float M_new = fmaxf(M, mx);
      const float alpha = fast_exp2(M - M_new);
      M = M_new;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    qk(KNEXT, Sn);           // independent of the softmax below: the MFMAs overlap its VALU work
    float lsum = 0.f;
    u32x4 pk[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(__builtin_fmaf(S[kb][r], c, -M));
        lsum += p[r];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
        pk[kb][h] = u32x4{pack2(Tag{}, p[h * 8 + 0], p[h * 8 + 1]), pack2(Tag{}, p[h * 8 + 2], p[h * 8 + 3]),
                          pack2(Tag{}, p[h * 8 + 4], p[h * 8 + 5]), pack2(Tag{}, p[h * 8 + 6], p[h * 8 + 7])};
    }
    l_part += lsum;
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint8_t* base = buf(VOFF) + (kb * 32 + h * 16) * ROW + vaddr[db];
          const u32x2 v1 = lds_read_tr16((const uint16_t*)base);
          const u32x2 v2 = lds_read_tr16((const uint16_t*)(base + 8 * ROW));
          oacc[db] = mfma32(Tag{}, u32x4{v1[0], v1[1], v2[0], v2[1]}, pk[kb][h], oacc[db]);
        }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using V0 = std::integral_constant<int, 2>;
  using V1 = std::integral_constant<int, 3>;

  load_k(0, K0{});
  load_v(0, V0{});
  if (T > 1) load_k(1, K1{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  qk(K0{}, Sa);
  __syncthreads();                                   // K0 is refilled with tile 2 next

  for (int t = 0; t < T; t += 2) {
    // even tile t: its scores in Sa, its V in V0; S^T of t+1 from K1 into Sb
    step(t, Sa, Sb, K1{}, K0{}, V0{}, V1{});
    if (t + 1 < T) step(t + 1, Sb, Sa, K0{}, K1{}, V1{}, V0{});
  }

  if (qrow >= N) return;
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
                     (int)total, scale * kLog2e);
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
