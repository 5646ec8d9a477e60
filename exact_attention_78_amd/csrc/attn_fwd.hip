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
// gfx950 mapping: 8 waves x 32 query rows per workgroup (two waves per SIMD), key tiles
// of BN = 64:
//   S^T = K Q^T   32x32x16 MFMAs: A = K rows from LDS (ds_read_b128), B = Q^T kept in
//                 VGPRs for the whole kernel. The result puts one query row per lane
//                 (lane l and l^32 share a row, each holding half of the keys), so the
//                 row max / row sum are in-lane plus one v_permlane32_swap.
//   O^T += V^T P^T  A = V^T via ds_read_b64_tr_b16 (LDS transpose read of row-major V),
//                 B = P rounded to 16 bits straight from the S^T accumulators. The key
//                 order inside each MFMA is permuted identically on both sides.
//   The S^T MFMAs of tile t+1 are issued in the same block as the softmax of tile t, so
//   the matrix core works while the VALU computes exponentials (the intra-warpgroup
//   overlap of "8.3 FlashAttention-3", section 4, inside one wave).
//   K/V tiles sit in a 3-slot LDS ring (3 x 32 KiB at d = 128), filled by direct
//   global->LDS loads (global_load_lds_dwordx4) two steps ahead of their use.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

#ifndef ATTN_WAVES
#define ATTN_WAVES 8
#endif
#ifndef ATTN_ROW_BLOCKS
#define ATTN_ROW_BLOCKS 1
#endif
constexpr int kBN = 64;                    // keys per tile
constexpr int kWaves = ATTN_WAVES;         // waves per workgroup
constexpr int kRowBlocks = ATTN_ROW_BLOCKS;  // 32-row query blocks per wave
#ifndef ATTN_PIPE
#define ATTN_PIPE 1
#endif
constexpr bool kPipe = ATTN_PIPE;          // issue S^T of tile t+1 alongside the softmax of tile t
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

// Wait until at most N vector-memory loads of this wave are outstanding.
// (s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at
// their maxima; the builtin keeps the compiler's own counter tracking informed.)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS hand-over only: LDS reads of this wave are complete, then
// s_barrier. Unlike __syncthreads() it does not drain this wave's outstanding global
// loads, so a load for a later tile can stay in flight across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename Tag, int D, bool CAUSAL, int W, int RB, bool PIPE>
__global__ __launch_bounds__(W * 64, 1) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_mtiles, int total_wg, float c /* scale*log2 e */) {
  constexpr int BM = W * RB * 32;                   // query rows per workgroup
  constexpr int NSTEP = D / 16;                     // MFMA k-steps over the head dim
  constexpr int NKB = kBN / 32;                     // 32-key blocks per tile
  constexpr int NDB = D / 32;                       // 32-wide head-dim blocks of O
  constexpr int ROW = D * 2;                        // bytes per K/V row
  constexpr int TB = kBN * ROW;                     // bytes per K (or V) tile
  constexpr int LPW = TB / 1024 / W;                // 1 KiB direct loads per wave per tile
  static_assert(LPW >= 1 && LPW * 1024 * W == TB, "tile must split into whole 1 KiB loads per wave");
  // LDS: three K and three V tiles (a ring: tile t lives in buffer t % 3), as six separate
  // objects so that the compiler can tell the direct loads into one buffer from the reads
  // of another (no needless vmcnt waits).
  __shared__ __attribute__((aligned(16))) uint8_t lds_k0[TB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_k1[TB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_k2[TB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v0[TB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v1[TB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v2[TB];

  const int logical = xcd_logical_id(blockIdx.x, total_wg);
  const int bh = logical / n_mtiles;
  int mt = logical % n_mtiles;
  if (CAUSAL) mt = n_mtiles - 1 - mt;               // longest query tiles first

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // wave-uniform: lives in an SGPR
  const int lane = tid % 64;
  const int half = lane / 32, l32 = lane % 32;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* Qh = Q + head_off;
  const uint16_t* Kh = K + head_off;
  const uint16_t* Vh = V + head_off;

  // This wave owns RB blocks of 32 query rows; each lane holds one row of each block.
  const int q0 = mt * BM + wave * RB * 32;
  int qrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) qrow[rb] = q0 + rb * 32 + l32;

  // Q^T as the B operand, resident for the whole kernel.
  u32x4 qreg[RB][NSTEP];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int s = 0; s < NSTEP; ++s)
      qreg[rb][s] = qrow[rb] < N ? *(const u32x4*)(Qh + (int64_t)qrow[rb] * D + s * 16 + half * 8)
                                 : u32x4{0, 0, 0, 0};

  const int n_ktiles = (N + kBN - 1) / kBN;
  const int T = CAUSAL ? min(n_ktiles, ((mt + 1) * BM + kBN - 1) / kBN) : n_ktiles;

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
  auto buf = [&](auto IDX) __attribute__((always_inline)) -> uint8_t* {       // 0..2: K ring, 3..5: V ring
    constexpr int i = decltype(IDX)::value;
    if constexpr (i == 0) return lds_k0;
    else if constexpr (i == 1) return lds_k1;
    else if constexpr (i == 2) return lds_k2;
    else if constexpr (i == 3) return lds_v0;
    else if constexpr (i == 4) return lds_v1;
    else return lds_v2;
  };
  // Full tiles: a uniform tile base plus a per-lane 32-bit byte offset (no per-lane 64-bit
  // address arithmetic). The tile that crosses the end of the sequence clamps rows.
  int ld_koff[LPW], ld_voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    ld_koff[i] = (ld_row[i] * D + ld_kch[i]) * 2;
    ld_voff[i] = (ld_row[i] * D + ld_vch[i]) * 2;
  }
  auto load_tile = [&](const uint16_t* src, const int (&off)[LPW], const int (&ch)[LPW], int kt, uint8_t* dst) __attribute__((always_inline)) {
    if (kt * kBN + kBN <= N) {
      const uint8_t* base = (const uint8_t*)(src + (int64_t)kt * kBN * D);
#pragma unroll
      for (int i = 0; i < LPW; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(base + off[i]),
                                         (__attribute__((address_space(3))) void*)(dst + (wave * LPW + i) * 1024), 16,
                                         0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int key = min(kt * kBN + ld_row[i], N - 1);
        __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)key * D + ch[i]),
                                         (__attribute__((address_space(3))) void*)(dst + (wave * LPW + i) * 1024), 16,
                                         0, 0);
      }
    }
  };
  auto load_k = [&](int kt, auto OFF) __attribute__((always_inline)) { load_tile(Kh, ld_koff, ld_kch, kt, buf(OFF)); };
  auto load_v = [&](int kt, auto OFF) __attribute__((always_inline)) { load_tile(Vh, ld_voff, ld_vch, kt, buf(OFF)); };

  // ---- S^T = K Q^T from the K tile in ring slot OFF; each K fragment feeds every row block
  auto qk = [&](auto OFF, f32x16 (&sacc)[RB][NKB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[rb][kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        const u32x4 a = *(const u32x4*)(buf(OFF) + kb * 32 * ROW + kaddr[s]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) sacc[rb][kb] = mfma32(Tag{}, a, qreg[rb][s], sacc[rb][kb]);
      }
    }
  };

  f32x16 oacc[RB][NDB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[rb][db] = f32x16{};
  // Running max in log2 units (score * scale * log2 e). It is raised only when a tile's
  // max exceeds it by more than kTau, so most tiles skip the O rescale; probabilities are
  // then bounded by 2^kTau, which bf16/fp16 P and the fp32 sums hold exactly as well.
  float M[RB], l_part[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    M[rb] = -INFINITY;
    l_part[rb] = 0.f;        // running sum over this lane's half of the keys
  }

  // ---- one pipelined step: softmax + P.V of tile t (scores in S, V in ring slot t % 3)
  // while the S^T MFMAs of tile t+1 (K in slot (t+1) % 3) are issued. Loads of V for
  // tile t+2 and K for tile t+3 go out at the start of the step; each has two steps to
  // land, so the wait at the end of the step leaves this step's loads in flight. Near
  // the end the tile index is clamped: a slot past the last tile is refilled with the
  // last tile and never read, which keeps the number of loads per step fixed.
  f32x16 Sa[RB][NKB], Sb[RB][NKB];
  auto step = [&](int t, f32x16 (&S)[RB][NKB], f32x16 (&Sn)[RB][NKB], auto KNEXT, auto KLOAD, auto VOFF,
                  auto VLOAD) __attribute__((always_inline)) {
    load_v(min(t + 2, T - 1), VLOAD);
    load_k(min(t + 3, T - 1), KLOAD);
    const int key0 = t * kBN;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if ((CAUSAL && key0 + kBN - 1 > q0 + rb * 32) || key0 + kBN > N) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
            if ((CAUSAL && key > qrow[rb]) || key >= N) S[rb][kb][r] = -INFINITY;
          }
      }
    }
    float mx[RB];
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // four independent max chains (v_max3), then combined: short dependency chains
      float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) m4[(r / 2) % 4] = fmaxf(m4[(r / 2) % 4], fmaxf(S[rb][kb][r], S[rb][kb][r + 1]));
      mx[rb] = max_halves(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]))) * c;
      grow |= mx[rb] > M[rb] + kTau;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float M_new = fmaxf(M[rb], mx[rb]);
        const float alpha = fast_exp2(M[rb] - M_new);
        M[rb] = M_new;
        l_part[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[rb][db] *= alpha;
      }
    }
    if constexpr (PIPE) qk(KNEXT, Sn);   // independent of the softmax below: the MFMAs overlap its VALU work
    u32x4 pk[RB][NKB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(__builtin_fmaf(S[rb][kb][r], c, -M[rb]));
          lsum += p[r];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
          pk[rb][kb][h] = u32x4{pack2(Tag{}, p[h * 8 + 0], p[h * 8 + 1]), pack2(Tag{}, p[h * 8 + 2], p[h * 8 + 3]),
                                pack2(Tag{}, p[h * 8 + 4], p[h * 8 + 5]), pack2(Tag{}, p[h * 8 + 6], p[h * 8 + 7])};
      }
      l_part[rb] += lsum;
    }
    // O^T += V^T P^T; each V fragment feeds every row block
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint8_t* base = buf(VOFF) + (kb * 32 + h * 16) * ROW + vaddr[db];
          const u32x2 v1 = lds_read_tr16((const uint16_t*)base);
          const u32x2 v2 = lds_read_tr16((const uint16_t*)(base + 8 * ROW));
          const u32x4 a = u32x4{v1[0], v1[1], v2[0], v2[1]};
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = mfma32(Tag{}, a, pk[rb][kb][h], oacc[rb][db]);
        }
    if constexpr (!PIPE) qk(KNEXT, Sn);  // scores of tile t+1, once P of tile t no longer needs S
    wait_vmcnt<2 * LPW>();   // tiles t+1 (V) and t+2 (K), issued a step earlier, have landed
    barrier_lds();
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;

  load_k(0, I0{});
  load_v(0, I3{});
  if (T > 1) load_k(1, I1{});
  if (T > 1) load_v(1, I4{});
  if (T > 2) load_k(2, I2{});
  wait_vmcnt<0>();
  barrier_lds();
  qk(I0{}, Sa);
  barrier_lds();                                     // K slot 0 is refilled with tile 3 next

  // Six steps per trip: ring slots repeat every 3 tiles, score registers every 2.
  for (int t = 0; t < T; t += 6) {
    step(t, Sa, Sb, I1{}, I0{}, I3{}, I5{});
    if (t + 1 < T) step(t + 1, Sb, Sa, I2{}, I1{}, I4{}, I3{});
    if (t + 2 < T) step(t + 2, Sa, Sb, I0{}, I2{}, I5{}, I4{});
    if (t + 3 < T) step(t + 3, Sb, Sa, I1{}, I0{}, I3{}, I5{});
    if (t + 4 < T) step(t + 4, Sa, Sb, I2{}, I1{}, I4{}, I3{});
    if (t + 5 < T) step(t + 5, Sb, Sa, I0{}, I2{}, I5{}, I4{});
  }
  wait_vmcnt<0>();           // no load may still target this workgroup's LDS when it exits

  // ---- epilogue: one division per row, O and LSE
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = add_halves(l_part[rb]);
    if (qrow[rb] >= N) continue;
    const float inv = 1.0f / l_tot;
    uint16_t* Orow = O + head_off + (int64_t)qrow[rb] * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + g * 8 + half * 4;
        const f32x16 a = oacc[rb][db];
        u32x2 w = {pack2(Tag{}, a[g * 4 + 0] * inv, a[g * 4 + 1] * inv),
                   pack2(Tag{}, a[g * 4 + 2] * inv, a[g * 4 + 3] * inv)};
        *(u32x2*)(Orow + d) = w;
      }
    if (half == 0) LSE[(int64_t)bh * N + qrow[rb]] = (M[rb] + __builtin_log2f(l_tot)) * kLn2;
  }
}

// Launch shape per head dim: waves per workgroup and 32-row blocks per wave.
template <int D> struct Cfg;
template <> struct Cfg<128> { static constexpr int W = kWaves, RB = kRowBlocks; static constexpr bool PIPE = kPipe; };
template <> struct Cfg<64> { static constexpr int W = kWaves, RB = kRowBlocks; static constexpr bool PIPE = kPipe; };

template <typename Tag, int D, bool CAUSAL>
hipError_t launch_one(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                      float scale, hipStream_t stream) {
  constexpr int W = Cfg<D>::W, RB = Cfg<D>::RB, BM = W * RB * 32;
  constexpr bool PIPE = Cfg<D>::PIPE;
  const int n_mtiles = (int)((N + BM - 1) / BM);
  const int64_t total = BH * n_mtiles;
  hipLaunchKernelGGL((attn_fwd_kernel<Tag, D, CAUSAL, W, RB, PIPE>), dim3((unsigned)total), dim3(W * 64), 0, stream,
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

int64_t max_workgroups_fwd16(int64_t BH, int64_t N) {
  constexpr int BM = kWaves * kRowBlocks * 32;   // the smallest tile of any head dim
  return BH * ((N + BM - 1) / BM);
}

}  // namespace attn
