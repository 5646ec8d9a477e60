// fp8 (E4M3FN) exact attention forward on gfx950, head dim 64 or 128.
//
// Inputs are E4M3 codes with one fp32 scale per 128-row block of each (batch, head)
// ("8.3 FlashAttention-3", section 5.1: block quantisation; section 5: fp8 operands,
// fp32 accumulation). The tiling and pipeline are those of the 16-bit kernel
// (FlashAttention-2 digest, framework-overview flowchart: online softmax over streamed
// K/V tiles, one final rescale, O and LSE written; split-Q waves of 32 rows, 8 waves per
// workgroup; causal tiles above the diagonal skipped, masks only on diagonal / tail
// tiles; step t issues P.V of tile t, the softmax of tile t+1 and S^T of tile t+2, with
// MFMAs, LDS reads and VALU work written in the intended issue order, which the machine
// scheduler then refines: unlike the 16-bit kernel, this one is 4% faster with it).
//
// Per tile of 64 keys (inside one 128-row scale block of K and V):
//   S^T = K Q^T with v_mfma_scale_f32_32x32x64_f8f6f4 on the raw codes (two per 32 keys);
//   the block scales and scale*log2(e) form one factor c_t = scale*log2e*sq*sk applied
//   inside the exp2 argument (the running max M is kept in these log2 units).
//   P enters the P.V MFMA as E4M3 codes of P'' = P' / w with P' = 2^kPShift * 2^(s - M)
//   and w = U / sv[block]: the P.V accumulator is kept in a unit U (a V block scale) and
//   the ratio of the tile's V block scale to U rides in the exp2 argument (a per-tile
//   bias), so the accumulator is not rescaled when the tiles enter the next V block. U
//   moves, lazily like the running max, only when that ratio leaves [1, 3/2] (U then
//   follows the smallest V block scale seen, and moves only a few times along a row of
//   blocks whose scales vary little); the accumulator is then rescaled once. With w <= 1,
//   P'' is never below P' = 2^kPShift * 2^(s - M), so probabilities down to 2^-15 of the
//   max stay representable, and as the running max is raised by more than kTau only,
//   P'' <= 1.5 * 2^(kPShift+kTau) = 384 stays below the E4M3 maximum (448).
//   O is normalised by the sum of the *rounded* P'' codes times w: one more MFMA per tile
//   (the 16x16x128 form, half the cycles of the others) sums the tile's codes exactly in
//   fp32, and that sum times the tile's w is added to the denominator. Its A operand is
//   E4M3 1.0 in a pattern of lanes that makes each lane's output the sum for its own
//   query row (see the construction of `ones`). Numerator and denominator
//   then use the same weights, so a row dominated by one key returns that key's V row
//   however P'' rounds. The LSE uses the sum of the unrounded fp32 probabilities.
//   V^T is gathered with ds_read_b64_tr_b8 (8-bit LDS transpose reads) in the key order
//   the S^T accumulators give P.
#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kBN = 64;
constexpr int kWaves = 8;
constexpr int kBM = kWaves * 32;
constexpr int kScaleRows = 128;
constexpr float kPShift = 6.0f;   // P' = 2^6 * P
constexpr float kTau = 2.0f;      // lazy-rescale threshold (log2 units): P' <= 2^(6+2) = 256
static_assert(kScaleRows % kBN == 0 && kBM % kScaleRows == 0, "tiles nest inside scale blocks");

typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format 0 = E4M3 for both operands; E8M0 scale 127 = 2^0 (no block scaling in the MFMA)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// The 16x16x128 form of the same instruction (half the cycles of the 32x32x64 form):
// lane l holds A row l%16 and B column l%16 over the same block l/16 of k, and receives
// C rows 4*(l/16) .. 4*(l/16)+3 of column l%16.
__device__ __forceinline__ f32x4 mfma_fp8_16(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 8-bit LDS transpose read: within a 16-lane group, lane i receives byte (i % 8) of the
// 8-byte segments addressed by lanes i/8 + 2j, j = 0..7 (result byte j).
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(p));
}

// 16-byte chunk c (of D/16 per row of D bytes) of tile row r lives at chunk c ^ swz(r); K
// and V tiles use the same swizzle, a function of row bits 1..3 only (row offsets that are
// multiples of 16 keep it). d = 128: two 128-byte rows share a 256-byte line of the 64
// LDS banks, so a 16-byte bank group is (r & 1) * 8 + (c ^ swz(r)) (mod 16). The K reads
// (one 16-byte chunk per lane from 16 consecutive rows) need swz to take 8 distinct values
// on the even rows and on the odd rows of 16; the V^T transpose reads (32 lanes: rows
// {0,1,2,3,8,9,10,11} + 4h, chunks c and c^1) need swz >> 1 to differ between the rows
// {0,2,8,10} (and {1,3,9,11}, {4,6,12,14}, {5,7,13,15}). Swapping bit 1 of the row to the
// top does both: swz = 4 * r[1] + r[3:2]. (Using r[3:1] directly put rows 0 and 2, 8 and
// 10 on one bank group for the V^T reads: 2-way conflicts, 33% of LDS cycles.)
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  return (r >> 1) & (D / 16 - 1);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

// Q preparation fused into the attention kernel ("8.3 FlashAttention-3", section 5.2: the
// rotation is folded into the kernel's own preprocessing): this lane's D/2 elements of its
// query row, rotated (signs, fast Walsh-Hadamard butterfly, 1/sqrt(d)) and quantised with
// the scale of the row's 128-row block into the B operand of S^T = K Q^T. The lane holds
// elements m*64 + half*32 + j (m < D/64; j = 0..31), the bytes of qreg[m]. Every value
// is rounded as attn_quant_fp8 rounds it (the butterfly's stages in order, spans 1..64,
// each output one rounded add or subtract; one fp32 multiply by 1/sqrt(d); amax/448; the
// correctly rounded x/scale; clamp; E4M3 round to nearest even), so the codes and scales
// equal that kernel's (spans 1..16 inside the lane, 32 across the lane pair l, l^32, 64
// inside the lane). Returns the block's scale; `blk_max` is LDS for one float per wave.
template <int D>
__device__ __forceinline__ float fused_q_prep(const uint16_t* __restrict__ Qr, bool valid,
                                              const float* __restrict__ signs, float inv_sqrt_d, int half,
                                              int wave, int lane, float* blk_max, i32x8 (&qreg)[D / 64]) {
  constexpr int NM = D / 64;                           // 64-element groups per row (MFMA k-steps)
  float x[NM * 32];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e0 = m * 64 + half * 32 + i * 8;
      const u32x4 raw = valid ? *(const u32x4*)(Qr + e0) : u32x4{0, 0, 0, 0};
      const f32x4 s0 = *(const f32x4*)(signs + e0), s1 = *(const f32x4*)(signs + e0 + 4);
      const float sg[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[m * 32 + i * 8 + 2 * e] = bf16_bits_to_f32(raw[e] & 0xFFFFu) * sg[2 * e];     // exact (+-1)
        x[m * 32 + i * 8 + 2 * e + 1] = bf16_bits_to_f32(raw[e] >> 16) * sg[2 * e + 1];
      }
    }
  // spans 1 .. 16: inside the lane
#pragma unroll
  for (int h = 1; h < 32; h *= 2)
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if (!(j & h)) {
          const float a = x[m * 32 + j], b = x[m * 32 + j + h];
          x[m * 32 + j] = a + b;
          x[m * 32 + j + h] = a - b;
        }
  // span 32: element bit 5 is the lane's half. After the swap lo holds the pair's element
  // with bit 5 clear (from the lower lane) and hi the one with bit 5 set, in both lanes; the
  // lower lane keeps lo + hi, the upper lo - hi (one rounded fma with a +-1 factor each).
  const float hs = half ? -1.f : 1.f;
#pragma unroll
  for (int e = 0; e < NM * 32; ++e) {
    float lo = x[e], hi = x[e];
    permlane32_swap_pair(lo, hi);
    x[e] = __builtin_fmaf(hs, hi, lo);
  }
  // span 64 (d = 128): inside the lane (m = 0 with m = 1)
  if constexpr (NM == 2) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float a = x[j], b = x[32 + j];
      x[j] = a + b;
      x[32 + j] = a - b;
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < NM * 32; ++e) {
    x[e] *= inv_sqrt_d;
    amax = __builtin_elementwise_maximum(amax, __builtin_fabsf(x[e]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (lane == 0) blk_max[wave] = amax;
  barrier_lds();
  const int w0 = (wave / 4) * 4;                       // the 4 waves of this 128-row block
  amax = fmaxf(fmaxf(blk_max[w0], blk_max[w0 + 1]), fmaxf(blk_max[w0 + 2], blk_max[w0 + 3]));
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  // x / s as the quantiser divides (correctly rounded; a tiny scale is divided in the form
  // scaled by 2^64, which gives the same quotient)
  float sd = s;
  if (s < 0x1p-64f) {
    sd = s * 0x1p64f;
#pragma unroll
    for (int e = 0; e < NM * 32; ++e) x[e] *= 0x1p64f;
  }
  const float y_rcp = 1.0f / sd;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    int w[8];
#pragma unroll
    for (int e = 0; e < 32; e += 2) {
      float y[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float xv = x[m * 32 + e + k];
        const float q0 = xv * y_rcp;
        const float q = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, sd, xv), y_rcp, q0), xv);
        y[k] = fminf(fmaxf(q, -448.0f), 448.0f);
      }
      if (e % 4 == 0) w[e / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      else w[e / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], w[e / 4], true);
    }
    qreg[m] = i32x8{w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]};
  }
  return s;
}

template <int D, bool CAUSAL, bool FUSEQ>
__global__ __launch_bounds__(kWaves * 64, 1) void attn_fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ SQ, const float* __restrict__ SK, const float* __restrict__ SV,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_mtiles, int nblk, int total_wg, float c_base,
    const uint16_t* __restrict__ Qbf /* FUSEQ: bf16 Q */, const float* __restrict__ signs /* FUSEQ */,
    uint8_t* __restrict__ q8_out /* FUSEQ, may be null */, float* __restrict__ sq_out /* FUSEQ, may be null */,
    float inv_sqrt_d /* FUSEQ: fp32 nearest 1/sqrt(d) */) {
  constexpr int ROW = D;                             // bytes per K/V row
  constexpr int TB = kBN * ROW;                      // bytes per K (or V) tile: 8 KiB (d = 128), 4 KiB (d = 64)
  constexpr int LOADERS = TB / 1024;                 // waves that load a tile, 1 KiB each: 8 or 4
  constexpr int NS = 4;                              // ring slots per operand
  constexpr int NKB = kBN / 32;                      // 32-key blocks per tile
  constexpr int NM = D / 64;                         // 64-element MFMA k-steps over the head dim
  constexpr int NDB = D / 32;                        // 32-wide head-dim blocks of O
  static_assert(LOADERS >= 1 && LOADERS <= kWaves && LOADERS * 1024 == TB, "whole 1 KiB loads");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * NS * TB];   // K ring, then V ring

  int bh, mt;
  xcd_query_tile(blockIdx.x, total_wg, n_mtiles, CAUSAL, bh, mt);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int half = lane / 32, l32 = lane % 32;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint8_t* Qh = Q + head_off;
  const uint8_t* Kh = K + head_off;
  const uint8_t* Vh = V + head_off;
  const float* sk = SK + (int64_t)bh * nblk;
  const float* sv = SV + (int64_t)bh * nblk;

  const int q0 = mt * kBM + wave * 32;               // this wave's 32 rows (inside one Q scale block)
  const int qrow = q0 + l32;
  float cq = 0.f;
  __shared__ float q_blk_max[kWaves];

  // Q^T as the B operand: for MFMA m (head-dim half), bytes [m*64 + half*32, +32) of the row
  // (FUSEQ: made in the prologue, after the first K/V tile loads are issued).
  i32x8 qreg[NM];
  if constexpr (!FUSEQ) {
    cq = c_base * SQ[(int64_t)bh * nblk + min(q0 / kScaleRows, nblk - 1)];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (qrow < N) {
        const i32x4 a = *(const i32x4*)(Qh + (int64_t)qrow * D + m * 64 + half * 32);
        const i32x4 b = *(const i32x4*)(Qh + (int64_t)qrow * D + m * 64 + half * 32 + 16);
        qreg[m] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      } else {
        qreg[m] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }

  const int n_ktiles = (N + kBN - 1) / kBN;
  const int T = CAUSAL ? min(n_ktiles, ((mt + 1) * kBM + kBN - 1) / kBN) : n_ktiles;

  // K fragment (kb, m): row kb*32 + l32, chunks m*4 + half*2 and +1 (32 bytes).
  uint32_t kaddr[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) kaddr[m] = l32 * ROW + (((m * 4 + half * 2) ^ swz<D>(l32)) << 4);
  // V^T fragment (db): four 8-byte transpose reads; read m covers the keys
  // (m/2)*32 + ((m%2)*2 + j/4)*8 + tr_h*4 + j%4, the order of this lane's P bytes. The
  // row offsets of m (multiples of 16) leave the swizzle unchanged.
  const int g16 = lane / 16, i16 = lane % 16;
  const int tr_h = g16 / 2, tr_j = i16 >> 1;
  const int tr_row = (tr_j / 4) * 8 + tr_h * 4 + (tr_j % 4);
  const int tr_col = 16 * (g16 % 2) + 8 * (i16 & 1);
  uint32_t vaddr[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int col = db * 32 + tr_col;
    vaddr[db] = tr_row * ROW + (((col >> 4) ^ swz<D>(tr_row)) << 4) + (col & 15);
  }

  // Direct global -> LDS loads: wave w < LOADERS fills bytes [w*1024, +1024) of a tile, 16
  // per lane; the other waves load nothing (their waits on their own loads pass at once,
  // and every wave waits at the barrier for the loaders).
  const int ld_slot = wave * 1024 + lane * 16;
  const int ld_row = ld_slot / ROW;
  const int ld_ch = ((ld_slot % ROW) / 16) ^ swz<D>(ld_row);
  const int ld_off = ld_row * ROW + ld_ch * 16;
  auto kbuf = [&](auto SLOT) __attribute__((always_inline)) -> uint8_t* { return lds + decltype(SLOT)::value * TB; };
  auto vbuf = [&](auto SLOT) __attribute__((always_inline)) -> uint8_t* {
    return lds + (NS + decltype(SLOT)::value) * TB;
  };
  auto load_tile = [&](const uint8_t* src, int kt, uint8_t* dst) __attribute__((always_inline)) {
    if (LOADERS < kWaves && wave >= LOADERS) return;
    if (kt * kBN + kBN <= N) {
      dma_load16(src + (int64_t)kt * TB + ld_off, lds_u32(dst) + wave * 1024);
    } else {   // rows past the end re-read the last row (masked scores, P = 0)
      const int key = min(kt * kBN + ld_row, N - 1);
      dma_load16(src + (int64_t)key * ROW + ld_ch * 16, lds_u32(dst) + wave * 1024);
    }
  };
  auto kfrag = [&](const uint8_t* kb_base, int kb, int m) __attribute__((always_inline)) -> i32x8 {
    const uint8_t* p = kb_base + kb * 32 * ROW + kaddr[m];
    const i32x4 a0 = *(const i32x4*)p;
    const i32x4 a1 = *(const i32x4*)(kb_base + kb * 32 * ROW + (kaddr[m] ^ 16));
    return i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  };
  auto qk = [&](auto SLOT, f32x16 (&S)[NKB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      S[kb] = f32x16{};
#pragma unroll
      for (int m = 0; m < NM; ++m) S[kb] = mfma_fp8(kfrag(kbuf(SLOT), kb, m), qreg[m], S[kb]);
    }
  };

  f32x16 oacc[NDB];                    // P''.V (in units of U)
  f32x4 lacc = f32x4{};                // the last tile's sum of rounded P''
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  // Running max M (log2 units), this lane's partial row sum of the unrounded
  // probabilities (for the LSE), and a pending rescale factor of the accumulators.
  float M = -INFINITY, l_part = 0.f, alpha_pend = 1.f;
  // Unit U of the P.V accumulator (a V block scale), an owed change of unit, and the
  // denominator: the sum over tiles of (sum of the tile's rounded P'' codes) * w.
  float U = 1.f, unit_pend = 1.f, l_rnd = 0.f;

  // Per-tile constants of tile u: score factor and V block scale.
  auto tile_sk = [&](int u) __attribute__((always_inline)) { return sk[min(u * kBN / kScaleRows, nblk - 1)]; };
  auto tile_c = [&](int u) __attribute__((always_inline)) { return cq * tile_sk(u); };
  auto tile_sv = [&](int u) __attribute__((always_inline)) { return sv[min(u * kBN / kScaleRows, nblk - 1)]; };
  // w = U / svb of a tile with V block scale svb; when svb / U leaves [1, 3/2] the unit
  // moves to svb (w = 1) and the accumulator owes the factor old U / new U. Returns
  // whether the unit moved (wave-uniform: both scales are).
  auto weight = [&](float svb, float& w) __attribute__((always_inline)) -> bool {
    if (svb >= U && svb <= 1.5f * U) {
      w = U * __builtin_amdgcn_rcpf(svb);
      return false;
    }
    unit_pend *= U * __builtin_amdgcn_rcpf(svb);
    U = svb;
    w = 1.f;
    return true;
  };

  auto mask_tile = [&](int u, f32x16 (&S)[NKB]) __attribute__((always_inline)) {
    const int key0 = u * kBN;
    if ((CAUSAL && key0 + kBN - 1 > q0) || key0 + kBN > N) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + (r / 4) * 8 + half * 4 + (r % 4);
          if ((CAUSAL && key > qrow) || key >= N) S[kb][r] = -INFINITY;
        }
    }
  };
  auto max_pairs = [&](float (&m4)[4], const f32x16 (&S)[NKB], int e_begin, int e_end) __attribute__((always_inline)) {
#pragma unroll
    for (int e = e_begin; e < e_end; e += 2)
      m4[(e / 2) % 4] = max3f(m4[(e / 2) % 4], S[e / 16][e % 16], S[e / 16][e % 16 + 1]);
  };
  // Raise M when some row of the wave grew by more than kTau (branch-free); l is
  // rescaled at once, O at the start of the next step. Returns whether M moved. A row
  // whose M moves to this tile's max takes M = max - log2 w (lw), so that its largest
  // probability is coded as P'' = 2^kPShift exactly, as with w = 1.
  auto max_final = [&](const float (&m4)[4], float ct, float lw) __attribute__((always_inline)) -> bool {
    const float mx = max_halves(max3f(m4[0], m4[1], __builtin_elementwise_maximum(m4[2], m4[3]))) * ct;
    const bool grow = __builtin_amdgcn_ballot_w64(mx > M + kTau) != 0;
    const float M_new = grow ? __builtin_elementwise_maximum(M, mx - lw) : M;
    const float alpha = grow ? fast_exp2(M - M_new) : 1.f;
    M = M_new;
    l_part *= alpha;
    alpha_pend *= alpha;
    return grow;
  };
  // P' of scores [e0, e1), in three passes issued apart so that no VALU op waits on the
  // one before it: the exp2 arguments (args), the exponentials, written over the scores
  // (exps), then the row sums (two chains) and the rounding to E4M3, four per word (finish).
  auto args = [&](f32x16 (&S)[NKB], float ct, float bias, int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
    for (int e = e0; e < e1; ++e) S[e / 16][e % 16] = __builtin_fmaf(S[e / 16][e % 16], ct, -bias);
  };
  auto exps = [&](f32x16 (&S)[NKB], int e0, int e1) __attribute__((always_inline)) {
#pragma unroll
    for (int e = e0; e < e1; ++e) S[e / 16][e % 16] = fast_exp2(S[e / 16][e % 16]);
  };
  auto finish = [&](const f32x16 (&S)[NKB], int (&P)[8], float (&lsum)[2], int e0, int e1)
                    __attribute__((always_inline)) {
#pragma unroll
    for (int e = e0; e < e1; ++e) {
      const float pe = S[e / 16][e % 16];
      lsum[e % 2] += pe;
      // (the first pair of a word writes bytes 0-1 over the word's previous contents, a
      // tile's codes that were consumed a step earlier: bytes 2-3 are written next)
      if (e % 4 == 1) P[e / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(S[e / 16][e % 16 - 1], pe, P[e / 4], false);
      if (e % 4 == 3) P[e / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(S[e / 16][e % 16 - 1], pe, P[e / 4], true);
    }
  };
  // Owed running-max rescale (accumulator and rounded-code denominator) and change of
  // unit (accumulator only: the denominator is in units of P').
  auto rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha_pend * unit_pend;
    l_rnd *= alpha_pend;
    alpha_pend = 1.f;
    unit_pend = 1.f;
  };

  f32x16 Sa[NKB], Sb[NKB];
  int Pa[8] = {}, Pb[8] = {};
  // A operand of the code-sum MFMA (16x16x128), which reads the P.V B operand as is. Seen
  // as that MFMA's B, lane 16g + n holds 32 codes of query n + 16 (g % 2) (lanes l and
  // l + 32 hold the two key halves of query l % 32); A row m is E4M3 1.0 on the k blocks
  // g with g % 2 == (m / 4) % 2 and 0 elsewhere, so output rows 0-3 and 8-11 of column n
  // hold the code sum of query n and rows 4-7 and 12-15 that of query n + 16: each lane
  // receives its own query's sum (lane 16g + n gets rows 4g..4g+3). Kept in eight
  // registers for the whole loop: eight distinct per-lane expressions (0 <= qrow < 2^31 - 8,
  // so each shift adds 0) that the compiler can neither merge into one register nor fold.
  i32x8 ones;
  const int ones_word = ((lane >> 4) & 1) == ((lane >> 2) & 1) ? 0x38383838 : 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) ones[k] = ones_word + ((qrow + k) >> 31);
  bool pend = false;     // wave-uniform: an O rescale is owed
  // w of the tile whose code sum lacc holds, and of the tile whose softmax ran last; the
  // K and V block scales of the tile whose softmax runs next, loaded one step early so
  // that their scalar loads complete under the step's barrier.
  float w_lacc = 0.f, w_soft = 0.f, sk_next = 0.f, sv_next = 1.f;

  // Step t: S(t+1) in S_soft, S(t+2) -> S_new, P(t) in P_use, P(t+1) -> P_new;
  // K(t+2) in K slot (t+2)%4, V(t) in V slot t%4; loads K(t+4) -> K slot t%4 and
  // V(t+3) -> V slot (t+3)%4 (clamped past the last tile, never read; the scores of tile
  // T, if computed, are fully masked).
  // DR (drain steps, T a multiple of 4): 1 at t = T-2, whose S^T MFMAs would compute the
  // nonexistent tile T (skipped; the softmax of tile T-1 runs as usual); 2 at t = T-1, which
  // runs only the P.V MFMAs of tile T-1 (no tile T+1 to compute, no tile T to take the
  // softmax of).
  auto step = [&](int t, f32x16 (&S_soft)[NKB], f32x16 (&S_new)[NKB], const int (&P_use)[8], int (&P_new)[8],
                  auto KRD, auto VRD, auto KLD, auto VLD, auto DRc) __attribute__((always_inline)) {
    constexpr int DR = decltype(DRc)::value;
    load_tile(Kh, min(t + 4, T - 1), kbuf(KLD));
    load_tile(Vh, min(t + 3, T - 1), vbuf(VLD));
    static_assert(kScaleRows == 2 * kBN, "a V scale block spans two tiles");
    // Causal: once the tile's first key lies past this wave's last row, this and every
    // later tile are fully masked for the wave; it only keeps up its loads and barriers.
    if (!CAUSAL || t * kBN <= q0 + 31) {
      l_rnd = __builtin_fmaf(lacc[0], w_lacc, l_rnd);    // tile t-1's rounded codes
      w_lacc = w_soft;                                    // tile t, whose codes lacc sums next
      if (pend) rescale();
      if constexpr (DR == 2) {
        i32x8 vf[NDB];
        auto vread = [&](int db) __attribute__((always_inline)) {
          int av[8];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const i32x2 x = lds_read_tr8(vbuf(VRD) + ((m / 2) * 32 + (m % 2) * 16) * ROW + vaddr[db]);
            av[2 * m] = x[0];
            av[2 * m + 1] = x[1];
          }
          vf[db] = i32x8{av[0], av[1], av[2], av[3], av[4], av[5], av[6], av[7]};
        };
        vread(0);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          if (db + 1 < NDB) vread(db + 1);
          const i32x8 pb = {P_use[0], P_use[1], P_use[2], P_use[3], P_use[4], P_use[5], P_use[6], P_use[7]};
          oacc[db] = mfma_fp8(vf[db], pb, oacc[db]);
          if (db == NDB - 1) lacc = mfma_fp8_16(ones, pb, f32x4{});
        }
      } else {
      mask_tile(t + 1, S_soft);
      const float ct = cq * sk_next;
      const bool uchg = weight(sv_next, w_soft);
      const float lw = __builtin_amdgcn_logf(w_soft);     // log2 w
      // Main block in intended issue order: NQ S^T MFMAs (K fragments one MFMA ahead) and
      // NDB P.V MFMAs (V^T fragments one MFMA ahead); the row max runs beside the first two
      // S^T MFMAs, the exponentials beside the others (d = 128: 4 + 4, six slots; d = 64:
      // 2 + 2, two slots).
      constexpr int NQ = NKB * NM;
      i32x8 kf[NQ], vf[NDB];
      auto kread = [&](int i) __attribute__((always_inline)) { kf[i] = kfrag(kbuf(KRD), i % NKB, i / NKB); };
      auto vread = [&](int db) __attribute__((always_inline)) {
        int av[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const i32x2 x = lds_read_tr8(vbuf(VRD) + ((m / 2) * 32 + (m % 2) * 16) * ROW + vaddr[db]);
          av[2 * m] = x[0];
          av[2 * m + 1] = x[1];
        }
        vf[db] = i32x8{av[0], av[1], av[2], av[3], av[4], av[5], av[6], av[7]};
      };
      float m4[4] = {S_soft[0][0], S_soft[0][1], S_soft[0][2], S_soft[0][3]};
      float lsum[2] = {0.f, 0.f}, bias = 0.f;
      // NSLOT slots (the S^T MFMAs after the first two, and the P.V MFMAs) share the 32
      // scores; slot k issues the arguments of slot k+1, the exponentials of slot k and the
      // sums of slot k-1
      constexpr int NSLOT = NQ - 2 + NDB;
      static_assert(NQ >= 2, "the row max needs two S^T MFMAs");
      auto lo = [&](int slot) __attribute__((always_inline)) { return slot * (NKB * 16) / NSLOT; };
      auto exps_slot = [&](int slot) __attribute__((always_inline)) {
        if (slot + 1 < NSLOT) args(S_soft, ct, bias, lo(slot + 1), lo(slot + 2));
        exps(S_soft, lo(slot), lo(slot + 1));
        if (slot > 0) finish(S_soft, P_new, lsum, lo(slot - 1), lo(slot));
      };
      if constexpr (DR == 0) kread(0);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {              // i = m * NKB + kb
        if (i + 1 < NQ) {
          if constexpr (DR == 0) kread(i + 1);
        } else {
          vread(0);
        }
        const int kb = i % NKB, m = i / NKB;
        if constexpr (DR == 0) S_new[kb] = mfma_fp8(kf[i], qreg[m], m == 0 ? f32x16{} : S_new[kb]);
        if (i == 0) {
          max_pairs(m4, S_soft, 4, 18);
        } else if (i == 1) {
          max_pairs(m4, S_soft, 18, NKB * 16);
          pend = max_final(m4, ct, lw) | uchg;
          bias = M - kPShift + lw;
          args(S_soft, ct, bias, lo(0), lo(1));
        } else {
          exps_slot(i - 2);
        }
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if (db + 1 < NDB) vread(db + 1);
        const i32x8 pb = {P_use[0], P_use[1], P_use[2], P_use[3], P_use[4], P_use[5], P_use[6], P_use[7]};
        oacc[db] = mfma_fp8(vf[db], pb, oacc[db]);
        if (db == NDB - 1) {
          lacc = mfma_fp8_16(ones, pb, f32x4{});
        }
        exps_slot(NQ - 2 + db);
      }
      finish(S_soft, P_new, lsum, lo(NSLOT - 1), NKB * 16);
      l_part = __builtin_fmaf(lsum[0] + lsum[1], w_soft, l_part);
      sk_next = tile_sk(t + 2);
      sv_next = tile_sv(t + 2);
      }
    }
    wait_vmcnt<2>();         // K(t+3) and V(t+1), issued a step earlier, have landed
    barrier_lds();
  };

  // Prologue: K tiles 0..3 and V tiles 0..2; S(0), softmax of tile 0, S(1).
  load_tile(Kh, 0, kbuf(IC<0>{}));
  load_tile(Kh, min(1, T - 1), kbuf(IC<1>{}));
  load_tile(Kh, min(2, T - 1), kbuf(IC<2>{}));
  load_tile(Kh, min(3, T - 1), kbuf(IC<3>{}));
  load_tile(Vh, 0, vbuf(IC<0>{}));
  load_tile(Vh, min(1, T - 1), vbuf(IC<1>{}));
  load_tile(Vh, min(2, T - 1), vbuf(IC<2>{}));
  if constexpr (FUSEQ) {
    // rotate and quantise this wave's query rows while the first tiles load
    const float sqb = fused_q_prep<D>(Qbf + head_off + (int64_t)qrow * D, qrow < N, signs, inv_sqrt_d, half, wave,
                                      lane, q_blk_max, qreg);
    cq = c_base * sqb;
    if (q8_out != nullptr && qrow < N) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        uint8_t* dst = q8_out + head_off + (int64_t)qrow * D + m * 64 + half * 32;
        *(i32x4*)dst = i32x4{qreg[m][0], qreg[m][1], qreg[m][2], qreg[m][3]};
        *(i32x4*)(dst + 16) = i32x4{qreg[m][4], qreg[m][5], qreg[m][6], qreg[m][7]};
      }
    }
    const int blk = q0 / kScaleRows;
    if (sq_out != nullptr && wave % 4 == 0 && lane == 0 && blk < nblk) sq_out[(int64_t)bh * nblk + blk] = sqb;
  }
  wait_vmcnt<0>();
  barrier_lds();
  qk(IC<0>{}, Sa);
  {
    mask_tile(0, Sa);
    const float ct = tile_c(0);
    float m4[4] = {Sa[0][0], Sa[0][1], Sa[0][2], Sa[0][3]};
    max_pairs(m4, Sa, 4, NKB * 16);
    max_final(m4, ct, 0.f);       // tile 0 has w = 1
    alpha_pend = 1.f;            // O is still zero: no rescale owed
    U = tile_sv(0);              // the first tile sets the unit: w = 1
    w_soft = 1.f;
    const float bias = M - kPShift;
    float lsum[2] = {0.f, 0.f};
    args(Sa, ct, bias, 0, NKB * 16);
    exps(Sa, 0, NKB * 16);
    finish(Sa, Pa, lsum, 0, NKB * 16);
    l_part = __builtin_fmaf(lsum[0] + lsum[1], w_soft, l_part);
    sk_next = tile_sk(1);
    sv_next = tile_sv(1);
  }
  qk(IC<1>{}, Sb);
  barrier_lds();                 // K slots 0 and 1 are refilled from step 0 on

  // Causal, T a multiple of 4: the last four steps follow the loop, the last two as drain
  // steps (the non-causal kernel keeps one loop: a second copy of the step costs it its
  // spill-free register allocation)
  const bool peel = CAUSAL && T % 4 == 0;
  const int t_main = peel ? T - 4 : T;
  for (int t = 0; t < t_main; t += 4) {
    step(t, Sb, Sa, Pa, Pb, IC<2>{}, IC<0>{}, IC<0>{}, IC<3>{}, IC<0>{});
    if (t + 1 < T) step(t + 1, Sa, Sb, Pb, Pa, IC<3>{}, IC<1>{}, IC<1>{}, IC<0>{}, IC<0>{});
    if (t + 2 < T) step(t + 2, Sb, Sa, Pa, Pb, IC<0>{}, IC<2>{}, IC<2>{}, IC<1>{}, IC<0>{});
    if (t + 3 < T) step(t + 3, Sa, Sb, Pb, Pa, IC<1>{}, IC<3>{}, IC<3>{}, IC<2>{}, IC<0>{});
  }
  if (CAUSAL && peel) {
    const int t = T - 4;
    step(t, Sb, Sa, Pa, Pb, IC<2>{}, IC<0>{}, IC<0>{}, IC<3>{}, IC<0>{});
    step(t + 1, Sa, Sb, Pb, Pa, IC<3>{}, IC<1>{}, IC<1>{}, IC<0>{}, IC<0>{});
    step(t + 2, Sb, Sa, Pa, Pb, IC<0>{}, IC<2>{}, IC<2>{}, IC<1>{}, IC<1>{});
    step(t + 3, Sa, Sb, Pb, Pa, IC<1>{}, IC<3>{}, IC<3>{}, IC<2>{}, IC<2>{});
  }
  wait_vmcnt<0>();               // no load may still target this workgroup's LDS when it exits
  l_rnd = __builtin_fmaf(lacc[0], w_lacc, l_rnd);       // the last tile's rounded codes
  if (pend) rescale();

  const float l_tot = add_halves(l_part) * (1.f / (1 << (int)kPShift));   // sum of probabilities
  const float inv = U / l_rnd;                       // (rows past N are not stored)
  // O (bf16) through LDS, so that the stores write whole rows: each wave stages its 32 rows
  // (row-major, 16-byte chunk c of row r at chunk c ^ (r mod chunks per row)) in its own
  // 32 * OROW bytes of the rings, then stores 16 bytes per lane, 1 KiB of consecutive rows
  // per instruction. Every wave has waited for its own loads above; after the barrier no
  // load is in flight into the rings and no wave reads them any more.
  constexpr int OROW = D * 2, NCH = OROW / 16;
  static_assert(kWaves * 32 * OROW <= 2 * NS * TB, "the staged rows fit the rings");
  barrier_lds();
  uint8_t* stg = lds + wave * 32 * OROW;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x16 a = oacc[db];
      *(u32x2*)(stg + l32 * OROW + (((db * 4 + g) ^ (l32 % NCH)) << 4) + half * 8) =
          u32x2{pack2(Bf16Tag{}, a[g * 4 + 0] * inv, a[g * 4 + 1] * inv),
                pack2(Bf16Tag{}, a[g * 4 + 2] * inv, a[g * 4 + 3] * inv)};
    }
  uint8_t* Ow = (uint8_t*)(O + head_off + (int64_t)q0 * D);   // the wave's 32 rows, contiguous
#pragma unroll
  for (int i = 0; i < 32 * OROW / 1024; ++i) {
    const int off = i * 1024 + lane * 16, r = off / OROW, ch = (off % OROW) / 16;
    const u32x4 x = *(const u32x4*)(stg + r * OROW + ((ch ^ (r % NCH)) << 4));
    if (q0 + r < N) *(u32x4*)(Ow + off) = x;
  }
  if (qrow < N && half == 0) LSE[(int64_t)bh * N + qrow] = (M + __builtin_log2f(l_tot)) * kLn2;
}

template <int D, bool CAUSAL, bool FUSEQ>
hipError_t launch(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* sq, const float* sk,
                  const float* sv, void* o, float* lse, int64_t BH, int64_t N, float scale, const void* qbf,
                  const float* signs, uint8_t* q8_out, float* sq_out, hipStream_t stream) {
  const int n_mtiles = (int)((N + kBM - 1) / kBM);
  const int nblk = (int)((N + kScaleRows - 1) / kScaleRows);
  const int64_t total = BH * n_mtiles;
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, CAUSAL, FUSEQ>), dim3((unsigned)total), dim3(kWaves * 64), 0, stream, q8,
                     k8, v8, sq, sk, sv, (uint16_t*)o, lse, (int)N, n_mtiles, nblk, (int)total, scale * kLog2e,
                     (const uint16_t*)qbf, signs, q8_out, sq_out, (float)(1.0 / __builtin_sqrt((double)D)));
  return hipGetLastError();
}

template <bool FUSEQ>
hipError_t launch_d(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* sq, const float* sk,
                    const float* sv, void* o, float* lse, int64_t BH, int64_t N, int64_t d, bool causal, float scale,
                    const void* qbf, const float* signs, uint8_t* q8_out, float* sq_out, hipStream_t stream) {
  if (d == 128)
    return causal ? launch<128, true, FUSEQ>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, qbf, signs, q8_out, sq_out,
                                             stream)
                  : launch<128, false, FUSEQ>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, qbf, signs, q8_out,
                                              sq_out, stream);
  return causal ? launch<64, true, FUSEQ>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, qbf, signs, q8_out, sq_out,
                                          stream)
                : launch<64, false, FUSEQ>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, qbf, signs, q8_out, sq_out,
                                           stream);
}

}  // namespace

hipError_t launch_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* sq, const float* sk,
                          const float* sv, void* o, float* lse, int64_t BH, int64_t N, int64_t d, bool causal,
                          float scale, hipStream_t stream) {
  return launch_d<false>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, d, causal, scale, nullptr, nullptr, nullptr, nullptr,
                         stream);
}

hipError_t launch_fwd_fp8_rotq(const void* q, const float* signs, const uint8_t* k8, const uint8_t* v8,
                               const float* sk, const float* sv, void* o, float* lse, uint8_t* q8_out, float* sq_out,
                               int64_t BH, int64_t N, int64_t d, bool causal, float scale, hipStream_t stream) {
  return launch_d<true>(nullptr, k8, v8, nullptr, sk, sv, o, lse, BH, N, d, causal, scale, q, signs, q8_out, sq_out,
                        stream);
}

int64_t max_workgroups_fwd8(int64_t BH, int64_t N) { return BH * ((N + kBM - 1) / kBM); }

}  // namespace attn
