// Exact attention backward for bf16 / fp16 on gfx950 (MI355X).
//
// The FlashAttention-2 digest (key technical points and method summary) has the backward
// pass recompute the attention from the one log-sum-exp per row that the forward pass
// stored, splitting the work the same way; it prints no formulas. The gradients are those
// of O = softmax(scale * Q K^T [+ causal mask]) V:
//   P = exp(scale * Q K^T - LSE)        recomputed per tile from the stored LSE
//   dV = P^T dO,   dP = dO V^T,   Delta_i = dO_i . O_i  (= sum_j P_ij dP_ij)
//   dS = P * (dP - Delta),   dQ = scale * dS K,   dK = scale * dS^T Q
// Two launches per call:
//   dq    one workgroup per (batch*head, 256-row query tile), 8 waves x 32 rows. First
//         Delta_i = dO_i . O_i and LSE_i of its rows (O is read here only), also written
//         to the caller's workspace for dkdv (as -Delta_i and -LSE_i / scale); then K and
//         V tiles of 64 keys stream through LDS (double-buffered direct loads). Per 32-key
//         block: S^T = K Q^T and dP^T = V dO^T (A = K / V rows read from LDS, B = Q^T and
//         dO^T kept in VGPRs), then P and dS in fp32 with one query row per lane (its LSE
//         and Delta are scalars), then dQ^T += K^T dS^T (A = K^T by LDS transpose reads,
//         B = dS rounded to 16 bits).
//   dkdv  one workgroup per (batch*head, 128-key tile), 8 waves: 4 key groups of 32 keys
//         x 2 halves of each 64-query tile. Each lane keeps its key's K and V rows in
//         registers (the B operands of S and dP); Q and dO tiles stream through a 3-slot
//         LDS ring. Per wave and tile: S = Q K^T and dP = dO V^T on its 32 queries, with
//         accumulators that start at -LSE / scale and -Delta of each query, so that the
//         MFMAs give the exponent and the factor of dS directly: P = 2^(scale log2 e * s),
//         dS = P * dp. The two waves of a key group split the gradients: the first
//         accumulates dV^T += dO^T P, the second dK^T += Q^T dS, each over all 64 queries
//         (A = dO^T / Q^T by LDS transpose reads, B = P / dS rounded to 16 bits); each
//         hands the other the 16-bit P or dS of its own 32 queries through LDS. These
//         contractions run one tile behind S and dP (tile u - 1 in the step of tile u),
//         so the softmax of a tile and the contraction of the one before sit in the same
//         step. Two waves per SIMD keep each wave within 256 VGPRs, so MFMA results stay
//         in VGPRs (no AGPR copies).
// The two gradient kernels each recompute S and dP, so that every gradient stays in
// registers until its one store: no fp32 partial sums or atomics in memory.
// Causal: query tiles of dq stop at the diagonal and key tiles of dkdv start at it; a dq
// wave skips key tiles that lie wholly past its rows (a dkdv wave computes its two fully
// masked blocks: the other waves set the step's length), and only blocks crossing the
// diagonal or the end of the sequence apply a mask.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "tile_lds.h"

namespace attn {
namespace {

constexpr int kWq = 8;      // dq: waves per workgroup (32 query rows each)
constexpr int kBN = 64;     // dq: keys per K/V tile
constexpr int kKG = 4;      // dkdv: key groups of 32 keys per workgroup
constexpr int kWk = 8;      // dkdv: waves per workgroup (a key group x a query half of each tile)
constexpr int kBQ = 64;     // dkdv: queries per Q/dO tile (two 32-query blocks)

__device__ __forceinline__ float to_f32(Bf16Tag, uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }
__device__ __forceinline__ float to_f32(F16Tag, uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

template <typename Tag, int D, bool CAUSAL>
__global__ __launch_bounds__(kWq * 64, 1) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ ws, uint16_t* __restrict__ dQ, int N, int n_mtiles, int total_wg, int64_t rows,
    float c /* scale*log2 e */, float scale) {
  constexpr int W = kWq, BM = W * 32, NSTEP = D / 16, NKB = kBN / 32, NDB = D / 32;
  constexpr int TB = kBN * D * 2;                   // bytes per K (or V) tile
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * TB];   // K slots 0, 1; V slots 0, 1

  int bh, mt;
  xcd_query_tile(blockIdx.x, total_wg, n_mtiles, CAUSAL, bh, mt);   // causal: longest query tiles first

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int half = lane / 32, l32 = lane % 32;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* Kh = K + head_off;
  const uint16_t* Vh = V + head_off;

  const int q0 = mt * BM + wave * 32;
  const int qrow = q0 + l32;
  u32x4 qreg[NSTEP], doreg[NSTEP], oreg[NSTEP];
  load_row_operand<D>(Q + head_off, qrow, N, half, qreg);
  load_row_operand<D>(dO + head_off, qrow, N, half, doreg);
  load_row_operand<D>(O + head_off, qrow, N, half, oreg);
  float delta, lse2;                                // this lane's row: dO . O and LSE * log2(e), set below

  const int n_ktiles = (N + kBN - 1) / kBN;
  const int T = CAUSAL ? min(n_ktiles, ((mt + 1) * BM + kBN - 1) / kBN) : n_ktiles;
  TileAddr<D> ta;
  ta.init(lane);

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  auto kbuf = [&](int slot) __attribute__((always_inline)) { return lds + slot * TB; };
  auto vbuf = [&](int slot) __attribute__((always_inline)) { return lds + (2 + slot) * TB; };

  // Step t: prefetch K/V tile t + 1 into the other slot, process tile t from slot SLOT
  // (compile-time, so every LDS read takes an immediate offset), then wait for the
  // prefetch. Only tiles crossing the diagonal or the end of the sequence mask scores,
  // in one block of their own ahead of the exponentials.
  auto step = [&](auto slot_c, int t) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_c)::value;
    if (t + 1 < T) {
      load_rows<D, kBN, W>(Kh, (t + 1) * kBN, N, kbuf(SLOT ^ 1), wave, lane);
      load_rows<D, kBN, W>(Vh, (t + 1) * kBN, N, vbuf(SLOT ^ 1), wave, lane);
    }
    if (!CAUSAL || t * kBN <= q0 + 31) {            // else: every key of the tile lies past this wave's rows
      const uint8_t* kt = kbuf(SLOT);
      const uint8_t* vt = vbuf(SLOT);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int key0 = t * kBN + kb * 32;
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) s = mfma32(Tag{}, row_frag<D>(kt, ta, kb * 32, st), qreg[st], s);
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) dp = mfma32(Tag{}, row_frag<D>(vt, ta, kb * 32, st), doreg[st], dp);
        if ((CAUSAL && key0 + 31 > q0) || key0 + 32 > N) {
          // keys past this lane's row (causal) or past the sequence
          const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - key0 - half * 4;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if ((r / 4) * 8 + (r % 4) > lim) s[r] = -INFINITY;
        }
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
          ds[r] = p * (dp[r] - delta);
        }
        u32x4 pb[2];
        pack16<Tag>(ds, pb);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[db] = mfma32(Tag{}, tr_frag<D>(kt, ta, kb * 32 + h * 16, db), pb[h], acc[db]);
      }
    }
    wait_vmcnt<0>();
    barrier_lds();
  };

  load_rows<D, kBN, W>(Kh, 0, N, kbuf(0), wave, lane);
  load_rows<D, kBN, W>(Vh, 0, N, vbuf(0), wave, lane);
  // Delta = dO . O of this lane's row (each half of the wave holds half of the row) and
  // LSE in log2 units, while the first K/V tile loads; published in the workspace for the
  // dK/dV kernel, which runs next.
  const float lse_raw = qrow < N ? LSE[(int64_t)bh * N + qrow] : 0.f;
  lse2 = lse_raw * kLog2e;
  float dpart = 0.f;
#pragma unroll
  for (int st = 0; st < NSTEP; ++st)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dpart = __builtin_fmaf(to_f32(Tag{}, oreg[st][e] & 0xFFFFu), to_f32(Tag{}, doreg[st][e] & 0xFFFFu), dpart);
      dpart = __builtin_fmaf(to_f32(Tag{}, oreg[st][e] >> 16), to_f32(Tag{}, doreg[st][e] >> 16), dpart);
    }
  delta = add_halves(dpart);
  if (qrow < N && half == 0) {
    ws[(int64_t)bh * N + qrow] = -delta;
    ws[rows + (int64_t)bh * N + qrow] = -(lse_raw / scale);
  }
  wait_vmcnt<0>();
  barrier_lds();
  for (int t = 0; t < T; t += 2) {
    step(IC<0>{}, t);
    if (t + 1 < T) step(IC<1>{}, t + 1);
  }
  // the loop ended on a barrier with no load in flight: the K/V slots are free for staging
  static_assert(W * 32 * D * 2 <= 4 * TB, "the staged rows fit the tiles' LDS");
  store_rows_staged<Tag, D>(dQ + head_off + (int64_t)q0 * D, N - q0, acc, lane, scale, lds + wave * 32 * D * 2);
}

template <typename Tag, int D, bool CAUSAL>
__global__ __launch_bounds__(kWk * 64, 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ ws, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int N, int n_ntiles, int total_wg, int64_t rows, float c, float scale) {
  constexpr int W = kWk, BNK = kKG * 32, NSTEP = D / 16, NDB = D / 32;
  constexpr int NS = 3;                             // Q / dO ring slots
  constexpr int TB = kBQ * D * 2;                   // bytes per Q (or dO) tile
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * NS * TB];   // Q slots, then dO slots
  __shared__ __attribute__((aligned(16))) float lsd[NS][2][kBQ];     // [slot][-LSE/scale | -Delta][query]
  __shared__ __attribute__((aligned(16))) u32x4 xch[2][W][2][64];    // [tile parity][wave][block][lane]
  static_assert(W == 2 * kKG && kBQ == 64, "two waves (query halves) per key group");

  // causal: low key tiles see the most queries; the query-tile order, reversed, runs
  // them first
  int bh, rt;
  xcd_query_tile(blockIdx.x, total_wg, n_ntiles, CAUSAL, bh, rt);
  const int nt = CAUSAL ? n_ntiles - 1 - rt : rt;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int half = lane / 32, l32 = lane % 32;
  const int kg = wave % kKG, qh = wave / kKG;       // key group; query half of each tile
  const int64_t head_off = (int64_t)bh * N * D;
  const uint16_t* Qh = Q + head_off;
  const uint16_t* dOh = dO + head_off;
  const float* ndelta_h = ws + (int64_t)bh * N;     // -Delta
  const float* nlsc_h = ws + rows + (int64_t)bh * N;  // -LSE / scale

  const int k0 = nt * BNK + kg * 32;
  const int krow = k0 + l32;
  // K^T and V^T as the B operands of S = Q K^T and dP = dO V^T: this lane's key row,
  // resident for the whole loop (zero past the end of the sequence: such a key's dK and dV
  // are never stored)
  u32x4 kreg[NSTEP], vreg[NSTEP];
  load_row_operand<D>(K + head_off, krow, N, half, kreg);
  load_row_operand<D>(V + head_off, krow, N, half, vreg);

  const int n_qtiles = (N + kBQ - 1) / kBQ;
  const int u0 = CAUSAL ? (nt * BNK) / kBQ : 0;
  TileAddr<D> ta;
  ta.init(lane);
  RowPieces<D, kBQ, W> rp;
  rp.init(wave, lane);

  auto qbuf = [&](auto SLOT) __attribute__((always_inline)) { return lds + decltype(SLOT)::value * TB; };
  auto gbuf = [&](auto SLOT) __attribute__((always_inline)) { return lds + (NS + decltype(SLOT)::value) * TB; };
  // -LSE / scale and -Delta of a query tile (the workspace holds them negated) by 4-byte
  // direct loads into LDS, 32 values per wave (lanes 0..31 of waves 0..3): the initial
  // values of the S and dP accumulators, so that the MFMAs produce S - LSE / scale and
  // dP - Delta, i.e. P = 2^(c * s) and dS = P * dp with c = scale * log2 e
  static_assert(2 * kBQ == 4 * 32 && W >= 4, "four waves fetch a tile's values");
  auto load_ld = [&](int u, auto SLOT) __attribute__((always_inline)) {
    if (wave < 4 && lane < 32) {
      const float* base = wave / 2 ? ndelta_h : nlsc_h;
      const uint32_t q = (uint32_t)min(u * kBQ + 32 * (wave % 2) + lane, N - 1);
      dma_load4_s(base, q * 4, lds_u32((const uint8_t*)&lsd[decltype(SLOT)::value][wave / 2][32 * (wave % 2)]));
    }
  };
  const int qr = qh * 32;                           // this wave's 32 queries start at row qr of each tile

  // The two waves of a key group split the gradients: query half 0 accumulates dV^T +=
  // dO^T P and half 1 dK^T += Q^T dS, each over all 64 queries of a tile. Each computes S,
  // dP, P and dS of its own 32 queries, keeps the 16-bit operand of its own contraction and
  // hands the other one to its partner through LDS (xch, by tile parity).
  auto run = [&](auto ROLE) __attribute__((always_inline)) {
    constexpr bool RV = decltype(ROLE)::value == 0;   // dV (else dK)
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    f32x16 s, dp;                                   // S and dP of the current tile (own 32 queries)
    u32x4 keep[2];                                  // own P (dV) or dS (dK) of the previous tile, 16-bit
    // Scheduling fences between the phases keep each phase's operand reads inside it (the
    // registers would not hold them hoisted).
    constexpr int NMV = 4 * NDB;                    // MFMAs of the contraction per tile
    constexpr int EPM = 16 / NMV;                   // softmax elements beside each of them
    static_assert(EPM * NMV == 16, "the 16 elements spread evenly over the MFMAs");
    // MFMA i: 16-query block b = i / NDB of the tile, head-dim block db = i % NDB; A = dO^T
    // (dV) or Q^T (dK) by transpose reads of the tile's slot, B = the block's P or dS (own
    // blocks: this wave's half; the others: the partner's, from xch).
    auto frag = [&](auto SLOT, int i) __attribute__((always_inline)) -> u32x4 {
      return tr_frag<D>(RV ? gbuf(SLOT) : qbuf(SLOT), ta, (i / NDB) * 16, i % NDB);
    };
    auto mfma_i = [&](int i, const u32x4& a, const u32x4 (&other)[2]) __attribute__((always_inline)) {
      const int b = i / NDB, db = i % NDB;
      acc[db] = mfma32(Tag{}, a, b / 2 == decltype(ROLE)::value ? keep[b % 2] : other[b % 2], acc[db]);
    };
    auto read_other = [&](int u, u32x4 (&other)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) other[j] = xch[u & 1][wave ^ kKG][j][lane];
    };
    // the last tile's contraction alone (after the loop)
    auto contract = [&](auto SLOT, int u) __attribute__((always_inline)) {
      u32x4 other[2];
      read_other(u, other);
#pragma unroll
      for (int i = 0; i < NMV; ++i) mfma_i(i, frag(SLOT, i), other);
    };
    // Step of tile u in slot CUR: loads of tile u + 1 into slot NXT (which held tile u - 2,
    // last read a step earlier); phase A: S and dP of tile u (A = Q / dO rows, B = K^T / V^T
    // in registers; accumulators from the offsets); the mask; phase C: the contraction of
    // tile u - 1 (slot PRV; none in the first step), written with the softmax of one (d =
    // 64: two) of the lane's 16 elements of tile u after each MFMA (the compiler moves the
    // exponentials after the last MFMA, next to the packing; pinned in place they ran no
    // faster: the two waves of a SIMD overlap each other's softmax); then P and dS of tile u
    // are packed, one kept, the other handed over. A wave whose queries all precede its keys
    // (causal, the first two tiles) computes fully masked blocks (P = dS = 0): the step's
    // length is set by the other waves.
    auto step = [&](auto CUR, auto PRV, auto NXT, auto FIRST, int u) __attribute__((always_inline)) {
      constexpr bool FST = decltype(FIRST)::value;
      constexpr int SC = decltype(CUR)::value;
      if (u + 1 < n_qtiles) {
        rp.load(Qh, (u + 1) * kBQ, N, qbuf(NXT), wave);
        rp.load(dOh, (u + 1) * kBQ, N, gbuf(NXT), wave);
        load_ld(u + 1, NXT);
      }
      const uint8_t* qt = qbuf(CUR);
      const uint8_t* gt = gbuf(CUR);
#pragma unroll
      for (int g = 0; g < 4; ++g) {                 // element 4g + e: query qr + 8g + 4 half + e
        const f32x4 a = *(const f32x4*)&lsd[SC][0][qr + g * 8 + half * 4];
        const f32x4 b = *(const f32x4*)&lsd[SC][1][qr + g * 8 + half * 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[g * 4 + e] = a[e];
          dp[g * 4 + e] = b[e];
        }
      }
      u32x4 fq[2], fg[2];
      fq[0] = row_frag<D>(qt, ta, qr, 0);
      fg[0] = row_frag<D>(gt, ta, qr, 0);
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        if (st + 1 < NSTEP) {
          fq[(st + 1) % 2] = row_frag<D>(qt, ta, qr, st + 1);
          fg[(st + 1) % 2] = row_frag<D>(gt, ta, qr, st + 1);
        }
        s = mfma32(Tag{}, fq[st % 2], kreg[st], s);
        dp = mfma32(Tag{}, fg[st % 2], vreg[st], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int qb0 = u * kBQ + qr;
      if ((CAUSAL && qb0 < k0 + 31) || qb0 + 32 > N) {
        // queries before this lane's key (causal) or past the sequence: element r is
        // query qb0 + 8 * (r / 4) + 4 * half + r % 4
        const int lo = (CAUSAL ? krow : 0) - qb0 - half * 4, hi = N - 1 - qb0 - half * 4;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = (r / 4) * 8 + (r % 4);
          if (o < lo || o > hi) s[r] = -INFINITY;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      float p[16], ds[16];
      u32x4 fa[3], other[2];
      if constexpr (!FST) {
        read_other(u - 1, other);
        fa[0] = frag(PRV, 0);
        fa[1] = frag(PRV, 1);
      }
#pragma unroll
      for (int i = 0; i < NMV; ++i) {
        if constexpr (!FST) {
          if (i + 2 < NMV) fa[(i + 2) % 3] = frag(PRV, i + 2);
          mfma_i(i, fa[i % 3], other);
        }
#pragma unroll
        for (int r = i * EPM; r < (i + 1) * EPM; ++r) {
          p[r] = fast_exp2(s[r] * c);
          ds[r] = p[r] * dp[r];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      u32x4 give[2];
      pack16<Tag>(RV ? p : ds, keep);
      pack16<Tag>(RV ? ds : p, give);
#pragma unroll
      for (int j = 0; j < 2; ++j) xch[u & 1][wave][j][lane] = give[j];
      wait_vmcnt<0>();
      barrier_lds();
    };

    rp.load(Qh, u0 * kBQ, N, qbuf(IC<0>{}), wave);   // u0 < n_qtiles: the tile's first key is < N
    rp.load(dOh, u0 * kBQ, N, gbuf(IC<0>{}), wave);
    load_ld(u0, IC<0>{});
    wait_vmcnt<0>();
    barrier_lds();
    using T1 = std::true_type;
    using F0 = std::false_type;
    step(IC<0>{}, IC<2>{}, IC<1>{}, T1{}, u0);
    for (int u = u0 + 1; u < n_qtiles; u += 3) {   // tile u in slot (u - u0) mod 3
      step(IC<1>{}, IC<0>{}, IC<2>{}, F0{}, u);
      if (u + 1 < n_qtiles) step(IC<2>{}, IC<1>{}, IC<0>{}, F0{}, u + 1);
      if (u + 2 < n_qtiles) step(IC<0>{}, IC<2>{}, IC<1>{}, F0{}, u + 2);
    }
    // the last tile's contraction, from its slot
    const int ul = n_qtiles - 1, last = (ul - u0) % 3;
    if (last == 0) contract(IC<0>{}, ul);
    else if (last == 1) contract(IC<1>{}, ul);
    else contract(IC<2>{}, ul);
    barrier_lds();                                  // every wave has read the rings and xch
    static_assert(W * 32 * D * 2 <= 2 * NS * TB, "the staged rows fit the rings");
    uint8_t* stg = lds + wave * 32 * D * 2;
    if constexpr (RV) store_rows_staged<Tag, D>(dV + head_off + (int64_t)k0 * D, N - k0, acc, lane, 1.f, stg);
    else store_rows_staged<Tag, D>(dK + head_off + (int64_t)k0 * D, N - k0, acc, lane, scale, stg);
  };
  if (qh == 0) run(IC<0>{});
  else run(IC<1>{});
}

template <typename Tag, int D, bool CAUSAL>
hipError_t launch_one(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, float* ws, int64_t BH, int64_t N, float scale, hipStream_t stream) {
  const int64_t rows = BH * N;
  const float c = scale * kLog2e;
  const int n_mtiles = (int)((N + kWq * 32 - 1) / (kWq * 32));
  const int64_t total_q = BH * n_mtiles;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<Tag, D, CAUSAL>), dim3((unsigned)total_q), dim3(kWq * 64), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout,
                     (const uint16_t*)o, lse, ws, (uint16_t*)dq, (int)N, n_mtiles, (int)total_q, rows, c, scale);
  const int n_ntiles = (int)((N + kKG * 32 - 1) / (kKG * 32));
  const int64_t total_k = BH * n_ntiles;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<Tag, D, CAUSAL>), dim3((unsigned)total_k), dim3(kWk * 64), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)dout, ws,
                     (uint16_t*)dk, (uint16_t*)dv, (int)N, n_ntiles, (int)total_k, rows, c, scale);
  return hipGetLastError();
}

template <typename Tag>
hipError_t launch_16bit(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, float* ws, int64_t BH, int64_t N, int64_t d,
                        bool causal, float scale, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_one<Tag, 128, true>(q, k, v, o, lse, dout, dq, dk, dv, ws, BH, N, scale, stream)
                  : launch_one<Tag, 128, false>(q, k, v, o, lse, dout, dq, dk, dv, ws, BH, N, scale, stream);
  return causal ? launch_one<Tag, 64, true>(q, k, v, o, lse, dout, dq, dk, dv, ws, BH, N, scale, stream)
                : launch_one<Tag, 64, false>(q, k, v, o, lse, dout, dq, dk, dv, ws, BH, N, scale, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, float* ws, int64_t BH, int64_t N, int64_t d,
                           bool causal, float scale, hipStream_t stream) {
  return launch_16bit<Bf16Tag>(q, k, v, o, lse, dout, dq, dk, dv, ws, BH, N, d, causal, scale, stream);
}

hipError_t launch_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, float* ws, int64_t BH, int64_t N, int64_t d,
                          bool causal, float scale, hipStream_t stream) {
  return launch_16bit<F16Tag>(q, k, v, o, lse, dout, dq, dk, dv, ws, BH, N, d, causal, scale, stream);
}

int64_t max_workgroups_bwd(int64_t BH, int64_t N) {
  const int64_t a = BH * ((N + kWq * 32 - 1) / (kWq * 32));
  const int64_t b = BH * ((N + kKG * 32 - 1) / (kKG * 32));
  return a > b ? a : b;
}

}  // namespace attn
