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
//         Delta_i = dO_i . O_i and LSE_i * log2(e) of its rows (O is read here only),
//         also written to the caller's workspace for dkdv; then K and V tiles of 64
//         keys stream through LDS (double-buffered direct loads). Per 32-key
//         block: S^T = K Q^T and dP^T = V dO^T (A = K / V rows read from LDS, B = Q^T and
//         dO^T kept in VGPRs), then P and dS in fp32 with one query row per lane (its LSE
//         and Delta are scalars), then dQ^T += K^T dS^T (A = K^T by LDS transpose reads,
//         B = dS rounded to 16 bits).
//   dkdv  one workgroup per (batch*head, 128-key tile), 8 waves: 4 key groups of 32 keys
//         x 2 halves of each 64-query tile. The tile's K and V stay in LDS, Q and dO tiles
//         stream through it. Per wave and tile: S = Q K^T and dP = dO V^T on its 32
//         queries (A = Q / dO rows, B = K^T / V^T as rows of K / V: one key per lane), P
//         and dS in fp32 with the 16 per-query LSE and Delta values of each lane read from
//         LDS, then dV^T += dO^T P and dK^T += Q^T dS (A = dO^T / Q^T by LDS transpose
//         reads, B = P / dS rounded to 16 bits). The two halves of a key group add their
//         partial dK / dV once, through LDS, at the end. Two waves per SIMD keep each
//         wave within 256 VGPRs, so MFMA results stay in VGPRs (no AGPR copies).
// The two gradient kernels each recompute S and dP, so that every gradient stays in
// registers until its one store: no fp32 partial sums or atomics in memory.
// Causal: query tiles of dq stop at the diagonal and key tiles of dkdv start at it;
// waves skip blocks that are wholly masked for them, and only blocks crossing the
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
  lse2 = qrow < N ? LSE[(int64_t)bh * N + qrow] * kLog2e : 0.f;
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
    ws[(int64_t)bh * N + qrow] = delta;
    ws[rows + (int64_t)bh * N + qrow] = lse2;
  }
  wait_vmcnt<0>();
  barrier_lds();
  for (int t = 0; t < T; t += 2) {
    step(IC<0>{}, t);
    if (t + 1 < T) step(IC<1>{}, t + 1);
  }
  if (qrow < N) store_rows<Tag, D>(dQ + head_off + (int64_t)qrow * D, acc, half, scale);
}

template <typename Tag, int D, bool CAUSAL>
__global__ __launch_bounds__(kWk * 64, 1) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ ws, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int N, int n_ntiles, int total_wg, int64_t rows, float c, float scale) {
  constexpr int W = kWk, BNK = kKG * 32, NSTEP = D / 16, NDB = D / 32;
  constexpr int TB = kBQ * D * 2;                   // bytes per Q (or dO) tile
  constexpr int TKV = BNK * D * 2;                  // bytes of the workgroup's K (or V)
  constexpr int LDS_BYTES = 4 * TB + 2 * TKV;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];   // Q slots 0, 1; dO slots 0, 1; K; V
  __shared__ __attribute__((aligned(16))) float lsd[2][2][kBQ];    // [slot][LSE*log2 e | Delta][query]
  static_assert(W == 2 * kKG && kBQ == 64, "two waves (query halves) per key group");
  static_assert(2 * kKG * NDB * 16 * 64 * 4 <= LDS_BYTES, "the final exchange fits the tiles' LDS");

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
  const float* delta_h = ws + (int64_t)bh * N;
  const float* lse2_h = ws + rows + (int64_t)bh * N;

  const int k0 = nt * BNK + kg * 32;
  const int krow = k0 + l32;

  const int n_qtiles = (N + kBQ - 1) / kBQ;
  const int u0 = CAUSAL ? (nt * BNK) / kBQ : 0;
  TileAddr<D> ta;
  ta.init(lane);

  f32x16 acck[NDB], accv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    acck[db] = f32x16{};
    accv[db] = f32x16{};
  }
  auto qbuf = [&](int slot) __attribute__((always_inline)) { return lds + slot * TB; };
  auto gbuf = [&](int slot) __attribute__((always_inline)) { return lds + (2 + slot) * TB; };
  uint8_t* const kt = lds + 4 * TB;                 // rows: the workgroup's keys (past N: row N-1, never stored)
  uint8_t* const vt = kt + TKV;
  // the first 2 * kBQ threads fetch the LSE (log2 units) and Delta of a query tile
  auto fetch_ld = [&](int u) __attribute__((always_inline)) -> float {
    const int q = min(u * kBQ + (tid % kBQ), N - 1);
    return tid < kBQ ? lse2_h[q] : delta_h[q];
  };
  static_assert(2 * kBQ <= W * 64, "one thread per fetched value");

  const int qr = qh * 32;                           // this wave's 32 queries start at row qr of each tile
  // Step u: prefetch Q/dO tile u + 1 (and its LSE / Delta) into the other slot, process
  // tile u from slot SLOT (compile-time, so the tile reads take immediate offsets), then
  // wait for the prefetch. Only blocks crossing the diagonal or the end of the sequence
  // mask scores, in one block of their own ahead of the exponentials.
  auto step = [&](auto slot_c, int u) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_c)::value;
    float pf = 0.f;
    if (u + 1 < n_qtiles) {
      load_rows<D, kBQ, W>(Qh, (u + 1) * kBQ, N, qbuf(SLOT ^ 1), wave, lane);
      load_rows<D, kBQ, W>(dOh, (u + 1) * kBQ, N, gbuf(SLOT ^ 1), wave, lane);
      if (tid < 2 * kBQ) pf = fetch_ld(u + 1);
    }
    const int qb0 = u * kBQ + qr;
    if (!CAUSAL || qb0 + 31 >= k0) {                // else: every query of the block precedes this wave's keys
      const uint8_t* qt = qbuf(SLOT);
      const uint8_t* gt = gbuf(SLOT);
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int st = 0; st < NSTEP; ++st)
        s = mfma32(Tag{}, row_frag<D>(qt, ta, qr, st), row_frag<D>(kt, ta, kg * 32, st), s);
#pragma unroll
      for (int st = 0; st < NSTEP; ++st)
        dp = mfma32(Tag{}, row_frag<D>(gt, ta, qr, st), row_frag<D>(vt, ta, kg * 32, st), dp);
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
      float p[16], ds[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qi = qr + g * 8 + half * 4;       // this lane's queries qi .. qi + 3 of the tile
        const f32x4 l4 = *(const f32x4*)&lsd[SLOT][0][qi];
        const f32x4 d4 = *(const f32x4*)&lsd[SLOT][1][qi];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = g * 4 + e;
          p[r] = fast_exp2(__builtin_fmaf(s[r], c, -l4[e]));
          ds[r] = p[r] * (dp[r] - d4[e]);
        }
      }
      u32x4 pb[2], sb[2];
      pack16<Tag>(p, pb);
      pack16<Tag>(ds, sb);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          accv[db] = mfma32(Tag{}, tr_frag<D>(gt, ta, qr + h * 16, db), pb[h], accv[db]);
          acck[db] = mfma32(Tag{}, tr_frag<D>(qt, ta, qr + h * 16, db), sb[h], acck[db]);
        }
    }
    if (u + 1 < n_qtiles && tid < 2 * kBQ) lsd[SLOT ^ 1][tid / kBQ][tid % kBQ] = pf;
    wait_vmcnt<0>();
    barrier_lds();
  };

  load_rows<D, BNK, W>(K + head_off, nt * BNK, N, kt, wave, lane);
  load_rows<D, BNK, W>(V + head_off, nt * BNK, N, vt, wave, lane);
  load_rows<D, kBQ, W>(Qh, u0 * kBQ, N, qbuf(0), wave, lane);      // u0 < n_qtiles: the tile's first key is < N
  load_rows<D, kBQ, W>(dOh, u0 * kBQ, N, gbuf(0), wave, lane);
  if (tid < 2 * kBQ) lsd[0][tid / kBQ][tid % kBQ] = fetch_ld(u0);
  wait_vmcnt<0>();
  barrier_lds();
  for (int u = u0; u < n_qtiles; u += 2) {
    step(IC<0>{}, u);
    if (u + 1 < n_qtiles) step(IC<1>{}, u + 1);
  }
  // The two query halves of a key group hold partial sums of the same dK and dV rows.
  // Half 1 hands over its dK part and half 0 its dV part through LDS (the tiles are no
  // longer read: the loop ended on a barrier); then half 0 stores dK and half 1 dV.
  // Layout: [tensor][key group][16-byte piece i of the lane's accumulators][lane].
  f32x4* xch = (f32x4*)lds;
  auto piece = [&](int which, int g, int i) __attribute__((always_inline)) -> f32x4* {
    return xch + ((which * kKG + g) * (NDB * 4) + i) * 64 + lane;
  };
  auto give = [&](const f32x16 (&a)[NDB], int which) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *piece(which, kg, db * 4 + q4) = f32x4{a[db][q4 * 4], a[db][q4 * 4 + 1], a[db][q4 * 4 + 2], a[db][q4 * 4 + 3]};
  };
  auto take = [&](f32x16 (&a)[NDB], int which) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 b = *piece(which, kg, db * 4 + q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[db][q4 * 4 + e] += b[e];
      }
  };
  if (qh == 1) give(acck, 0);
  else give(accv, 1);
  barrier_lds();
  if (qh == 0) take(acck, 0);
  else take(accv, 1);
  if (krow < N) {
    if (qh == 0) store_rows<Tag, D>(dK + head_off + (int64_t)krow * D, acck, half, scale);
    else store_rows<Tag, D>(dV + head_off + (int64_t)krow * D, accv, half, 1.f);
  }
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
