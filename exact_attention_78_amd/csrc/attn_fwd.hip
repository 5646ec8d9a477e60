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
//   Software pipeline three tiles deep: step t issues the P.V MFMAs of tile t, the
//   softmax of tile t+1 and the S^T MFMAs of tile t+2, which do not depend on each other,
//   so the matrix core and the VALU work side by side (the intra-warpgroup overlap of
//   "8.3 FlashAttention-3", section 4, taken one stage further inside one wave). The
//   step's MFMAs, LDS reads and VALU work are written in the order they are issued.
//   K and V tiles sit in two 4-slot LDS rings (128 KiB at d = 128), filled by direct
//   global->LDS loads (global_load_lds_dwordx4) two or three steps ahead of their use.
//   A call runs a fast pass that keeps the first tile's row max as the softmax reference
//   for every tile; a workgroup whose probabilities outgrew that reference redoes its
//   query tile at once with the exact pass (a per-tile running max). The exact pass can
//   also be asked to run alone, on every tile.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kBN = 64;        // keys per tile
constexpr int kWaves = 8;      // waves per workgroup (32 query rows each)
constexpr int kKD = 4;         // S^T MFMAs by which a K fragment read runs ahead
constexpr int kVD = 2;         // P.V MFMAs by which a V fragment read runs ahead
constexpr int kTail = 1;       // last MFMAs of a step that carry no exponentials (they cover the step's last sums and packing)
constexpr float kTau = 8.0f;   // lazy-rescale threshold for the running max, in log2 units
// The fast pass computes no per-tile row max: every tile uses the max of the first tile,
// which softmax allows (the result does not depend on the reference value) as long as
// the probabilities stay representable. A row whose probabilities relative to it reach
// the guard (a partial row sum above it, or not finite) marks its query tile, and the
// workgroup then redoes that tile with the exact pass, a per-tile max, before it leaves
// (one launch per call: a second launch over all tiles, most of which would leave at
// once, cost ~1-4% more, measured). The guard, 2^8
// on each lane's partial sum of a tile (32 probabilities), keeps every probability of the
// fast pass within the range the exact pass allows (P <= 2^kTau against its running
// max), so rounding P to 16 bits costs the fast pass no more accuracy than the exact
// pass: when one key dominates a row, its rounded weight enters O while the row sum uses
// the unrounded one, and a weight far above the reference (P ~ 2^50 after a jump in the
// scores) would carry the full 2^-9 relative rounding of bf16 into O; the exact pass
// instead moves its max onto such a key, whose weight is then exactly 1. The guard is
// far from 16-bit overflow, and on N(0,1) inputs the largest partial sum against the
// first tile's max stays below 2^6.5, so such inputs are not marked.
constexpr float kGuard = 256.0f;                     // 2^kTau

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

template <typename Tag, int D, bool CAUSAL, int W, bool FAST, bool PERSIST>
__global__ __launch_bounds__(W * 64, 1) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_mtiles, int total_wg, float c /* scale*log2 e */,
    int order /* TileOrder of a plain grid */, int persist /* PERSIST: 1 fixed stride, 2 queue */,
    int* __restrict__ queue /* persist 2: 8 tile counters, then 8 exit counts */) {
  constexpr int BM = W * 32;                        // query rows per workgroup
  constexpr int NSTEP = D / 16;                     // MFMA k-steps over the head dim
  constexpr int NKB = kBN / 32;                     // 32-key blocks per tile
  constexpr int NDB = D / 32;                       // 32-wide head-dim blocks of O
  constexpr int ROW = D * 2;                        // bytes per K/V row
  constexpr int TB = kBN * ROW;                     // bytes per K (or V) tile
  constexpr int LPW = TB / 1024 / W;                // 1 KiB direct loads per wave per tile
  constexpr int NS = 4;                             // ring slots per operand
  static_assert(LPW >= 1 && LPW * 1024 * W == TB, "tile must split into whole 1 KiB loads per wave");
  // V ring first, then K ring: the 32 V transpose reads of a step then fit the 16-bit
  // immediate offset of ds_read (< 64 KiB) with no address add; the K reads need one add
  // per head-dim step.
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * NS * TB];
  __shared__ int marked;                            // fast pass: some wave of the tile is marked
  __shared__ int stop[2];                           // fast pass: some wave is marked (by step parity)
  __shared__ int ticket[2];                         // persistent grids: current and next ticket
  // Static persistent orders, ticket = index into the XCD's tiles (default order, longest
  // first when causal): the fixed stride (persist 1) takes every P-th tile (P workgroups per
  // XCD); the snake (persist 3) deals them round by round, forward in even rounds and
  // backward in odd ones, so that the workgroup with the longest tile of one round gets the
  // shortest of the next (with tile lengths that fall evenly, every workgroup gets the same
  // total, as a queue that hands the next tile to whoever finishes first would do).
  auto next_static = [&](int tk) __attribute__((always_inline)) -> int {
    const int P = gridDim.x / 8, j = blockIdx.x / 8;
    if (persist == 1) return tk + P;
    const int r = tk / P + 1;
    return r * P + (r % 2 == 0 ? j : P - 1 - j);
  };
  u32x4 qreg[NSTEP];                                // Q^T as the B operand, resident (persistent grids:
                                                    // the next tile's rows arrive while a tile ends)

  // One query tile (batch*head, m-tile), by the fast pass (FASTP) or the exact pass.
  // Persistent grids (fast pass): pf_in says that the previous tile of this workgroup has
  // already loaded this tile's Q rows (into qreg) and its first K / V tiles (into the
  // rings). draw >= 0: this tile draws the workgroup's next ticket into ticket[draw], as
  // late as it can, so that the queue still hands tiles out in the order the workgroups
  // finish them: the fast pass, when its own tile count is a multiple of 4 (the ring slots
  // then line up), draws it four steps before its end and loads the next tile's Q and first
  // K / V tiles during its last four steps; otherwise a tile draws it after its loop.
  // Returns whether it loaded the next tile's data.
  auto tile = [&](auto fast_c, const int bh, const int mt, const bool pf_in, const int draw)
                  __attribute__((always_inline)) -> bool {
    constexpr bool FASTP = decltype(fast_c)::value;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64;
    const int half = lane / 32, l32 = lane % 32;
    const int64_t head_off = (int64_t)bh * N * D;
    const uint16_t* Qh = Q + head_off;
    const uint16_t* Kh = K + head_off;
    const uint16_t* Vh = V + head_off;

    const int q0 = mt * BM + wave * 32;               // this wave's 32 rows; one per lane (and lane^32)
    const int qrow = q0 + l32;
    if constexpr (FASTP) {
      if (tid == 0) {                                   // read only after the prologue's barriers
        stop[0] = 0;
        stop[1] = 0;
        marked = 0;
      }
    }
    auto load_q = [&](const uint16_t* Qb, int row) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
        qreg[s] = row < N ? *(const u32x4*)(Qb + (int64_t)row * D + s * 16 + half * 8) : u32x4{0, 0, 0, 0};
    };
    if (!(PERSIST && FASTP && pf_in)) load_q(Qh, qrow);

    const int n_ktiles = (N + kBN - 1) / kBN;
    auto tiles_of = [&](int m) __attribute__((always_inline)) {
      return CAUSAL ? min(n_ktiles, ((m + 1) * BM + kBN - 1) / kBN) : n_ktiles;
    };
    const int T = tiles_of(mt);
    // the next tile (persistent fast pass): cap, this tile runs its last four steps apart
    // (they can load the next tile's first data); pfo, it does load it (the next ticket is
    // valid); the next tile's head offset, m-tile and tile count, looked up from its ticket
    // after the main loop, so that nothing of it stays live through the loop
    const bool cap = FASTP && (!PERSIST || draw >= 0) && T % 4 == 0;
    bool pfo = false;
    int64_t nhead_off = 0;
    int nmt = 0, nT = 1;
    auto next_tile = [&]() __attribute__((always_inline)) -> bool {
      const int64_t wl = (int64_t)ticket[draw] * 8 + blockIdx.x % 8;
      if (wl < 0 || wl >= total_wg) return false;
      int nbh;
      query_tile_ordered(kOrderXcdPairs, (int)wl, total_wg, n_mtiles, CAUSAL, nbh, nmt);
      nhead_off = (int64_t)nbh * N * D;
      nT = tiles_of(nmt);
      return true;
    };
    // the next ticket (persistent grids): from the XCD's queue, the fixed stride or the snake; thread
    // 0 writes it to LDS for the other waves (after a wait for loads that covers it)
    int tnext = 0;
    bool drawn = false;
    auto draw_ticket = [&]() __attribute__((always_inline)) {
      if (tid == 0) tnext = persist == 2 ? atomicAdd(queue + blockIdx.x % 8, 1) : next_static(ticket[draw ^ 1]);
      drawn = true;
    };
    auto publish = [&]() __attribute__((always_inline)) {
      if (tid == 0) ticket[draw] = tnext;
    };
    if constexpr (PERSIST && FASTP) {
      if (cap && T < 8) draw_ticket();          // no main loop: drawn before the prologue's loads
    }

    uint32_t kaddr[NSTEP];
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) kaddr[s] = NS * TB + l32 * ROW + (((2 * s + half) ^ Swz<D>::k(l32)) << 4);
    const int g16 = lane / 16, i16 = lane % 16;
    const int tr_row = (g16 / 2) * 4 + i16 / 4;
    const int tr_col = 16 * (g16 % 2) + 4 * (i16 % 4);
    uint32_t vaddr[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int col = db * 32 + tr_col;
      vaddr[db] = tr_row * ROW + ((((col >> 3) ^ Swz<D>::v(tr_row))) << 4) + ((col & 7) << 1);
    }

    int ld_row[LPW], ld_kch[LPW], ld_vch[LPW], ld_koff[LPW], ld_voff[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int slot = (wave * LPW + i) * 1024 + lane * 16;
      const int r = slot / ROW, phys = (slot % ROW) / 16;
      ld_row[i] = r;
      ld_kch[i] = (phys ^ Swz<D>::k(r)) * 8;
      ld_vch[i] = (phys ^ Swz<D>::v(r)) * 8;
      ld_koff[i] = (ld_row[i] * D + ld_kch[i]) * 2;
      ld_voff[i] = (ld_row[i] * D + ld_vch[i]) * 2;
    }
    // K slot SLOT is at lds + (NS + SLOT) * TB; reads add the ring base through kaddr (a
    // register), so that only SLOT * TB + the 32-key block offset is an immediate.
    auto kbuf = [&](auto SLOT) __attribute__((always_inline)) -> uint8_t* {
      return lds + (NS + decltype(SLOT)::value) * TB;
    };
    auto kread_base = [&](auto SLOT) __attribute__((always_inline)) -> const uint8_t* {
      return lds + decltype(SLOT)::value * TB;
    };
    auto vbuf = [&](auto SLOT) __attribute__((always_inline)) -> uint8_t* { return lds + decltype(SLOT)::value * TB; };
    auto load_tile = [&](const uint16_t* src, const int (&off)[LPW], const int (&ch)[LPW], int kt, uint8_t* dst)
                         __attribute__((always_inline)) {
      if (kt * kBN + kBN <= N) {
        const uint8_t* base = (const uint8_t*)(src + (int64_t)kt * kBN * D);
#pragma unroll
        for (int i = 0; i < LPW; ++i) dma_load16(base + off[i], lds_u32(dst) + (wave * LPW + i) * 1024);
      } else {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
          const int key = min(kt * kBN + ld_row[i], N - 1);
          dma_load16(src + (int64_t)key * D + ch[i], lds_u32(dst) + (wave * LPW + i) * 1024);
        }
      }
    };

    auto qk = [&](auto SLOT, f32x16 (&S)[NKB]) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        S[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < NSTEP; ++s)
          S[kb] = mfma32(Tag{}, *(const u32x4*)(kread_base(SLOT) + kb * 32 * ROW + kaddr[s]), qreg[s], S[kb]);
      }
    };
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    // Running max M (log2 units; raised only when a tile's max exceeds it by more than
    // kTau, so that probabilities stay below 2^kTau), this lane's partial row sum of the
    // fp32 probabilities (before their rounding to 16 bits), and a pending O rescale factor.
    float M = -INFINITY, l_part = 0.f, alpha_pend = 1.f;
    // Scores of tile u that lie above the diagonal or past the end of the sequence -> -inf.
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
    // Row max of a tile's (masked) scores: max_pairs folds the score pairs in [e_begin,
    // e_end) into four v_maximum3 chains (seeded with scores 0..3); max_final combines the
    // chains and the partner lane l^32 and scales to log2 units.
    auto max_pairs = [&](float (&m4)[4], const f32x16 (&S)[NKB], int e_begin, int e_end) __attribute__((always_inline)) {
#pragma unroll
      for (int e = e_begin; e < e_end; e += 2)
        m4[(e / 2) % 4] = max3f(m4[(e / 2) % 4], S[e / 16][e % 16], S[e / 16][e % 16 + 1]);
    };
    // Raise M when some row of the wave grew by more than kTau (branch-free, so that the
    // exponentials can share a basic block with the MFMAs); l is rescaled at once, O at
    // the start of the next step. Returns whether M moved (wave-uniform).
    auto max_final = [&](const float (&m4)[4]) __attribute__((always_inline)) -> bool {
      const float mx = max_halves(max3f(m4[0], m4[1], __builtin_elementwise_maximum(m4[2], m4[3]))) * c;
      const bool grow = __builtin_amdgcn_ballot_w64(mx > M + kTau) != 0;
      const float M_new = grow ? __builtin_elementwise_maximum(M, mx) : M;
      const float alpha = grow ? fast_exp2(M - M_new) : 1.f;
      M = M_new;
      l_part *= alpha;
      alpha_pend *= alpha;
      return grow;
    };
    // Probabilities of scores e in [e0, e1): P = 2^(S*c - M) in fp32, written over the
    // scores (exps); later, so that the exponentials' latency is covered, their row sum
    // (two chains, before rounding) and the rounding to 16 bits, packed in pairs into the
    // B operand of P.V (finish).
    auto args = [&](f32x16 (&S)[NKB], int e0, int e1) __attribute__((always_inline)) {   // S*c - M
#pragma unroll
      for (int e = e0; e < e1; ++e) S[e / 16][e % 16] = __builtin_fmaf(S[e / 16][e % 16], c, -M);
    };
    auto exps = [&](f32x16 (&S)[NKB], int e0, int e1) __attribute__((always_inline)) {     // 2^(S*c - M)
#pragma unroll
      for (int e = e0; e < e1; ++e) S[e / 16][e % 16] = fast_exp2(S[e / 16][e % 16]);
    };
    auto finish = [&](const f32x16 (&S)[NKB], u32x4 (&P)[NKB][2], float (&lsum)[2], int e0, int e1)
                      __attribute__((always_inline)) {
#pragma unroll
      for (int e = e0; e < e1; ++e) {
        lsum[e % 2] = e < 2 ? S[e / 16][e % 16] : lsum[e % 2] + S[e / 16][e % 16];   // chains start at e = 0, 1
        if (e % 2 == 1) P[e / 16][(e % 16) / 8][(e % 8) / 2] = pack2(Tag{}, S[e / 16][e % 16 - 1], S[e / 16][e % 16]);
      }
    };
    auto rescale_o = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha_pend;
      alpha_pend = 1.f;
    };

    f32x16 Sa[NKB], Sb[NKB];
    u32x4 Pa[NKB][2], Pb[NKB][2];
    bool pend = false;     // wave-uniform: an O rescale is owed
    bool ovf = false;      // fast pass: a probability of this lane reached the guard

    // Step t (j = t mod 4 fixes every register set and ring slot at compile time):
    //   S(t+1) in S_soft, S(t+2) -> S_new, P(t) in P_use, P(t+1) -> P_new,
    //   K(t+2) in K slot (t+2)%4, V(t) in V slot t%4; loads: K(t+4) -> K slot t%4,
    //   V(t+3) -> V slot (t+3)%4. Past the last tile the loads are clamped (never read),
    //   and the scores of tile T (if computed) are fully masked, so P(T) = 0 adds nothing.
    // K(t+4) and V(t+3) of a step; past the last tile, the next tile's first tiles when
    // this tile loads them (pfo), else the last tile again (never read)
    auto kv_loads = [&](int t, auto KLD, auto VLD, auto ROUTEc) __attribute__((always_inline)) {
      if (decltype(ROUTEc)::value && pfo && t + 4 >= T) load_tile(K + nhead_off, ld_koff, ld_kch, min(t + 4 - T, nT - 1), kbuf(KLD));
      else load_tile(Kh, ld_koff, ld_kch, min(t + 4, T - 1), kbuf(KLD));
      if (decltype(ROUTEc)::value && pfo && t + 3 >= T) load_tile(V + nhead_off, ld_voff, ld_vch, min(t + 3 - T, nT - 1), vbuf(VLD));
      else load_tile(Vh, ld_voff, ld_vch, min(t + 3, T - 1), vbuf(VLD));
    };
    auto step = [&](int t, f32x16 (&S_soft)[NKB], f32x16 (&S_new)[NKB], const u32x4 (&P_use)[NKB][2],
                    u32x4 (&P_new)[NKB][2], auto KRD, auto VRD, auto KLD, auto VLD, auto ROUTEc)
                    __attribute__((always_inline)) {
      kv_loads(t, KLD, VLD, ROUTEc);
      // Causal: once the tile's first key lies past this wave's last row, this and every
      // later tile are fully masked for the wave; it only keeps up its loads and barriers.
      if (!CAUSAL || t * kBN <= q0 + 31) {
        if constexpr (!FASTP) {
          if (pend) rescale_o();
        }
        mask_tile(t + 1, S_soft);
        // Main block, written in issue order (this file is compiled without the machine
        // scheduler): 16 S^T MFMAs (K fragments read KD ahead) then 16 P.V MFMAs (V^T
        // fragments read VD ahead); the softmax VALU work of tile t+1 is spread between them:
        // (exact pass) the row max over the first five S^T MFMAs, then the exponentials,
        // one or two per MFMA; (fast pass) the exponentials from the second MFMA on.
        constexpr int NQ = NKB * NSTEP, NP = NDB * NKB * 2, KD = kKD, VD = kVD;
        constexpr int NMAX = FASTP ? 1 : 5;                 // MFMAs before the first exponential
        constexpr int NSLOT = NQ + NP - NMAX - kTail;      // MFMAs that carry exponentials
        u32x4 kf[NQ], vf[NP];
        auto kread = [&](int i) __attribute__((always_inline)) {   // i = s * NKB + kb
          kf[i] = *(const u32x4*)(kread_base(KRD) + (i % NKB) * 32 * ROW + kaddr[i / NKB]);
        };
        auto vread = [&](int i) __attribute__((always_inline)) {   // i = (kb * 2 + h) * NDB + db
          const int db = i % NDB, kb = i / (2 * NDB), h = (i / NDB) % 2;
          const uint8_t* base = vbuf(VRD) + (kb * 32 + h * 16) * ROW + vaddr[db];
          const u32x2 v1 = lds_read_tr16((const uint16_t*)base);
          const u32x2 v2 = lds_read_tr16((const uint16_t*)(base + 8 * ROW));
          vf[i] = u32x4{v1[0], v1[1], v2[0], v2[1]};
        };
        float m4[4] = {S_soft[0][0], S_soft[0][1], S_soft[0][2], S_soft[0][3]};
        float lsum[2] = {0.f, 0.f};
        // slot k: arguments of slot k+1, exponentials of slot k, sums and packing of slot k-1
        auto lo = [&](int slot) __attribute__((always_inline)) { return min(slot * (NKB * 16) / NSLOT, NKB * 16); };
        auto exps_slot = [&](int slot) __attribute__((always_inline)) {
          if (slot + 1 < NSLOT) args(S_soft, lo(slot + 1), lo(slot + 2));
          exps(S_soft, lo(slot), lo(slot + 1));
          if (slot > 0) finish(S_soft, P_new, lsum, lo(slot - 1), lo(slot));
        };
#pragma unroll
        for (int i = 0; i < KD; ++i) kread(i);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          if (i + KD < NQ) kread(i + KD);
          if (i + KD >= NQ && i + KD - NQ < VD) vread(i + KD - NQ);
          const int kb = i % NKB, s = i / NKB;
          S_new[kb] = mfma32(Tag{}, kf[i], qreg[s], s == 0 ? f32x16{} : S_new[kb]);
          if (i < NMAX - 1) {
            max_pairs(m4, S_soft, 4 + i * 8, min(4 + (i + 1) * 8, NKB * 16));
          } else if (i == NMAX - 1) {
            if constexpr (!FASTP) pend = max_final(m4);
            args(S_soft, lo(0), lo(1));
          } else {
            exps_slot(i - NMAX);
          }
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          if (i + VD < NP) vread(i + VD);
          const int db = i % NDB, kb = i / (2 * NDB), h = (i / NDB) % 2;
          oacc[db] = mfma32(Tag{}, vf[i], P_use[kb][h], oacc[db]);
          exps_slot(NQ - NMAX + i);
        }
        if constexpr (kTail == 0) finish(S_soft, P_new, lsum, lo(NSLOT - 1), NKB * 16);
        const float lt = lsum[0] + lsum[1];
        l_part += lt;
        if constexpr (FASTP) ovf |= !(lt <= kGuard);
      }
      if constexpr (FASTP) {
        // a marked wave dooms the whole query tile to the exact pass: say so to the others
        if (__builtin_amdgcn_ballot_w64(ovf) != 0 && lane == 0) stop[t & 1] = 1;
      }
      wait_vmcnt<2 * LPW>();   // K(t+3) and V(t+1), issued a step earlier, have landed
      barrier_lds();
    };

    // The last two steps of a tile that loads its successor (pfo: T a multiple of 4, fast
    // pass), with no S^T MFMAs (the tiles T and T+1 they would compute do not exist), so
    // that qreg is free: DRAIN 1 (t = T-2) loads the next tile's Q rows into qreg and runs
    // the softmax of tile T-1 beside the P.V MFMAs of tile T-2; DRAIN 2 (t = T-1) runs the
    // P.V MFMAs of tile T-1. Neither waits for loads: nothing reads the rings again before
    // the next tile's prologue, which waits for all of them.
    auto drain = [&](auto DRc, int t, f32x16 (&S_soft)[NKB], const u32x4 (&P_use)[NKB][2], u32x4 (&P_new)[NKB][2],
                     auto VRD, auto KLD, auto VLD) __attribute__((always_inline)) {
      constexpr int DR = decltype(DRc)::value;
      if constexpr (DR == 1) {
        if (pfo) load_q(Q + nhead_off, nmt * BM + wave * 32 + l32);
      }
      kv_loads(t, KLD, VLD, std::true_type{});
      if (!CAUSAL || t * kBN <= q0 + 31) {
        constexpr int NP = NDB * NKB * 2, VD = kVD;
        constexpr int NSL = NP - kTail;                  // P.V MFMAs that carry exponentials
        u32x4 vf[NP];
        auto vread = [&](int i) __attribute__((always_inline)) {   // i = (kb * 2 + h) * NDB + db
          const int db = i % NDB, kb = i / (2 * NDB), h = (i / NDB) % 2;
          const uint8_t* base = vbuf(VRD) + (kb * 32 + h * 16) * ROW + vaddr[db];
          const u32x2 v1 = lds_read_tr16((const uint16_t*)base);
          const u32x2 v2 = lds_read_tr16((const uint16_t*)(base + 8 * ROW));
          vf[i] = u32x4{v1[0], v1[1], v2[0], v2[1]};
        };
        float lsum[2] = {0.f, 0.f};
        auto lo = [&](int slot) __attribute__((always_inline)) { return min(slot * (NKB * 16) / NSL, NKB * 16); };
        if constexpr (DR == 1) {
          mask_tile(t + 1, S_soft);
          args(S_soft, lo(0), lo(1));
        }
#pragma unroll
        for (int i = 0; i < VD; ++i) vread(i);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          if (i + VD < NP) vread(i + VD);
          const int db = i % NDB, kb = i / (2 * NDB), h = (i / NDB) % 2;
          oacc[db] = mfma32(Tag{}, vf[i], P_use[kb][h], oacc[db]);
          if constexpr (DR == 1) {
            if (i < NSL) {
              if (i + 1 < NSL) args(S_soft, lo(i + 1), lo(i + 2));
              exps(S_soft, lo(i), lo(i + 1));
              if (i > 0) finish(S_soft, P_new, lsum, lo(i - 1), lo(i));
            }
          }
        }
        if constexpr (DR == 1) {
          finish(S_soft, P_new, lsum, lo(NSL - 1), NKB * 16);
          const float lt = lsum[0] + lsum[1];
          l_part += lt;
          ovf |= !(lt <= kGuard);
        }
      }
      if (__builtin_amdgcn_ballot_w64(ovf) != 0 && lane == 0) stop[t & 1] = 1;
      barrier_lds();
    };

    // Prologue: K tiles 0..3 and V tiles 0..2 (unless the previous tile loaded them); S(0),
    // softmax of tile 0, S(1).
    if (!(PERSIST && FASTP && pf_in)) {
      load_tile(Kh, ld_koff, ld_kch, 0, kbuf(IC<0>{}));
      load_tile(Kh, ld_koff, ld_kch, min(1, T - 1), kbuf(IC<1>{}));
      load_tile(Kh, ld_koff, ld_kch, min(2, T - 1), kbuf(IC<2>{}));
      load_tile(Kh, ld_koff, ld_kch, min(3, T - 1), kbuf(IC<3>{}));
      load_tile(Vh, ld_voff, ld_vch, 0, vbuf(IC<0>{}));
      load_tile(Vh, ld_voff, ld_vch, min(1, T - 1), vbuf(IC<1>{}));
      load_tile(Vh, ld_voff, ld_vch, min(2, T - 1), vbuf(IC<2>{}));
    }
    wait_vmcnt<0>();
    if constexpr (PERSIST && FASTP) {
      if (drawn) publish();
    }
    barrier_lds();
    // the next tile of this workgroup (persistent fast pass): its head's K and V, its tile
    // count and whether this tile loads its first tiles
    qk(IC<0>{}, Sa);
    {
      mask_tile(0, Sa);
      float m4[4] = {Sa[0][0], Sa[0][1], Sa[0][2], Sa[0][3]};
      max_pairs(m4, Sa, 4, NKB * 16);
      max_final(m4);
      alpha_pend = 1.f;            // O is still zero: no rescale owed
      float lsum[2] = {0.f, 0.f};
      args(Sa, 0, NKB * 16);
      exps(Sa, 0, NKB * 16);
      finish(Sa, Pa, lsum, 0, NKB * 16);
      l_part += lsum[0] + lsum[1];
    }
    qk(IC<1>{}, Sb);
    barrier_lds();                 // K slots 0 and 1 are refilled from step 0 on

    int t_end = T;
    const int t_main = cap ? T - 4 : T;                // cap: the last four steps follow the loop
    for (int t = 0; t < min(t_end, t_main); t += 4) {
      using F0 = std::false_type;
      step(t, Sb, Sa, Pa, Pb, IC<2>{}, IC<0>{}, IC<0>{}, IC<3>{}, F0{});
      if (t + 1 < T) step(t + 1, Sa, Sb, Pb, Pa, IC<3>{}, IC<1>{}, IC<1>{}, IC<0>{}, F0{});
      if (t + 2 < T) step(t + 2, Sb, Sa, Pa, Pb, IC<0>{}, IC<2>{}, IC<2>{}, IC<1>{}, F0{});
      if (t + 3 < T) {
        // cap: step T-5 draws the next ticket, published before the last four steps
        const bool dr = PERSIST && FASTP && cap && t + 4 == t_main;
        if constexpr (PERSIST && FASTP) {
          if (dr) draw_ticket();
        }
        step(t + 3, Sa, Sb, Pb, Pa, IC<1>{}, IC<3>{}, IC<3>{}, IC<2>{}, F0{});
        if constexpr (PERSIST && FASTP) {
          if (dr) {
            publish();
            barrier_lds();
          }
        }
      }
      // Fast pass: once some wave is marked, the tile is left to the exact pass. stop[1]
      // was last written in step t+3 (or t+1) before its barrier and is next written in
      // step t+5, after the barrier of step t+4, so every wave reads the same value here
      // and all leave the loop together.
      if constexpr (FASTP) {
        if (stop[1] != 0) t_end = t + 4;
      }
    }
    bool pf_out = false;
    if constexpr (FASTP) {
      if (cap && t_end == T) {     // not stopped: the last four steps (persistent: they load the next tile)
        if constexpr (PERSIST) pfo = next_tile();
        const int t = T - 4;
        step(t, Sb, Sa, Pa, Pb, IC<2>{}, IC<0>{}, IC<0>{}, IC<3>{}, std::true_type{});
        step(t + 1, Sa, Sb, Pb, Pa, IC<3>{}, IC<1>{}, IC<1>{}, IC<0>{}, std::true_type{});
        drain(IC<1>{}, t + 2, Sb, Pa, Pb, IC<2>{}, IC<2>{}, IC<1>{});
        drain(IC<2>{}, t + 3, Sa, Pb, Pa, IC<3>{}, IC<3>{}, IC<2>{});
        pf_out = pfo;
      }
    }
    if constexpr (PERSIST) {
      if (draw >= 0 && !drawn) {   // not drawn yet: now (published by the barrier after the tile)
        draw_ticket();
        publish();
      }
    }
    // no load may still target this workgroup's LDS when it exits, or when the exact pass
    // redoes the tile (the next tile's loads, when this tile issued them, are left in flight)
    if (!pf_out) wait_vmcnt<0>();
    if (pend) rescale_o();

    const float l_tot = add_halves(l_part);
    if constexpr (FASTP) {
      if (__builtin_amdgcn_ballot_w64(ovf) != 0 && lane == 0) marked = 1;   // redo the tile exactly
    }
    const float inv = 1.0f / l_tot;                   // (rows past N are not stored)
    // this lane's 4 consecutive head dims db * 32 + g * 8 + half * 4 .. + 3 of row qrow
    auto o_piece = [&](int db, int g) __attribute__((always_inline)) -> u32x2 {
      const f32x16 a = oacc[db];
      return u32x2{pack2(Tag{}, a[g * 4 + 0] * inv, a[g * 4 + 1] * inv),
                   pack2(Tag{}, a[g * 4 + 2] * inv, a[g * 4 + 3] * inv)};
    };
    if constexpr (!PERSIST) {
      // O through LDS, so that the stores write whole rows: stored from the accumulators,
      // every instruction would put 16 bytes into each of 32 rows. Each wave stages its 32
      // rows (row-major, 16-byte chunk c of row r at chunk c ^ (r mod chunks per row)) in
      // its own 32 * ROW bytes, then stores 16 bytes per lane, 1 KiB of consecutive rows
      // per instruction. Every wave has waited for its own loads above; after the barrier
      // no load is in flight into the rings and no wave reads them any more.
      barrier_lds();
      constexpr int NCH = ROW / 16;                   // 16-byte chunks per row
      uint8_t* stg = lds + wave * 32 * ROW;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(u32x2*)(stg + l32 * ROW + (((db * 4 + g) ^ (l32 % NCH)) << 4) + half * 8) = o_piece(db, g);
      uint8_t* Ow = (uint8_t*)(O + head_off + (int64_t)q0 * D);   // the wave's 32 rows, contiguous
#pragma unroll
      for (int i = 0; i < 32 * ROW / 1024; ++i) {
        const int off = i * 1024 + lane * 16, r = off / ROW, ch = (off % ROW) / 16;
        const u32x4 x = *(const u32x4*)(stg + r * ROW + ((ch ^ (r % NCH)) << 4));
        if (q0 + r < N) *(u32x4*)(Ow + off) = x;
      }
    } else if (qrow < N) {
      uint16_t* Orow = O + head_off + (int64_t)qrow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) *(u32x2*)(Orow + db * 32 + g * 8 + half * 4) = o_piece(db, g);
    }
    const float lse = (M + __builtin_log2f(l_tot)) * kLn2;   // (a marked tile's O and LSE are rewritten)
    if (qrow < N && half == 0) LSE[(int64_t)bh * N + qrow] = lse;
    return pf_out;
  };
  // A tile that the fast pass marked is redone at once by the exact pass, in the same
  // workgroup (after the barrier no wave reads the LDS rings any more).
  // Returns whether the next tile's first loads were issued (persistent fast pass).
  auto run_tile = [&](const int bh, const int mt, const bool pf_in, const int draw) __attribute__((always_inline)) -> bool {
    if constexpr (FAST) {
      bool pf = tile(std::true_type{}, bh, mt, pf_in, draw);
      // The flag is in LDS: an LDS-only barrier publishes it. (__syncthreads() would also
      // wait for this wave's O and LSE stores to complete, several microseconds under load,
      // before the workgroup can leave.) A redo first drains those stores, since it
      // rewrites the same rows, and any loads of the next tile, since it refills the rings;
      // the next tile then loads its own.
      barrier_lds();
      if (marked != 0) {
        wait_vmcnt<0>();
        tile(std::false_type{}, bh, mt, false, -1);
        pf = false;
      }
      return pf;
    } else {
      return tile(std::false_type{}, bh, mt, false, draw);
    }
  };
  // The query tiles of this workgroup. A plain grid has one workgroup per tile, picked by
  // the tile order from the workgroup id. A persistent grid has one workgroup per CU and
  // 8 queues, one per XCD (queue x = workgroups x, x + 8, ..., which the dispatcher
  // places on XCD x): queue x serves the tiles that the default order gives XCD x, in
  // that order (longest first when causal). Its workgroups take either every P-th of them
  // (P workgroups per queue: a fixed stride, as a persistent kernel that walks its share
  // in a loop does), or the next one from the queue's counter, an atomic in caller memory.
  // A workgroup's next ticket is drawn during its current tile, so that the fast pass can
  // load the next tile's Q rows and first K / V tiles in the current tile's last steps.
  // (The plain grid is a separate instantiation without the loop, so that the compiler
  // keeps the one-tile kernel's code as it is.)
  if constexpr (!PERSIST) {
    int bh, mt;
    query_tile_ordered(order, blockIdx.x, total_wg, n_mtiles, CAUSAL, bh, mt);
    run_tile(bh, mt, false, -1);
    return;
  }
  const int xq = blockIdx.x % 8, per_q = gridDim.x / 8;
  if (threadIdx.x == 0) ticket[0] = persist == 2 ? atomicAdd(queue + xq, 1) : blockIdx.x / 8;   // round 0 of both static orders
  __syncthreads();
  bool pf = false;
  for (int par = 0;; par ^= 1) {
    // ticket[par] was published by the previous tile's prologue barrier (or the one above)
    const int64_t wl = (int64_t)ticket[par] * 8 + xq;
    if (wl < 0 || wl >= total_wg) break;   // every workgroup reaches this: the tickets only grow
    int bh, mt;
    query_tile_ordered(kOrderXcdPairs, (int)wl, total_wg, n_mtiles, CAUSAL, bh, mt);
    pf = run_tile(bh, mt, pf, par ^ 1);
    barrier_lds();                 // every wave has read this tile's flags before the next resets them
  }
  if (persist == 2 && threadIdx.x == 0) {
    // Every workgroup of queue xq has drawn its last (failing) ticket before counting its
    // exit, so the last one to exit may return the queue to zero for the next call.
    if (atomicAdd(queue + 8 + xq, 1) == per_q - 1) {
      atomicExch(queue + xq, 0);
      atomicExch(queue + 8 + xq, 0);
    }
  }
}

// Workgroups of a persistent grid: one per CU (this kernel's LDS allows one workgroup per
// CU), rounded up to a multiple of the 8 queues.
int persistent_workgroups() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  return (cus + 7) / 8 * 8;
}

template <typename Tag, int D, bool CAUSAL, int W>
hipError_t launch_one(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                      float scale, const FwdVariant& var, hipStream_t stream) {
  constexpr int BM = W * 32;
  const int n_mtiles = (int)((N + BM - 1) / BM);
  const int64_t total = BH * n_mtiles;
  // The fast pass (with the in-kernel redo of marked tiles) unless the exact pass alone is
  // asked for: on inputs that mark no tile it was 0.6-6.6% faster than the exact pass at
  // every size measured, from 4.6e7 to 5.5e11 counted FLOPs.
  const bool two_pass = var.passes != kPassesExact;
  // The plain entry points run one workgroup per tile in the default order: the persistent
  // grids, with their tiles loading their successors' first data, were within +-2% of it on
  // H, C3 and C4, faster on some boxes and slower on others.
  const int sched = var.sched != kSchedAuto ? var.sched : 0;
  const int persist = sched >= kSchedPersistentStride ? sched - kSchedPersistentStride + 1 : 0;
  const int order = persist ? 0 : sched;
  const unsigned grid = persist ? (unsigned)persistent_workgroups() : (unsigned)total;
  auto run = [&](auto FASTC, auto PERSISTC) {
    hipLaunchKernelGGL((attn_fwd_kernel<Tag, D, CAUSAL, W, decltype(FASTC)::value, decltype(PERSISTC)::value>),
                       dim3(grid), dim3(W * 64), 0, stream, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (uint16_t*)o, lse, (int)N, n_mtiles, (int)total, scale * kLog2e, order,
                       persist, var.queue);
  };
  using T1 = std::true_type;
  using F0 = std::false_type;
  if (persist) {
    if (two_pass) run(T1{}, T1{});
    else run(F0{}, T1{});
  } else {
    if (two_pass) run(T1{}, F0{});
    else run(F0{}, F0{});
  }
  return hipGetLastError();
}

template <typename Tag>
hipError_t launch_16bit(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                        int64_t d, bool causal, float scale, const FwdVariant& var, hipStream_t stream) {
  if (d == 128)
    return causal ? launch_one<Tag, 128, true, kWaves>(q, k, v, o, lse, BH, N, scale, var, stream)
                  : launch_one<Tag, 128, false, kWaves>(q, k, v, o, lse, BH, N, scale, var, stream);
  return causal ? launch_one<Tag, 64, true, kWaves>(q, k, v, o, lse, BH, N, scale, var, stream)
                : launch_one<Tag, 64, false, kWaves>(q, k, v, o, lse, BH, N, scale, var, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                           int64_t d, bool causal, float scale, hipStream_t stream, const FwdVariant& var) {
  return launch_16bit<Bf16Tag>(q, k, v, o, lse, BH, N, d, causal, scale, var, stream);
}

hipError_t launch_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                          int64_t d, bool causal, float scale, hipStream_t stream, const FwdVariant& var) {
  return launch_16bit<F16Tag>(q, k, v, o, lse, BH, N, d, causal, scale, var, stream);
}

int64_t max_workgroups_fwd16(int64_t BH, int64_t N) {
  constexpr int BM = kWaves * 32;
  return BH * ((N + BM - 1) / BM);
}

}  // namespace attn
