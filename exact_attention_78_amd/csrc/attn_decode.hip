// Split-KV attention for decoding on gfx950: a few query rows (Nq <= 32) against a long
// key/value cache (Nk keys), no mask.
//
// The FlashAttention-2 digest (discussion points) asks whether the query-split kernel
// still fits a decoding step's access to the key/value cache or whether a separate
// kernel is needed; with one query row per (batch, head), the forward kernel's grid
// would have one workgroup per head and leave most CUs idle while it streams the whole
// cache. This path splits the keys instead, and combines the partial results through the
// one log-sum-exp per row that the digest stores (the same identity that would merge
// results across GPUs): for key splits s with partial O_s (normalised) and LSE_s,
//     LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
// It is bound by HBM: every key and value byte is read once, and the work per byte is
// 4 Nq FLOPs per 2 bytes of K or V.
//
// Two launches:
//   split    one wave per (batch*head, key split), four waves per workgroup, each with
//            its own double-buffered LDS tiles of 32 keys filled by direct global->LDS
//            loads. Split s of n takes the tiles s, s + n, s + 2n, ... of its head, so
//            that the waves of a head stream adjacent tiles at any moment (the softmax
//            does not depend on the order of the keys); 5-8% faster than contiguous
//            chunks per split. S^T = K Q^T (A = K rows from LDS, B = Q^T of the <= 32
//            query rows in VGPRs: one query per lane), an exact online softmax (row max per tile, the
//            accumulator rescaled only when some row's max grew), O^T += V^T P^T (V^T by
//            LDS transpose reads, P rounded to 16 bits); writes O_s / l_s (fp32) and LSE_s
//            to the caller's workspace.
//   combine  one workgroup per (batch*head, query row): the weights exp(LSE_s - LSE) and
//            the weighted sum of the O_s (splits spread over 8 (d=128) or 16 (d=64)
//            groups of threads, added through LDS), rounded once to 16 bits.
#include <mutex>

#include "device_common.h"
#include "launch.h"
#include "tile_lds.h"

namespace attn {
namespace {

constexpr int kDW = 4;            // waves (key splits) per workgroup
constexpr int kKT = 32;           // keys per tile
constexpr int kTargetWaves = 2048;
constexpr int kCombineThreads = 256;

// Key splits: n_split = ceil(Nk / chunk) with chunk a multiple of kKT, so that every
// split holds at least one tile (n_split <= the number of tiles).
struct Split {
  int64_t chunk, n_split;
};
Split split_of(int64_t BH, int64_t Nk) {
  int64_t want = (kTargetWaves + BH - 1) / BH;
  const int64_t tiles = (Nk + kKT - 1) / kKT;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t tiles_per = (tiles + want - 1) / want;
  const int64_t chunk = tiles_per * kKT;
  return {chunk, (Nk + chunk - 1) / chunk};
}

template <typename Tag, int D>
__global__ __launch_bounds__(kDW * 64) void attn_decode_split_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    float* __restrict__ ws_o, float* __restrict__ ws_l, int Nq, int Nk, int n_split, int total_waves,
    float c /* scale*log2 e */) {
  constexpr int NSTEP = D / 16, NDB = D / 32, TB = kKT * D * 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kDW * 4 * TB];   // per wave: K slots 0, 1; V slots 0, 1

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64;
  const int half = lane / 32, l32 = lane % 32;
  const int gw = blockIdx.x * kDW + wave;           // (batch*head, split), splits of one head adjacent
  if (gw >= total_waves) return;                    // no barriers below: waves are independent
  const int bh = gw / n_split, sp = gw % n_split;
  const int n_tiles = (Nk + kKT - 1) / kKT;
  const int T = (n_tiles - sp + n_split - 1) / n_split;   // tiles sp, sp + n_split, ...
  const int key_end = Nk;
  auto tile_key = [&](int t) __attribute__((always_inline)) { return (sp + t * n_split) * kKT; };
  const uint16_t* Kh = K + (int64_t)bh * Nk * D;
  const uint16_t* Vh = V + (int64_t)bh * Nk * D;

  u32x4 qreg[NSTEP];
  load_row_operand<D>(Q + (int64_t)bh * Nq * D, l32, Nq, half, qreg);
  TileAddr<D> ta;
  ta.init(lane);
  uint8_t* const mine = lds + wave * 4 * TB;
  auto kbuf = [&](int slot) __attribute__((always_inline)) { return mine + slot * TB; };
  auto vbuf = [&](int slot) __attribute__((always_inline)) { return mine + (2 + slot) * TB; };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float M = -INFINITY, l_part = 0.f;                // running max (log2 units), partial row sum

  load_rows<D, kKT, 1>(Kh, tile_key(0), key_end, kbuf(0), 0, lane);
  load_rows<D, kKT, 1>(Vh, tile_key(0), key_end, vbuf(0), 0, lane);
  for (int t = 0; t < T; ++t) {
    const int slot = t & 1;
    if (t + 1 < T) {
      load_rows<D, kKT, 1>(Kh, tile_key(t + 1), key_end, kbuf(slot ^ 1), 0, lane);
      load_rows<D, kKT, 1>(Vh, tile_key(t + 1), key_end, vbuf(slot ^ 1), 0, lane);
      wait_vmcnt<2 * (TB / 1024)>();                // tile t has landed; tile t+1 may still be in flight
    } else {
      wait_vmcnt<0>();
    }
    const uint8_t* kt = kbuf(slot);
    const uint8_t* vt = vbuf(slot);
    f32x16 s = f32x16{};
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) s = mfma32(Tag{}, row_frag<D>(kt, ta, 0, st), qreg[st], s);
    const int key0 = tile_key(t);
    if (key0 + kKT > key_end) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + (r / 4) * 8 + half * 4 + (r % 4) >= key_end) s[r] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, s[r]);
    const float m_new = __builtin_elementwise_maximum(M, max_halves(mx) * c);   // finite: a tile holds a key
    if (__builtin_amdgcn_ballot_w64(m_new > M) != 0) {
      const float alpha = fast_exp2(M - m_new);     // 0 on the first tile (M = -inf)
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      l_part *= alpha;
      M = m_new;
    }
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = fast_exp2(__builtin_fmaf(s[r], c, -M));
      l_part += p[r];
    }
    u32x4 pb[2];
    pack16<Tag>(p, pb);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(Tag{}, tr_frag<D>(vt, ta, h * 16, db), pb[h], oacc[db]);
    // (the next iteration's loads overwrite slot ^ 1 only: this wave's reads of slot are
    // complete before its own later instructions reuse it two tiles on)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  const float l_tot = add_halves(l_part);
  if (l32 >= Nq) return;
  const int64_t row = (int64_t)gw * Nq + l32;       // [bh][split][q]
  const float inv = 1.f / l_tot;
  float* dst = ws_o + row * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + g * 8 + half * 4;
      const f32x16 a = oacc[db];
      *(f32x4*)(dst + d) = f32x4{a[g * 4] * inv, a[g * 4 + 1] * inv, a[g * 4 + 2] * inv, a[g * 4 + 3] * inv};
    }
  if (half == 0) ws_l[row] = (M + __builtin_log2f(l_tot)) * kLn2;
}

template <typename Tag, int D>
__global__ __launch_bounds__(kCombineThreads) void attn_decode_combine_kernel(const float* __restrict__ ws_o,
                                                                              const float* __restrict__ ws_l,
                                                                              uint16_t* __restrict__ O,
                                                                              float* __restrict__ LSE, int Nq,
                                                                              int n_split) {
  // kGroups groups of D/4 threads; group g sums the splits sp = g, g + kGroups, ... for
  // 4 head dims per thread, then the groups' sums are added through LDS.
  constexpr int TPG = D / 4, kGroups = kCombineThreads / TPG;
  __shared__ float red_m[kCombineThreads / 64];
  __shared__ __attribute__((aligned(16))) f32x4 part_o[kGroups][TPG];
  __shared__ float part_w[kGroups];
  const int row = blockIdx.x;                       // bh * Nq + q
  const int bh = row / Nq, q = row % Nq;
  const int tid = threadIdx.x, g = tid / TPG, t = tid % TPG;
  auto part = [&](int sp) -> int64_t { return ((int64_t)bh * n_split + sp) * Nq + q; };
  float m = -INFINITY;
  for (int sp = tid; sp < n_split; sp += kCombineThreads) m = fmaxf(m, ws_l[part(sp)]);
#pragma unroll
  for (int off = 32; off >= 1; off /= 2) m = fmaxf(m, __shfl_xor(m, off));
  if (tid % 64 == 0) red_m[tid / 64] = m;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kCombineThreads / 64; ++i) m = fmaxf(m, red_m[i]);
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sp = g; sp < n_split; sp += kGroups) {
    const float w = __expf(ws_l[part(sp)] - m);
    wsum += w;
    const f32x4 x = *(const f32x4*)(ws_o + part(sp) * D + t * 4);
    acc = f32x4{__builtin_fmaf(w, x[0], acc[0]), __builtin_fmaf(w, x[1], acc[1]), __builtin_fmaf(w, x[2], acc[2]),
                __builtin_fmaf(w, x[3], acc[3])};
  }
  part_o[g][t] = acc;
  if (t == 0) part_w[g] = wsum;
  __syncthreads();
  if (g != 0) return;
  float wt = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kGroups; ++i) {
    wt += part_w[i];
    o += part_o[i][t];
  }
  const float inv = 1.f / wt;
  *(u32x2*)(O + (int64_t)row * D + t * 4) = u32x2{pack2(Tag{}, o[0] * inv, o[1] * inv), pack2(Tag{}, o[2] * inv, o[3] * inv)};
  if (t == 0) LSE[row] = m + __logf(wt);
}

template <typename Tag, int D>
hipError_t launch_one(const void* q, const void* k, const void* v, void* o, float* lse, float* ws, int64_t BH,
                      int64_t Nq, int64_t Nk, float scale, hipStream_t stream) {
  const Split sp = split_of(BH, Nk);
  const int64_t waves = BH * sp.n_split;
  float* ws_o = ws;
  float* ws_l = ws + waves * Nq * D;
  hipLaunchKernelGGL((attn_decode_split_kernel<Tag, D>), dim3((unsigned)((waves + kDW - 1) / kDW)), dim3(kDW * 64), 0,
                     stream, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, ws_o, ws_l, (int)Nq, (int)Nk,
                     (int)sp.n_split, (int)waves, scale * kLog2e);
  hipLaunchKernelGGL((attn_decode_combine_kernel<Tag, D>), dim3((unsigned)(BH * Nq)), dim3(kCombineThreads), 0, stream,
                     ws_o, ws_l, (uint16_t*)o, lse, (int)Nq, (int)sp.n_split);
  return hipGetLastError();
}

template <typename Tag>
hipError_t launch_16bit(const void* q, const void* k, const void* v, void* o, float* lse, float* ws, int64_t BH,
                        int64_t Nq, int64_t Nk, int64_t d, float scale, hipStream_t stream) {
  return d == 128 ? launch_one<Tag, 128>(q, k, v, o, lse, ws, BH, Nq, Nk, scale, stream)
                  : launch_one<Tag, 64>(q, k, v, o, lse, ws, BH, Nq, Nk, scale, stream);
}

}  // namespace

int64_t decode_workspace_floats(int64_t BH, int64_t Nq, int64_t Nk, int64_t d) {
  const Split sp = split_of(BH, Nk);
  return BH * sp.n_split * Nq * (d + 1);
}

int64_t max_workgroups_decode(int64_t BH, int64_t Nq, int64_t Nk) {
  const Split sp = split_of(BH, Nk);
  const int64_t a = (BH * sp.n_split + kDW - 1) / kDW, b = BH * Nq;
  return a > b ? a : b;
}

hipError_t launch_decode_bf16(const void* q, const void* k, const void* v, void* o, float* lse, float* ws,
                              int64_t BH, int64_t Nq, int64_t Nk, int64_t d, float scale, hipStream_t stream) {
  return launch_16bit<Bf16Tag>(q, k, v, o, lse, ws, BH, Nq, Nk, d, scale, stream);
}

// Scratch of the allocation-free decoding entry point: the per-split partials (O and LSE
// of every (head, key split, query row)) live in this file-scope device array instead of
// a caller workspace. Each GPU the library runs on holds its own copy, at its own address,
// until the process ends. Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address of each GPU's copy is
// looked up once per device with hipGetSymbolAddress and kept in scratch_ptr.
static __device__ __align__(256) float scratch[kDecodeScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
float* scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(float** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // the current device's copy
    if (e != hipSuccess) return e;
    scratch_ptr[dev] = (float*)p;
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_bf16_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH,
                                      int64_t Nq, int64_t Nk, int64_t d, float scale, hipStream_t stream) {
  float* ws = nullptr;
  const hipError_t e = decode_scratch(&ws);
  if (e != hipSuccess) return e;
  // every partial the combine kernel reads is written by the split kernel first: nothing
  // in the scratch needs clearing between calls
  return launch_16bit<Bf16Tag>(q, k, v, o, lse, ws, BH, Nq, Nk, d, scale, stream);
}

hipError_t launch_decode_f16(const void* q, const void* k, const void* v, void* o, float* lse, float* ws,
                             int64_t BH, int64_t Nq, int64_t Nk, int64_t d, float scale, hipStream_t stream) {
  return launch_16bit<F16Tag>(q, k, v, o, lse, ws, BH, Nq, Nk, d, scale, stream);
}

}  // namespace attn
