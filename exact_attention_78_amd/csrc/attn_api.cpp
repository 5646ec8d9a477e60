// C ABI of the attention library: host-side validation, then dispatch to the launchers.
// Validation never calls into HIP, so a rejected call touches no device state.
#include "attn.h"

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "launch.h"

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by all entry points; writes the element count of one [B,H,N,d] tensor.
attn_status_t check_shape(int64_t B, int64_t H, int64_t N, int64_t d, int64_t* elems, int64_t* rows) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
  int64_t bh, bhn, e;
  if (__builtin_mul_overflow(B, H, &bh) || __builtin_mul_overflow(bh, N, &bhn) ||
      __builtin_mul_overflow(bhn, d, &e) || e > INT64_MAX / 8)
    return ATTN_ERR_INVALID_ARG;
  if (N > INT32_MAX) return ATTN_ERR_INVALID_ARG;   // kernels index rows with 32-bit ints
  *elems = e;
  *rows = bhn;
  return ATTN_OK;
}

bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

attn_status_t from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

// Validation of the 16/32-bit forward entry points (element size esz bytes).
attn_status_t check_fwd(const void* q, const void* k, const void* v, const void* o, const void* lse, int64_t B,
                        int64_t H, int64_t N, int64_t d, float scale, size_t esz,
                        int64_t (*workgroups)(int64_t, int64_t)) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID_ARG;
  int64_t elems, rows;
  attn_status_t st = check_shape(B, H, N, d, &elems, &rows);
  if (st != ATTN_OK) return st;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (workgroups(B * H, N) > INT32_MAX) return ATTN_ERR_INVALID_ARG;   // shape checked: no overflow
  const uintptr_t tb = (uintptr_t)elems * esz;
  const Range rq{(uintptr_t)q, (uintptr_t)q + tb}, rk{(uintptr_t)k, (uintptr_t)k + tb},
      rv{(uintptr_t)v, (uintptr_t)v + tb}, ro{(uintptr_t)o, (uintptr_t)o + tb},
      rl{(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)rows * sizeof(float)};
  if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv) || overlaps(ro, rl)) return ATTN_ERR_INVALID_ARG;
  if (overlaps(rl, rq) || overlaps(rl, rk) || overlaps(rl, rv)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// Validation of the 16-bit backward entry points.
attn_status_t check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, const void* dq, const void* dk, const void* dv, const float* ws,
                        int64_t B, int64_t H, int64_t N, int64_t d, float scale) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !ws) return ATTN_ERR_INVALID_ARG;
  int64_t elems, rows;
  attn_status_t st = check_shape(B, H, N, d, &elems, &rows);
  if (st != ATTN_OK) return st;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  const void* ptrs[10] = {q, k, v, o, lse, dout, dq, dk, dv, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (attn::max_workgroups_bwd(B * H, N) > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  const uintptr_t tb = (uintptr_t)elems * 2;
  auto span = [](const void* p, uintptr_t n) { return Range{(uintptr_t)p, (uintptr_t)p + n}; };
  const Range ins[6] = {span(q, tb), span(k, tb), span(v, tb), span(o, tb),
                        span(lse, (uintptr_t)rows * sizeof(float)), span(dout, tb)};
  const Range outs[4] = {span(dq, tb), span(dk, tb), span(dv, tb), span(ws, (uintptr_t)rows * 2 * sizeof(float))};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return ATTN_ERR_INVALID_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], outs[j])) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

// Shapes of the decode entry points: q [B,H,Nq,d], k/v [B,H,Nk,d]; writes element counts.
attn_status_t check_decode_shape(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t* q_elems,
                                 int64_t* kv_elems, int64_t* rows) {
  if (Nq < 1 || Nq > 32) return ATTN_ERR_INVALID_ARG;
  attn_status_t st = check_shape(B, H, Nk, d, kv_elems, rows);
  if (st != ATTN_OK) return st;
  if (__builtin_mul_overflow(B * H, Nq, rows) || __builtin_mul_overflow(*rows, d, q_elems) || *q_elems > INT64_MAX / 8)
    return ATTN_ERR_INVALID_ARG;                   // (B * H cannot overflow: check_shape bounded B * H * Nk * d)
  return ATTN_OK;
}

// Validation of the decode entry points; ws == NULL with no_ws: the static-scratch variant.
attn_status_t check_decode(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const float* ws, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                           bool no_ws = false) {
  if (!q || !k || !v || !o || !lse || (!ws && !no_ws)) return ATTN_ERR_INVALID_ARG;
  int64_t qe, kve, rows;
  attn_status_t st = check_decode_shape(B, H, Nq, Nk, d, &qe, &kve, &rows);
  if (st != ATTN_OK) return st;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  const void* ptrs[6] = {q, k, v, o, lse, no_ws ? q : ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (attn::max_workgroups_decode(B * H, Nq, Nk) > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  auto span = [](const void* p, uintptr_t n) { return Range{(uintptr_t)p, (uintptr_t)p + n}; };
  const int64_t wsf = no_ws ? 0 : attn::decode_workspace_floats(B * H, Nq, Nk, d);
  const Range ins[3] = {span(q, (uintptr_t)qe * 2), span(k, (uintptr_t)kve * 2), span(v, (uintptr_t)kve * 2)};
  const Range outs[3] = {span(o, (uintptr_t)qe * 2), span(lse, (uintptr_t)rows * sizeof(float)),
                         span(ws, (uintptr_t)wsf * sizeof(float))};
  for (int i = 0; i < 3; ++i) {
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return ATTN_ERR_INVALID_ARG;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outs[j])) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

// Shared by the one-launch quantisers: nt = 2 (K, V) or 3 (Q, K, V) bf16 inputs x[i] of one
// shape, the signs, and their codes x8[i] and scales sc[i]; every pointer non-null and
// 16-byte aligned, no output overlapping an input or another output.
attn_status_t quant_multi(int nt, const void* const* x, const float* signs, uint8_t* const* x8, float* const* sc,
                          int64_t B, int64_t H, int64_t N, int64_t d, void* stream) {
  if (!signs || !aligned16(signs)) return ATTN_ERR_INVALID_ARG;
  for (int i = 0; i < nt; ++i)
    if (!x[i] || !x8[i] || !sc[i] || !aligned16(x[i]) || !aligned16(x8[i]) || !aligned16(sc[i]))
      return ATTN_ERR_INVALID_ARG;
  int64_t elems, rows;
  attn_status_t st = check_shape(B, H, N, d, &elems, &rows);
  if (st != ATTN_OK) return st;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (nt * attn::max_workgroups_quant(B * H, N) > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  const int64_t nblk = (N + 127) / 128;
  const uintptr_t sb = (uintptr_t)(B * H * nblk) * sizeof(float);
  auto span = [](const void* p, uintptr_t n) { return Range{(uintptr_t)p, (uintptr_t)p + n}; };
  Range ins[4], outs[6];
  int ni = 0, no = 0;
  ins[ni++] = span(signs, (uintptr_t)d * sizeof(float));
  for (int i = 0; i < nt; ++i) {
    ins[ni++] = span(x[i], (uintptr_t)elems * 2);
    outs[no++] = span(x8[i], (uintptr_t)elems);
    outs[no++] = span(sc[i], sb);
  }
  for (int i = 0; i < no; ++i) {
    for (int j = 0; j < ni; ++j)
      if (overlaps(outs[i], ins[j])) return ATTN_ERR_INVALID_ARG;
    for (int j = i + 1; j < no; ++j)
      if (overlaps(outs[i], outs[j])) return ATTN_ERR_INVALID_ARG;
  }
  const int o = nt == 3 ? 1 : 0;                    // index of K
  return from_hip(attn::launch_quant_fp8_qkv(nt == 3 ? x[0] : nullptr, x[o], x[o + 1], nt == 3 ? x8[0] : nullptr,
                                             x8[o], x8[o + 1], nt == 3 ? sc[0] : nullptr, sc[o], sc[o + 1], signs,
                                             B * H, N, d, (hipStream_t)stream));
}
}  // namespace

extern "C" {

attn_status_t attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                            int64_t N, int64_t d, int causal, float scale, void* stream) {
  attn_status_t st = check_fwd(q, k, v, o, lse, B, H, N, d, scale, 2, attn::max_workgroups_fwd16);
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_fwd_bf16(q, k, v, o, lse, B * H, N, d, causal != 0, scale, (hipStream_t)stream));
}

attn_status_t attn_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                           int64_t N, int64_t d, int causal, float scale, void* stream) {
  attn_status_t st = check_fwd(q, k, v, o, lse, B, H, N, d, scale, 2, attn::max_workgroups_fwd16);
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_fwd_f16(q, k, v, o, lse, B * H, N, d, causal != 0, scale, (hipStream_t)stream));
}

attn_status_t attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                               int64_t H, int64_t N, int64_t d, int causal, float scale, int dtype, int sched,
                               int passes, int32_t* queue, void* stream) {
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16) return ATTN_ERR_INVALID_ARG;
  if (sched < ATTN_SCHED_DEFAULT || sched > ATTN_SCHED_PERSISTENT_SNAKE) return ATTN_ERR_INVALID_ARG;
  if (passes < ATTN_PASSES_AUTO || passes > ATTN_PASSES_TWO) return ATTN_ERR_INVALID_ARG;
  attn_status_t st = check_fwd(q, k, v, o, lse, B, H, N, d, scale, 2, attn::max_workgroups_fwd16);
  if (st != ATTN_OK) return st;
  attn::FwdVariant var;
  var.sched = sched;
  var.passes = passes;
  if (sched == ATTN_SCHED_PERSISTENT_QUEUE) {
    if (!queue || !aligned16(queue)) return ATTN_ERR_INVALID_ARG;
    const uintptr_t tb = (uintptr_t)(B * H * N * d) * 2;   // checked by check_fwd: no overflow
    const Range rq{(uintptr_t)queue, (uintptr_t)queue + 16 * sizeof(int32_t)};
    const Range others[5] = {{(uintptr_t)q, (uintptr_t)q + tb}, {(uintptr_t)k, (uintptr_t)k + tb},
                             {(uintptr_t)v, (uintptr_t)v + tb}, {(uintptr_t)o, (uintptr_t)o + tb},
                             {(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)(B * H * N) * sizeof(float)}};
    for (const Range& r : others)
      if (overlaps(rq, r)) return ATTN_ERR_INVALID_ARG;
    var.queue = queue;
  }
  const hipStream_t s = (hipStream_t)stream;
  return from_hip(dtype == ATTN_DTYPE_BF16
                      ? attn::launch_fwd_bf16(q, k, v, o, lse, B * H, N, d, causal != 0, scale, s, var)
                      : attn::launch_fwd_f16(q, k, v, o, lse, B * H, N, d, causal != 0, scale, s, var));
}

attn_status_t attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int64_t B, int64_t H,
                           int64_t N, int64_t d, int causal, float scale, void* stream) {
  attn_status_t st = check_fwd(q, k, v, o, lse, B, H, N, d, scale, 4, attn::max_workgroups_fwd32);
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_fwd_f32(q, k, v, o, lse, B * H, N, d, causal != 0, scale, (hipStream_t)stream));
}

attn_status_t attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                           const float* k_scale, const float* v_scale, void* o, float* lse, int64_t B, int64_t H,
                           int64_t N, int64_t d, int causal, float scale, void* stream) {
  if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !o || !lse) return ATTN_ERR_INVALID_ARG;
  int64_t elems, rows;
  attn_status_t st = check_shape(B, H, N, d, &elems, &rows);
  if (st != ATTN_OK) return st;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  const void* ptrs[8] = {q8, k8, v8, q_scale, k_scale, v_scale, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (attn::max_workgroups_fwd8(B * H, N) > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  const int64_t nblk = (N + 127) / 128;
  const uintptr_t sb = (uintptr_t)(B * H * nblk) * sizeof(float);
  const Range ro{(uintptr_t)o, (uintptr_t)o + (uintptr_t)elems * 2},
      rl{(uintptr_t)lse, (uintptr_t)lse + (uintptr_t)rows * sizeof(float)};
  const Range ins[6] = {{(uintptr_t)q8, (uintptr_t)q8 + (uintptr_t)elems},
                        {(uintptr_t)k8, (uintptr_t)k8 + (uintptr_t)elems},
                        {(uintptr_t)v8, (uintptr_t)v8 + (uintptr_t)elems},
                        {(uintptr_t)q_scale, (uintptr_t)q_scale + sb},
                        {(uintptr_t)k_scale, (uintptr_t)k_scale + sb},
                        {(uintptr_t)v_scale, (uintptr_t)v_scale + sb}};
  if (overlaps(ro, rl)) return ATTN_ERR_INVALID_ARG;
  for (const Range& r : ins)
    if (overlaps(ro, r) || overlaps(rl, r)) return ATTN_ERR_INVALID_ARG;
  return from_hip(attn::launch_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B * H, N, d, causal != 0, scale,
                                       (hipStream_t)stream));
}

attn_status_t attn_quant_fp8(const void* x, uint8_t* x8, float* scales, const float* signs, int64_t B, int64_t H,
                             int64_t N, int64_t d, void* stream) {
  if (!x || !x8 || !scales) return ATTN_ERR_INVALID_ARG;
  int64_t elems, rows;
  attn_status_t st = check_shape(B, H, N, d, &elems, &rows);
  if (st != ATTN_OK) return st;
  if (!aligned16(x) || !aligned16(x8) || !aligned16(scales) || (signs && !aligned16(signs)))
    return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (attn::max_workgroups_quant(B * H, N) > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  const int64_t nblk = (N + 127) / 128;
  const Range rx{(uintptr_t)x, (uintptr_t)x + (uintptr_t)elems * 2}, r8{(uintptr_t)x8, (uintptr_t)x8 + (uintptr_t)elems},
      rs{(uintptr_t)scales, (uintptr_t)scales + (uintptr_t)(B * H * nblk) * sizeof(float)},
      rg{(uintptr_t)signs, (uintptr_t)signs + (signs ? (uintptr_t)d * sizeof(float) : 0)};
  if (overlaps(r8, rx) || overlaps(r8, rs) || overlaps(rs, rx)) return ATTN_ERR_INVALID_ARG;
  if (signs && (overlaps(rg, r8) || overlaps(rg, rs))) return ATTN_ERR_INVALID_ARG;
  return from_hip(attn::launch_quant_fp8(x, x8, scales, signs, B * H, N, d, (hipStream_t)stream));
}

attn_status_t attn_quant_fp8_kv(const void* k, const void* v, const float* signs, uint8_t* k8, uint8_t* v8,
                                float* k_scale, float* v_scale, int64_t B, int64_t H, int64_t N, int64_t d,
                                void* stream) {
  const void* x[2] = {k, v};
  uint8_t* x8[2] = {k8, v8};
  float* sc[2] = {k_scale, v_scale};
  return quant_multi(2, x, signs, x8, sc, B, H, N, d, stream);
}

attn_status_t attn_quant_fp8_qkv(const void* q, const void* k, const void* v, const float* signs, uint8_t* q8,
                                 uint8_t* k8, uint8_t* v8, float* q_scale, float* k_scale, float* v_scale, int64_t B,
                                 int64_t H, int64_t N, int64_t d, void* stream) {
  const void* x[3] = {q, k, v};
  uint8_t* x8[3] = {q8, k8, v8};
  float* sc[3] = {q_scale, k_scale, v_scale};
  return quant_multi(3, x, signs, x8, sc, B, H, N, d, stream);
}

attn_status_t attn_fwd_fp8_rotq(const void* q, const float* signs, const uint8_t* k8, const uint8_t* v8,
                                const float* k_scale, const float* v_scale, void* o, float* lse, uint8_t* q8_out,
                                float* q_scale_out, int64_t B, int64_t H, int64_t N, int64_t d, int causal,
                                float scale, void* stream) {
  if (!q || !signs || !k8 || !v8 || !k_scale || !v_scale || !o || !lse) return ATTN_ERR_INVALID_ARG;
  int64_t elems, rows;
  attn_status_t st = check_shape(B, H, N, d, &elems, &rows);
  if (st != ATTN_OK) return st;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID_ARG;
  const void* ptrs[10] = {q, signs, k8, v8, k_scale, v_scale, o, lse, q8_out ? q8_out : q,
                          q_scale_out ? (const void*)q_scale_out : q};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (attn::max_workgroups_fwd8(B * H, N) > INT32_MAX) return ATTN_ERR_INVALID_ARG;
  const int64_t nblk = (N + 127) / 128;
  const uintptr_t sb = (uintptr_t)(B * H * nblk) * sizeof(float);
  auto span = [](const void* p, uintptr_t n) { return Range{(uintptr_t)p, (uintptr_t)p + n}; };
  const Range ins[6] = {span(q, (uintptr_t)elems * 2), span(signs, (uintptr_t)d * sizeof(float)),
                        span(k8, (uintptr_t)elems), span(v8, (uintptr_t)elems), span(k_scale, sb),
                        span(v_scale, sb)};
  const Range outs[4] = {span(o, (uintptr_t)elems * 2), span(lse, (uintptr_t)rows * sizeof(float)),
                         span(q8_out, q8_out ? (uintptr_t)elems : 0), span(q_scale_out, q_scale_out ? sb : 0)};
  for (int i = 0; i < 4; ++i) {
    if (outs[i].lo == outs[i].hi) continue;
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return ATTN_ERR_INVALID_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (outs[j].lo != outs[j].hi && overlaps(outs[i], outs[j])) return ATTN_ERR_INVALID_ARG;
  }
  return from_hip(attn::launch_fwd_fp8_rotq(q, signs, k8, v8, k_scale, v_scale, o, lse, q8_out, q_scale_out, B * H, N,
                                            d, causal != 0, scale, (hipStream_t)stream));
}

attn_status_t attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                            const void* dout, void* dq, void* dk, void* dv, float* workspace, int64_t B, int64_t H,
                            int64_t N, int64_t d, int causal, float scale, void* stream) {
  attn_status_t st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, workspace, B * H, N, d, causal != 0, scale,
                                        (hipStream_t)stream));
}

attn_status_t attn_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, float* workspace, int64_t B, int64_t H,
                           int64_t N, int64_t d, int causal, float scale, void* stream) {
  attn_status_t st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_bwd_f16(q, k, v, o, lse, dout, dq, dk, dv, workspace, B * H, N, d, causal != 0, scale,
                                       (hipStream_t)stream));
}

int64_t attn_decode_workspace_floats(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
  int64_t qe, kve, rows;
  if (check_decode_shape(B, H, Nq, Nk, d, &qe, &kve, &rows) != ATTN_OK) return -1;
  return attn::decode_workspace_floats(B * H, Nq, Nk, d);
}

attn_status_t attn_decode_bf16(const void* q, const void* k, const void* v, void* o, float* lse, float* workspace,
                               int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, void* stream) {
  attn_status_t st = check_decode(q, k, v, o, lse, workspace, B, H, Nq, Nk, d, scale);
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_decode_bf16(q, k, v, o, lse, workspace, B * H, Nq, Nk, d, scale, (hipStream_t)stream));
}

attn_status_t attn_decode_bf16_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                       int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, void* stream) {
  attn_status_t st = check_decode(q, k, v, o, lse, nullptr, B, H, Nq, Nk, d, scale, true);
  if (st != ATTN_OK) return st;
  if (attn::decode_workspace_floats(B * H, Nq, Nk, d) > attn::kDecodeScratchFloats) return ATTN_ERR_SCRATCH_TOO_SMALL;
  return from_hip(
      attn::launch_decode_bf16_noalloc(q, k, v, o, lse, B * H, Nq, Nk, d, scale, (hipStream_t)stream));
}

attn_status_t attn_decode_f16(const void* q, const void* k, const void* v, void* o, float* lse, float* workspace,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, void* stream) {
  attn_status_t st = check_decode(q, k, v, o, lse, workspace, B, H, Nq, Nk, d, scale);
  if (st != ATTN_OK) return st;
  return from_hip(attn::launch_decode_f16(q, k, v, o, lse, workspace, B * H, Nq, Nk, d, scale, (hipStream_t)stream));
}

attn_status_t attn_calibrate(int kind, const uint32_t* seed, float* out, int64_t workgroups, int iters,
                             void* stream) {
  if (kind < 0 || kind > 8 || !seed || !out || workgroups < 1 || workgroups > INT32_MAX || iters < 1)
    return ATTN_ERR_INVALID_ARG;
  // kind 6 reads workgroups * 256 * iters 16-byte elements from seed: the count must fit
  // the kernel's int64 indexing
  if (kind == 6 && workgroups * 256 > INT64_MAX / 16 / iters) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(seed) || !aligned16(out)) return ATTN_ERR_INVALID_ARG;
  return from_hip(attn::launch_calib(kind, seed, out, workgroups, iters, (hipStream_t)stream));
}

int64_t attn_calibrate_ops(int kind, int iters) {
  if (kind < 0 || kind > 8 || iters < 1) return -1;
  return attn::calib_ops_per_workgroup(kind, iters);
}

const char* attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_SCRATCH_TOO_SMALL: return "sizes need more than the library's static scratch (64 MiB per GPU)";
  }
  return "unknown status";
}

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

}  // extern "C"
