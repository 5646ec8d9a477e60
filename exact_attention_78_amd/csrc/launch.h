// Internal launchers behind the C ABI. Arguments are already validated by the caller
// (attn_api.cpp); each returns the hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Launch variants of the 16-bit forward pass: tile order or persistent grid (sched), and
// which passes run. The values match attn_sched_t and attn_passes_t of attn.h.
enum : int { kSchedAuto = -1, kSchedPersistentStride = 6, kSchedPersistentQueue = 7, kSchedPersistentSnake = 8 };
enum : int { kPassesAuto = 0, kPassesExact = 1, kPassesTwo = 2 };
struct FwdVariant {
  int sched = kSchedAuto;    // 0..5: TileOrder of a plain grid; 6..8: persistent grids; auto (the
                             // plain entry points): the plain grid in the default order
  int passes = kPassesAuto;
  int* queue = nullptr;      // kSchedPersistentQueue: 16 ints of caller memory, zero between calls
};

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                           int64_t d, bool causal, float scale, hipStream_t stream, const FwdVariant& var = {});
hipError_t launch_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                          int64_t d, bool causal, float scale, hipStream_t stream, const FwdVariant& var = {});
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int64_t BH, int64_t N,
                          int64_t d, bool causal, float scale, hipStream_t stream);
hipError_t launch_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* sq, const float* sk,
                          const float* sv, void* o, float* lse, int64_t BH, int64_t N, int64_t d, bool causal,
                          float scale, hipStream_t stream);
hipError_t launch_quant_fp8(const void* x, uint8_t* x8, float* scales, const float* signs, int64_t BH, int64_t N,
                            int64_t d, hipStream_t stream);
// Q (rotated; skipped when q is null), K (rotated) and V (unrotated) in one launch.
hipError_t launch_quant_fp8_qkv(const void* q, const void* k, const void* v, uint8_t* q8, uint8_t* k8, uint8_t* v8,
                                float* q_scales, float* k_scales, float* v_scales, const float* signs, int64_t BH,
                                int64_t N, int64_t d, hipStream_t stream);
hipError_t launch_fwd_fp8_rotq(const void* q, const float* signs, const uint8_t* k8, const uint8_t* v8,
                               const float* sk, const float* sv, void* o, float* lse, uint8_t* q8_out, float* sq_out,
                               int64_t BH, int64_t N, int64_t d, bool causal, float scale, hipStream_t stream);

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, float* ws, int64_t BH, int64_t N, int64_t d,
                           bool causal, float scale, hipStream_t stream);
hipError_t launch_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, float* ws, int64_t BH, int64_t N, int64_t d,
                          bool causal, float scale, hipStream_t stream);

hipError_t launch_decode_bf16(const void* q, const void* k, const void* v, void* o, float* lse, float* ws,
                              int64_t BH, int64_t Nq, int64_t Nk, int64_t d, float scale, hipStream_t stream);
hipError_t launch_decode_f16(const void* q, const void* k, const void* v, void* o, float* lse, float* ws,
                             int64_t BH, int64_t Nq, int64_t Nk, int64_t d, float scale, hipStream_t stream);
// Floats of workspace the decode launches use.
int64_t decode_workspace_floats(int64_t BH, int64_t Nq, int64_t Nk, int64_t d);
// The bf16 decoding step with its partials in the library's static device scratch of
// kDecodeScratchFloats floats per GPU (sizes already checked against it by the caller);
// the first call on a device looks up that device's copy (hipGetSymbolAddress).
constexpr int64_t kDecodeScratchFloats = int64_t(16) << 20;   // 64 MiB
hipError_t launch_decode_bf16_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH,
                                      int64_t Nq, int64_t Nk, int64_t d, float scale, hipStream_t stream);

// Calibration loops (kind 0: dense bf16 MFMA, kind 1: v_exp_f32) and the operations one
// workgroup of them performs.
hipError_t launch_calib(int kind, const uint32_t* seed, float* out, int64_t workgroups, int iters, hipStream_t stream);
int64_t calib_ops_per_workgroup(int kind, int iters);

// Workgroup counts of the launches above (validated against the 32-bit grid limit).
int64_t max_workgroups_fwd16(int64_t BH, int64_t N);
int64_t max_workgroups_fwd32(int64_t BH, int64_t N);
int64_t max_workgroups_fwd8(int64_t BH, int64_t N);
int64_t max_workgroups_quant(int64_t BH, int64_t N);
int64_t max_workgroups_bwd(int64_t BH, int64_t N);
int64_t max_workgroups_decode(int64_t BH, int64_t Nq, int64_t Nk);

}  // namespace attn
