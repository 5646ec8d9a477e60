/*
 * attn.h — C ABI of the exact attention library (forward, backward, fp8 input preparation)
 * for AMD Instinct MI355X (gfx950).
 *
 * Operation (all entry points). For every batch b and head h independently, with
 * Q, K, V the [N, d] slices of that head:
 *
 *     O   = softmax(scale * Q K^T [+ causal mask]) V          (row-wise softmax)
 *     LSE = log(sum_j exp(scale * q_i . k_j))  over the keys row i may see
 *
 * This is exact attention as defined in "FlashAttention-2: faster attention with better
 * parallelism and work partitioning" (digest, irregular6612.github.io): its framework-
 * overview flowchart streams K/V tiles through an online softmax, rescales once at the
 * end and writes O plus one log-sum-exp per row; its glossary defines the log-sum-exp
 * as the log of the sum of exponentials (natural log here). The causal mask lets query
 * row i see keys j <= i; key tiles entirely above the diagonal are never loaded (the
 * digest's key-components list: mask only boundary blocks, skip the strictly upper ones).
 * Inputs are low precision and every contraction accumulates in fp32 ("Triton 07: Flash
 * Attention v3", Method, item 3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Layout: Q, K, V and O are contiguous row-major [B, H, N, d] (row stride d elements;
 *    decode: Nq query rows against Nk keys); LSE is contiguous fp32 [B, H, N]. Per-block
 *    fp8 scales are fp32 [B, H, ceil(N/128)].
 *  - Ownership: every pointer is caller-owned device memory on the current HIP device.
 *    The library allocates nothing, frees nothing and keeps no state between calls; calls
 *    are reentrant. Tensor pointers must be 16-byte aligned.
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without synchronising. A device fault surfaces at the caller's
 *    next synchronisation on that stream.
 *  - Validation happens on the host, before any HIP call, and on failure nothing is
 *    enqueued:
 *      ATTN_ERR_INVALID_ARG  a NULL pointer, B/H/N < 1, a scale that is not finite and
 *                            > 0, a pointer not 16-byte aligned, an element count that
 *                            overflows int64, or an output range overlapping an input
 *                            or another output;
 *      ATTN_ERR_UNSUPPORTED  d not in {64, 128};
 *      ATTN_ERR_LAUNCH       the kernel launch itself failed (hipGetLastError).
 *  - Numbers: inputs with NaN or Inf give undefined outputs (not checked on the device).
 *    Any N >= 1 is accepted; partial tiles are masked.
 *  - Scale: pass the softmax scale as the fp32 value the caller wants (1/sqrt(d) is
 *    usual); it is used as given.
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,
  ATTN_ERR_UNSUPPORTED = 2,
  ATTN_ERR_LAUNCH = 3,
  ATTN_ERR_SCRATCH_TOO_SMALL = 4
} attn_status_t;

#define ATTN_ABI_VERSION 3

/* bf16 Q/K/V in, bf16 O out (round to nearest even), fp32 LSE out. P is rounded to
 * bf16 before the P.V contraction; both contractions accumulate in fp32. The call
 * enqueues one kernel on `stream`: a pass that uses the first key tile's row max as the
 * softmax reference, whose workgroups redo with a per-tile max any query tile whose
 * probabilities outgrew it. O and LSE are complete when the kernel has run. */
attn_status_t attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                            void* stream);

/* Launch variants of the 16-bit forward pass, for measuring its design choices against
 * each other; every variant computes the same O and LSE as attn_fwd_bf16 / attn_fwd_f16.
 *
 * sched: how query tiles map to workgroups. The 1D grid over (batch*head, query tile)
 * with neighbouring ids on one head is item 4 of the Method section of "Triton 07: Flash
 * Attention v3"; its section on the persistent kernel describes the alternative of one
 * program per multiprocessor that walks its share of the tiles in a loop (slower there,
 * from work imbalance). On MI355X workgroup w runs on XCD w mod 8 (8 XCDs, each with
 * its own L2), so the orders below either keep a head's tiles on one XCD or not.
 *   ATTN_SCHED_DEFAULT            per XCD, pairs of heads, longest query tile first (causal)
 *   ATTN_SCHED_XCD_ALL_HEADS      per XCD, all its heads together, longest first
 *   ATTN_SCHED_XCD_HEAD           per XCD, one head at a time, longest first
 *   ATTN_SCHED_XCD_NATURAL        per XCD, one head at a time, natural order
 *   ATTN_SCHED_LINEAR_LONGEST     no XCD remap (consecutive ids on one head), longest first
 *   ATTN_SCHED_LINEAR_NATURAL     no XCD remap, natural order
 *   ATTN_SCHED_PERSISTENT_STRIDE  one workgroup per CU; the workgroups of XCD x walk XCD x's
 *                                 tiles of the default order with a fixed stride
 *   ATTN_SCHED_PERSISTENT_QUEUE   one workgroup per CU; each XCD's workgroups take XCD x's
 *                                 tiles of the default order one at a time from a counter
 *                                 in `queue` (dynamic: a workgroup that finishes early
 *                                 takes the next tile)
 *   ATTN_SCHED_PERSISTENT_SNAKE  one workgroup per CU; the workgroups of XCD x take XCD x's
 *                                 tiles of the default order round by round, forward in
 *                                 even rounds and backward in odd ones (static: the longest
 *                                 tile of one round pairs with the shortest of the next)
 * In the persistent grids a workgroup's tile loads the next tile's Q rows and first K / V
 * tiles during its last steps (when its tile count is a multiple of 4). attn_fwd_bf16 and
 * attn_fwd_f16 run ATTN_SCHED_DEFAULT.
 * passes: ATTN_PASSES_AUTO as attn_fwd_bf16 (the same as ATTN_PASSES_TWO);
 *   ATTN_PASSES_EXACT the running-max pass alone, on every tile (the online softmax of the
 *   FlashAttention-2 digest, glossary: a per-tile max and a rescaled running sum);
 *   ATTN_PASSES_TWO the first-tile-reference pass, its marked query tiles redone by the
 *   running-max pass in the same launch, at any size.
 * dtype: ATTN_DTYPE_BF16 or ATTN_DTYPE_F16 (q, k, v, o of that type).
 * queue: ATTN_SCHED_PERSISTENT_QUEUE only (else ignored, may be NULL): caller-owned device
 *   memory of 16 int32 values, all zero before the first call; every call leaves them zero
 *   again when its kernels have run. Calls that share one queue array must not overlap in
 *   time (use one array per stream). A sched, passes or dtype value outside these lists,
 *   or a NULL or misaligned queue for ATTN_SCHED_PERSISTENT_QUEUE, is ATTN_ERR_INVALID_ARG. */
typedef enum {
  ATTN_SCHED_DEFAULT = 0,
  ATTN_SCHED_XCD_ALL_HEADS = 1,
  ATTN_SCHED_XCD_HEAD = 2,
  ATTN_SCHED_XCD_NATURAL = 3,
  ATTN_SCHED_LINEAR_LONGEST = 4,
  ATTN_SCHED_LINEAR_NATURAL = 5,
  ATTN_SCHED_PERSISTENT_STRIDE = 6,
  ATTN_SCHED_PERSISTENT_QUEUE = 7,
  ATTN_SCHED_PERSISTENT_SNAKE = 8
} attn_sched_t;

typedef enum { ATTN_PASSES_AUTO = 0, ATTN_PASSES_EXACT = 1, ATTN_PASSES_TWO = 2 } attn_passes_t;

typedef enum { ATTN_DTYPE_BF16 = 0, ATTN_DTYPE_F16 = 1 } attn_dtype_t;

attn_status_t attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                               int dtype, int sched, int passes, int32_t* queue, void* stream);

/* fp16 Q/K/V in, fp16 O out; as attn_fwd_bf16 with fp16 in place of bf16. */
attn_status_t attn_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                           void* stream);

/* fp32 Q/K/V in, fp32 O out: scores, probabilities and both contractions stay in fp32. */
attn_status_t attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                           void* stream);

/* fp8 attention ("8.3 FlashAttention-3", section 5: fp8 inputs with per-block scales).
 * q8/k8/v8 are OCP E4M3FN codes [B, H, N, d] (d = 64 or 128); q_scale/k_scale/v_scale are the
 * fp32 scales of each 128-row block, so the value of a code x in block t is
 * decode(x) * scale[b, h, t]. O is bf16 [B, H, N, d], LSE fp32 [B, H, N]. Scores
 * accumulate e4m3 x e4m3 products in fp32 and are scaled by q_scale * k_scale * scale;
 * the probabilities enter the P.V contraction (fp32 accumulation) as E4M3 codes of
 * 2^6 * P / w relative to a running max that trails the true one by at most 2 (log2
 * units), where w = U / v_scale[key block] in [2/3, 1] carries the key's V block scale
 * against the accumulator's unit U (a V block scale, moved only when w would leave that
 * range), so codes stay <= 384; O is divided by the sum of those rounded codes times w
 * and the LSE uses the unrounded fp32 sum. All scales must be finite and > 0. */
attn_status_t attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                           const float* q_scale, const float* k_scale, const float* v_scale,
                           void* o, float* lse,
                           int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                           void* stream);

/* fp8 input preparation ("8.3 FlashAttention-3", sections 5.1 and 5.2). x is bf16
 * [B, H, N, d] (d in {64, 128}). If `signs` (fp32 [d], every entry +1 or -1) is not
 * NULL, each row is first rotated: x <- fp32((x * signs) H_d) * fp32(1/sqrt(d)), with
 * H_d Sylvester's Hadamard matrix applied as the fast Walsh-Hadamard butterfly in fp32.
 * With signs == NULL the rows are quantised unrotated (used for V). Then, per block of
 * 128 rows of one (b, h): scale = fp32(amax / 448) (1 if the block is all zero), and
 * each code is the E4M3FN value nearest to clamp(fp32(x / scale), -448, 448), ties to
 * even. Writes x8 (uint8 [B, H, N, d]) and scales (fp32 [B, H, ceil(N/128)]). */
attn_status_t attn_quant_fp8(const void* x, uint8_t* x8, float* scales, const float* signs,
                             int64_t B, int64_t H, int64_t N, int64_t d, void* stream);

/* K and V preparation of one fp8 attention call in a single launch: k (bf16 [B, H, N, d])
 * rotated with `signs` and quantised, v quantised unrotated, each exactly as
 * attn_quant_fp8(k, signs) and attn_quant_fp8(v, NULL) would (same codes and scales).
 * signs must not be NULL. Outputs must not overlap each other or the inputs. */
attn_status_t attn_quant_fp8_kv(const void* k, const void* v, const float* signs, uint8_t* k8, uint8_t* v8,
                                float* k_scale, float* v_scale, int64_t B, int64_t H, int64_t N, int64_t d,
                                void* stream);

/* Q, K and V preparation of one fp8 attention call in a single launch ("8.3
 * FlashAttention-3", sections 5.1 and 5.2, as attn_quant_fp8): q and k (bf16 [B, H, N, d])
 * rotated with `signs` and quantised, v quantised unrotated, each exactly as
 * attn_quant_fp8(q, signs), attn_quant_fp8(k, signs) and attn_quant_fp8(v, NULL) would (same
 * codes and scales), with one launch's start and end instead of three. signs must not be
 * NULL. Outputs must not overlap each other or the inputs. */
attn_status_t attn_quant_fp8_qkv(const void* q, const void* k, const void* v, const float* signs, uint8_t* q8,
                                 uint8_t* k8, uint8_t* v8, float* q_scale, float* k_scale, float* v_scale,
                                 int64_t B, int64_t H, int64_t N, int64_t d, void* stream);

/* fp8 attention with the preparation of Q fused into the attention kernel ("8.3
 * FlashAttention-3", section 5.2: the Hadamard rotation is folded into the preprocessing
 * the kernel already does, at almost no extra cost). q is bf16 [B, H, N, d] (d = 64, 128);
 * each workgroup owns 256 query rows, i.e. two whole 128-row scale blocks, so it rotates
 * its rows (x * signs * H_d / sqrt(d), the fp32 butterfly of attn_quant_fp8), takes each
 * block's amax, scale and E4M3 codes in registers, and runs the attention of attn_fwd_fp8
 * on them. k8, v8, k_scale, v_scale as for attn_fwd_fp8 (e.g. from attn_quant_fp8_kv with
 * the same signs). If q8_out / q_scale_out are not NULL they receive the Q codes
 * (uint8 [B, H, N, d]) and scales (fp32 [B, H, ceil(N/128)]) the kernel made, which equal
 * those of attn_quant_fp8(q, signs); O and LSE then equal attn_fwd_fp8's on those codes
 * bit for bit. signs must not be NULL. */
attn_status_t attn_fwd_fp8_rotq(const void* q, const float* signs, const uint8_t* k8, const uint8_t* v8,
                                const float* k_scale, const float* v_scale, void* o, float* lse,
                                uint8_t* q8_out, float* q_scale_out,
                                int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                                void* stream);

/* Backward pass of attn_fwd_bf16 (FlashAttention-2 digest, key technical points and
 * method summary: the gradients are recomputed from the one stored log-sum-exp per row,
 * with the same split of the work as the forward pass). Inputs: q, k, v, the forward
 * outputs o and lse of the same call (same causal flag and scale), and dout = dL/dO, all
 * bf16 [B, H, N, d] except lse (fp32 [B, H, N]). Outputs (bf16 [B, H, N, d], round to
 * nearest even): dq, dk, dv, the gradients of sum(dout * O) with respect to q, k, v for
 * O = softmax(scale * q k^T [+ causal mask]) v. workspace is caller-owned device memory
 * of 2 * B * H * N floats; the call overwrites it (per row: -(dout . o), then -lse / scale)
 * and it holds nothing of use afterwards. The products use bf16 operands (P and dS
 * rounded to bf16) with fp32 accumulation. The call enqueues two kernels on `stream`;
 * dq, dk and dv are complete when the second has run. Outputs must not overlap each other,
 * the inputs or the workspace. */
attn_status_t attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                            const void* dout, void* dq, void* dk, void* dv, float* workspace,
                            int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                            void* stream);

/* fp16 tensors in and out; as attn_bwd_bf16 with fp16 in place of bf16. */
attn_status_t attn_bwd_f16(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, float* workspace,
                           int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                           void* stream);

/* Decoding step against a key/value cache (split-KV): q [B, H, Nq, d] with 1 <= Nq <= 32
 * query rows, k and v [B, H, Nk, d], no mask (every query row sees all Nk keys), in bf16;
 * writes O bf16 [B, H, Nq, d] and LSE fp32 [B, H, Nq] with the same definitions as
 * attn_fwd_bf16. The FlashAttention-2 digest (discussion points) asks whether decoding
 * needs its own kernel; here each head's keys are split (split s of n takes the 32-key
 * tiles s, s + n, ...), each split's partial O and LSE go to `workspace` (caller-owned
 * device memory of attn_decode_workspace_floats(...) fp32 values, overwritten, nothing of
 * use afterwards), and a second kernel merges them through the LSEs. Two kernels are
 * enqueued on `stream`. Nq outside [1, 32] is ATTN_ERR_INVALID_ARG; d as for the other
 * entry points. */
attn_status_t attn_decode_bf16(const void* q, const void* k, const void* v, void* o, float* lse, float* workspace,
                               int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                               void* stream);

/* fp16 tensors in and out; as attn_decode_bf16 with fp16 in place of bf16. */
attn_status_t attn_decode_f16(const void* q, const void* k, const void* v, void* o, float* lse, float* workspace,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                              void* stream);

/* attn_decode_bf16 for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and
 * results, with the per-split partials in a static device array of the library (64 MiB,
 * 2^24 floats, per GPU, held until the process ends) instead of a caller workspace. The
 * call allocates and frees nothing; the first call on a device looks up that device's
 * copy of the array. Sizes whose attn_decode_workspace_floats(...) exceeds 2^24 return
 * ATTN_ERR_SCRATCH_TOO_SMALL before anything is enqueued (at Nq = 32, d = 128 that is up
 * to 4064 (head, key split) pairs: any B*H <= 2016 at any Nk). Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (two streams, two threads) race and give
 * undefined results; calls enqueued on one stream do not overlap. */
attn_status_t attn_decode_bf16_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                       int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                       void* stream);

/* Workspace size (fp32 values) that attn_decode_* needs for these sizes; -1 if the sizes
 * are invalid. Host-only, no HIP call. */
int64_t attn_decode_workspace_floats(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d);

/* Calibration loops: what the part sustains at the clock it runs under load. kind 0 runs
 * a dense loop of independent 32x32x16 bf16 MFMAs, kind 1 a dense loop of v_exp_f32
 * (exponentials; "8.3 FlashAttention-3", section 1, names the exponential unit as the
 * softmax's bottleneck next to the matrix units), each in `workgroups` workgroups of 512
 * threads (the attention kernels' launch shape) for `iters` iterations. Kinds 2-5 price
 * the work the attention kernels put between their MFMAs: after every MFMA one fp32 FMA,
 * one exponential and one add (independent of the MFMAs), and a 16-byte LDS read feeding
 * the next MFMA after every MFMA (2), after every second MFMA (3), after every second
 * MFMA with one wave per SIMD instead of two (4: workgroups of 256 threads), or no LDS
 * read (5). seed: device memory of 4 uint32 values (operands, so that nothing folds);
 * out: device memory of workgroups * 512 floats, overwritten with one value per thread.
 * Kind 6 streams reads, the attainable rate of the HBM-bound kernels: workgroups of 256
 * threads each load one 16-byte element per iteration, the grid sweeping seed once front
 * to back, so seed must hold workgroups * 256 * iters 16-byte elements (only read); out
 * gets workgroups * 256 values. Kinds 7 and 8 read LDS, the operand path of the
 * attention kernels' MFMAs: 512-thread workgroups (one per CU) in which every lane reads
 * 16 bytes (ds_read_b128, kind 7) or 8 bytes (the transpose read ds_read_b64_tr_b16, kind
 * 8) per instruction, 16 instructions per iteration, from bank-disjoint addresses; seed and
 * out as for kinds 0-5. attn_calibrate_ops gives the operations (FLOPs, exponentials for
 * kind 1, bytes read for kinds 6-8) of one workgroup, so that rate = ops * workgroups /
 * elapsed time. kind outside [0, 8], workgroups or iters < 1, or a NULL pointer is
 * ATTN_ERR_INVALID_ARG (attn_calibrate_ops returns -1). */
attn_status_t attn_calibrate(int kind, const uint32_t* seed, float* out, int64_t workgroups, int iters,
                             void* stream);
int64_t attn_calibrate_ops(int kind, int iters);

/* Static description of a status code; never NULL. */
const char* attn_status_string(attn_status_t s);

/* Returns ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */
