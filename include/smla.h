/*
 * smla.h -- C ABI of libsmla: DSA sparse-MLA attention, forward and backward,
 * native on AMD Instinct MI355X (gfx950).
 *
 * The operation (absorbed-latent layout, one KV group shared by all heads):
 * each query token s has H heads of 576-wide queries and a row of `topk`
 * indices into a shared latent KV of 576-wide rows.  Index -1 marks a padding
 * slot.  Keys are the whole 576-wide rows, values their first 512 columns.
 *
 *   forward:   out[s,h,:] = sum_k p_k kv[J_k, :512],  p = softmax_k(scale * q[s,h] . kv[J_k])
 *              lse[s,h]   = natural-log normaliser of that softmax
 *   backward:  dq, dkv of the loss sum(dout * out), given out and lse
 *
 * Sources: the backward call takes (q, kv, out, dout, indices, lse, sm_scale)
 * and returns (dq, dkv), with the value width fixed at 512 (slime issue
 * #2201, "GLM-5.2 SparseMLA TileLang backward returns NaN gradients from
 * finite inputs", sections Strongest repro evidence and Suspected area).
 * Padding slots contribute exactly zero, the per-head softmax denominator is
 * floored at 1e-30 so an all-padding row outputs exact zeros with a finite
 * LSE, and dkv is accumulated through the indices (miles PR #2079 digest,
 * "fix GLM-5 sparse-MLA kernel -1 index OOB and NaN gradients", section
 * 实现拆解 items 1-3 and the key code snippets).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are device pointers owned by the caller, row-major
 *    and contiguous, 16-byte aligned.  bf16 tensors are passed as void*.
 *  - q [s_q, heads, 576] bf16; kv [s_kv, 576] bf16 (one KV group; the *_g
 *    calls below take several);
 *    indices [s_q, topk] int32; out and dout [s_q, heads, 512] bf16;
 *    lse [s_q, heads] fp32 (natural log); dq [s_q, heads, 576] bf16;
 *    dkv [s_kv, 576] bf16; dkv_f32 [s_kv, 576] fp32.
 *  - A slot is valid iff 0 <= index < s_kv.  -1 is padding.  Any other value
 *    is a contract violation; the kernels treat it as padding (they never
 *    read or write outside the buffers) and smla_validate_indices counts it.
 *  - Supported: heads in {8, 16, 32, 64, 128}; 1 <= topk <= 16384;
 *    1 <= s_kv < 2^24; s_q >= 0.  With s_q == 0 the pointers of the q-sized
 *    tensors (q, indices, out, dout, lse, dq) may be NULL; the forward then
 *    launches nothing and the backward only writes dkv (zeros).
 *  - Every call returns SMLA_OK (0) or a positive error code.  Argument errors
 *    are returned before anything is launched; smla_last_error() then gives a
 *    message (thread-local).  No exception crosses the ABI.
 *  - The library never allocates device memory and never synchronizes: work
 *    is enqueued on `stream` (a hipStream_t; NULL is the default stream) and
 *    the call returns.  Scratch space comes from the caller's `workspace`,
 *    whose size the *_workspace_size queries give.  A workspace must not be
 *    shared by calls that may run concurrently.
 *  - Inputs must be finite.  A nonfinite value in a kv row selected by one
 *    token can reach the other tokens of its query group through zero
 *    probabilities; rows never selected are never read.
 */
#ifndef SMLA_H_
#define SMLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_ABI_VERSION 1

enum smla_status {
  SMLA_OK = 0,
  SMLA_ERR_NULL = 1,        /* a required pointer is NULL */
  SMLA_ERR_SHAPE = 2,       /* unsupported heads/topk/s_kv, or negative sizes */
  SMLA_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  SMLA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
  SMLA_ERR_FLAGS = 5,       /* unknown flag bits, or a flag without its buffer */
  SMLA_ERR_HIP = 6,         /* a HIP launch failed */
  SMLA_ERR_DEVICE = 7       /* the current device is not gfx950 */
};

/* smla_bwd flags.  flags == 0 is the default, deterministic mode: dkv is a
 * per-row reduction over the (token, slot) pairs sorted by kv row, bitwise
 * reproducible run to run. */
#define SMLA_DKV_ACCUMULATE 1u  /* add into the caller's fp32 dkv_f32 instead of
                                   overwriting it; rows no valid slot selects
                                   are left untouched (bit for bit) */
#define SMLA_DKV_ATOMIC 2u      /* scatter dkv with fp32 atomic adds (the
                                   pages' default mode: slime issue #2201,
                                   "GLM-5.2 SparseMLA TileLang backward returns
                                   NaN gradients from finite inputs", Suspected
                                   area): each kv-block partial of the kv-major
                                   pass is added into an fp32 accumulator with
                                   no-return atomics, so results vary in the
                                   last bits run to run; the workspace must be
                                   smla_bwd_workspace_size(..., SMLA_DKV_ATOMIC)
                                   bytes */
#define SMLA_PLAN_READY 4u      /* smla_fwd_ex / smla_bwd: the workspace already
                                   holds the index plan smla_plan built for the
                                   same indices and sizes; skip planning */
#define SMLA_FP8_POW2_SCALES 16u /* smla_fwd_fp8: every scale of the fp8 kv
                                   records is a power of two (E8M0-style
                                   scales); each pair of codes then converts in
                                   one scaled instruction, which applies only
                                   the scale's exponent -- with any other scale
                                   the values are wrong (no error is raised) */
#define SMLA_DKV_STORED_P 8u    /* smla_bwd: the dq pass stores P and
                                   sm_scale * dS (bf16, per union entry and
                                   query row) in the workspace and the dkv pass
                                   reads them instead of recomputing the scores
                                   and dP; same results within rounding, one
                                   recompute of the scores per backward; the
                                   workspace must be
                                   smla_bwd_workspace_size(..., SMLA_DKV_STORED_P)
                                   bytes (256 bytes more per union slot bound:
                                   s_q * topk * 256 at most) */

/* Index plan: which slots are valid (an index is a row iff it is not -1 and
 * lies in [0, s_kv): miles PR #2079 digest, "fix GLM-5 sparse-MLA kernel -1
 * index OOB and NaN gradients", 实现拆解 item 1), grouped for the kernels --
 * per query group the union of its tokens' rows with token masks, per
 * (64-row kv block, query group) the tokens' row masks, and the work orders.
 * It depends only on indices and the sizes, so a training step can build it
 * once and pass SMLA_PLAN_READY to smla_fwd_ex and smla_bwd with the same
 * workspace.  workspace: at least smla_bwd_workspace_size(...) bytes,
 * 256-byte aligned, owned by the caller, which must not change indices, the
 * sizes or the workspace between this call and the calls that use the plan. */
int smla_plan(const int32_t* indices, int64_t s_q, int64_t s_kv, int32_t heads, int32_t topk,
              void* workspace, size_t workspace_bytes, void* stream);

/* Forward.
 * in:  q, kv, indices, sm_scale (the softmax scale applied to q . k).
 * out: out [s_q, heads, 512] bf16 -- exact zeros for rows without a valid slot;
 *      lse [s_q, heads] fp32 natural log -- ln(1e-30) for rows without a valid
 *      slot, otherwise max_k z_k + ln(sum_k exp(z_k - max)).
 * workspace: at least smla_fwd_workspace_size(...) bytes, 256-byte aligned. */
int smla_fwd(const void* q, const void* kv, const int32_t* indices,
             int64_t s_q, int64_t s_kv, int32_t heads, int32_t topk, float sm_scale,
             void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* smla_fwd with flags: 0 (= smla_fwd) or SMLA_PLAN_READY (the workspace
 * holds smla_plan's plan for these indices and sizes; it is not rebuilt). */
int smla_fwd_ex(const void* q, const void* kv, const int32_t* indices,
                int64_t s_q, int64_t s_kv, int32_t heads, int32_t topk, float sm_scale,
                void* out, float* lse, uint32_t flags, void* workspace, size_t workspace_bytes,
                void* stream);

/* smla_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, bit for bit, with its scratch space in a buffer the
 * library holds on each device -- SMLA_NOALLOC_SCRATCH_BYTES, 64 MiB, from
 * the first call on a device until the process ends -- so the call itself
 * allocates nothing.  The caller still owns q, kv, indices, out and lse.
 * Shapes whose smla_fwd_workspace_size(s_q, s_kv, heads, topk) exceeds
 * SMLA_NOALLOC_SCRATCH_BYTES (about s_q * topk * 5 bytes; e.g. s_q = 4096,
 * topk = 2048 needs 42 MB) return SMLA_ERR_WORKSPACE before anything is
 * launched.  All calls on one device share its buffer: calls that may run
 * concurrently on that device (different streams, or different host threads
 * without ordering) race and must not overlap; calls on one stream are
 * ordered.  Nothing in the buffer needs to start cleared. */
#define SMLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int smla_fwd_noalloc(const void* q, const void* kv, const int32_t* indices,
                     int64_t s_q, int64_t s_kv, int32_t heads, int32_t topk, float sm_scale,
                     void* out, float* lse, void* stream);

size_t smla_fwd_workspace_size(int64_t s_q, int64_t s_kv, int32_t heads, int32_t topk);

/* Backward.
 * in:  q, kv, indices and sm_scale as given to the forward; out and lse as the
 *      forward returned them (delta = rowsum(dout * out) uses this out, the
 *      probabilities are recomputed as exp(scale q.k - lse) from this lse);
 *      dout [s_q, heads, 512] bf16.
 * out: dq [s_q, heads, 576] bf16 (required);
 *      dkv [s_kv, 576] bf16 (may be NULL if only dkv_f32 is wanted);
 *      dkv_f32 [s_kv, 576] fp32 (may be NULL; required with SMLA_DKV_ACCUMULATE).
 *      Rows of dkv that no valid slot selects are exact zeros (without
 *      SMLA_DKV_ACCUMULATE).  dkv and dkv_f32 must not both be NULL.
 * flags: 0, SMLA_DKV_ACCUMULATE, SMLA_DKV_ATOMIC and/or SMLA_PLAN_READY.
 * workspace: at least smla_bwd_workspace_size(...) bytes, 256-byte aligned. */
int smla_bwd(const void* q, const void* kv, const void* out, const void* dout,
             const int32_t* indices, const float* lse,
             int64_t s_q, int64_t s_kv, int32_t heads, int32_t topk, float sm_scale,
             void* dq, void* dkv, float* dkv_f32, uint32_t flags,
             void* workspace, size_t workspace_bytes, void* stream);

size_t smla_bwd_workspace_size(int64_t s_q, int64_t s_kv, int32_t heads, int32_t topk,
                               uint32_t flags);

/* KV groups.  The kernel excerpts of the miles PR #2079 digest ("fix GLM-5
 * sparse-MLA kernel -1 index OOB and NaN gradients", key code snippets) index
 * the indices and the kv by a kv-group coordinate derived from the query head
 * block: the heads split into kv_groups equal blocks and block g attends over
 * kv group g with its own index rows.  These calls take that layout:
 *   q [s_q, heads, 576], out / dout [s_q, heads, 512], lse [s_q, heads],
 *   dq [s_q, heads, 576] as before; kv [s_kv, kv_groups, 576] bf16;
 *   indices [s_q, kv_groups, topk] int32 (row (s, g) lists rows of kv group
 *   g; valid iff 0 <= index < s_kv, as before); dkv [s_kv, kv_groups, 576]
 *   bf16 and dkv_f32 [s_kv, kv_groups, 576] fp32.
 * Head h uses kv group h / (heads / kv_groups).  heads / kv_groups must be 8,
 * 16, 32, 64 or 128; 1 <= kv_groups <= 64; s_kv * kv_groups < 2^24.  Flags,
 * workspace rules and errors are those of the calls above (SMLA_PLAN_READY
 * needs a plan from smla_plan_g with the same sizes).  kv_groups = 1 is
 * exactly smla_plan / smla_fwd_ex / smla_bwd. */
int smla_plan_g(const int32_t* indices, int64_t s_q, int64_t s_kv, int32_t heads,
                int32_t kv_groups, int32_t topk, void* workspace, size_t workspace_bytes,
                void* stream);
int smla_fwd_g(const void* q, const void* kv, const int32_t* indices,
               int64_t s_q, int64_t s_kv, int32_t heads, int32_t kv_groups, int32_t topk,
               float sm_scale, void* out, float* lse, uint32_t flags, void* workspace,
               size_t workspace_bytes, void* stream);
size_t smla_fwd_workspace_size_g(int64_t s_q, int64_t s_kv, int32_t heads, int32_t kv_groups,
                                 int32_t topk);
int smla_bwd_g(const void* q, const void* kv, const void* out, const void* dout,
               const int32_t* indices, const float* lse,
               int64_t s_q, int64_t s_kv, int32_t heads, int32_t kv_groups, int32_t topk,
               float sm_scale, void* dq, void* dkv, float* dkv_f32, uint32_t flags,
               void* workspace, size_t workspace_bytes, void* stream);
size_t smla_bwd_workspace_size_g(int64_t s_q, int64_t s_kv, int32_t heads, int32_t kv_groups,
                                 int32_t topk, uint32_t flags);

/* Forward over an fp8 kv cache (a serving-side variant: the sources name fp8
 * as a rollout format, Megatron-Bridge and miles digests; the record layout
 * is this library's).  kv_fp8 holds one 656-byte record per kv row
 * ([s_kv, kv_groups, 656] bytes, 16-byte aligned): bytes 0..511 the latent
 * columns 0..511 as OCP e4m3 codes (4 exponent bits, bias 7, 3 mantissa
 * bits), bytes 512..527 four little-endian fp32 scales (scale b multiplies
 * columns 128b .. 128b+127), bytes 528..655 the rope columns 512..575 as
 * bf16.  Each selected row is decoded as code * scale, rounded to bf16, and
 * the forward then runs as smla_fwd_g does; every other argument, the
 * workspace (smla_fwd_workspace_size_g) and the errors are those of
 * smla_fwd_g; flags: 0, SMLA_PLAN_READY and/or SMLA_FP8_POW2_SCALES.  Codes
 * 0x7F / 0xFF (NaN) must not occur. */
int smla_fwd_fp8(const void* q, const void* kv_fp8, const int32_t* indices,
                 int64_t s_q, int64_t s_kv, int32_t heads, int32_t kv_groups, int32_t topk,
                 float sm_scale, void* out, float* lse, uint32_t flags, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Index production, the step before the attention: for every query row s,
 * the top-k kv positions of its indexer logits inside its key range
 * [ks[s], ke[s]) (clipped to [0, s_kv)), with k capped at the range length
 * and the row padded back to the fixed width topk with -1 -- Megatron-Bridge
 * PR #17, "GLM-5 DSA option: tilelang (2/2)", Bug fixes.  The chosen
 * positions are written in ascending order; among equal logits the smaller
 * position wins.
 * in:  logits [s_q, ld] fp32 (row s at logits + s * ld; columns 0..s_kv-1
 *      are read, only inside the row's range; values must be finite);
 *      ks, ke [s_q] int32 (ke <= ks is an empty range: a row of -1).
 * out: indices [s_q, topk] int32, ready for smla_fwd / smla_bwd.
 * Errors: SMLA_ERR_NULL, SMLA_ERR_SHAPE (s_q < 0, s_kv < 1, ld < s_kv, topk
 * outside 1..16384), SMLA_ERR_ALIGN (pointers must be 4-byte aligned). */
int smla_topk_indices(const float* logits, int64_t s_q, int64_t s_kv, int64_t ld,
                      const int32_t* ks, const int32_t* ke, int32_t topk, int32_t* indices,
                      void* stream);

/* Nonfinite diagnostics: the device-side steps of the finite-check workflow
 * of slime issue #2201, "GLM-5.2 SparseMLA TileLang backward returns NaN
 * gradients from finite inputs", Workarounds tested (check the backward's dq /
 * dkv for NaN / Inf; when some are found, take a reference's values at those
 * entries only; writing zeros there instead was the diagnostic confinement
 * patch).  An entry is nonfinite when all its exponent bits are ones.
 *
 * dtype: SMLA_DTYPE_BF16 (2-byte elements) or SMLA_DTYPE_F32 (4-byte).
 * x, ref: n elements, device memory, 16-byte aligned.  count: a device
 * pointer to one uint64, 8-byte aligned; the number of nonfinite entries
 * found (count) or replaced (replace) is ADDED to *count, so one zeroed
 * counter can gather several buffers before a single read back.
 * smla_nonfinite_replace writes ref[i] into x[i] wherever x[i] is nonfinite
 * (ref NULL: +0) and leaves every other entry untouched; ref must not
 * overlap x except as the same buffer.  The library computes no reference:
 * the caller supplies one.
 * Errors: SMLA_ERR_NULL, SMLA_ERR_SHAPE (n < 0, unknown dtype),
 * SMLA_ERR_ALIGN. */
#define SMLA_DTYPE_BF16 0
#define SMLA_DTYPE_F32 1
int smla_nonfinite_count(const void* x, int32_t dtype, int64_t n, unsigned long long* count,
                         void* stream);
int smla_nonfinite_replace(void* x, const void* ref, int32_t dtype, int64_t n,
                           unsigned long long* count, void* stream);

/* Counts index entries that are neither -1 nor in [0, s_kv) and stores the
 * count in *n_bad (a device pointer to one uint64, overwritten). */
int smla_validate_indices(const int32_t* indices, int64_t s_q, int32_t topk, int64_t s_kv,
                          unsigned long long* n_bad, void* stream);

/* Kernel timing, for benchmarks (not thread-safe).  Between
 * smla_timing_start(max_launches) and smla_timing_stop(), every launch step
 * of this library is bracketed by two HIP events recorded on its stream (at
 * most max_launches steps are recorded; the events are created by
 * smla_timing_start and destroyed by the next start).  smla_timing_read waits
 * for the recorded events of the steps named `kernel` and returns how many
 * were recorded and their summed duration in milliseconds.  Step names:
 * "plan", "order" (work order of the query groups), "fwd",
 * "bwd_dq", "dkv_schedule" (chunk lists and the dkv work split: two small
 * kernels), "dkv_clear" (atomic mode: zeroing the accumulator), "bwd_dkv"
 * (the dkv kernel alone), "dkv_finalize", "validate". */
int smla_timing_start(int max_launches);
int smla_timing_stop(void);
int smla_timing_read(const char* kernel, int* launches, double* total_ms);

/* Message of the last error returned on this thread ("" if none). */
const char* smla_last_error(void);

/* SMLA_ABI_VERSION of the built library. */
int smla_version(void);

/* 1 if `device` is a gfx950 GPU this library was built for, else 0. */
int smla_device_supported(int device);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H_ */
