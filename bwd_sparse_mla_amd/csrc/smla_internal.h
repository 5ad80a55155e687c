// Host-visible launch interface between the C ABI (smla_capi.hip) and the
// kernels.  Nothing here is exported from the shared library.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace smla {

// Rows of queries one workgroup of the query-major kernels owns: T = 64 / H
// consecutive tokens ("query group").  64 rows fill four 16-row MFMA tiles.
constexpr int GROUP_ROWS = 64;
constexpr int TILE_KV = 64;      // kv rows per LDS tile / per kv block
constexpr int MAX_TOPK = 16384;
constexpr int64_t MAX_SKV = (int64_t(1) << 24) - 1;

inline int tokens_per_group(int heads) { return GROUP_ROWS / heads; }

// Sizes derived from the problem shape; also the workspace layout.
struct Plan {
  int64_t s_q = 0, s_kv = 0;
  int heads = 0, topk = 0;
  int T = 0;          // tokens per query group
  int64_t G = 0;      // number of query groups
  int64_t NB = 0;     // number of 64-row kv blocks
  int64_t qcap = 0;   // union entries reserved per group: T * topk rounded up to 64
  int64_t rcap = 0;   // kv-block records reserved per group: T * min(T * topk, NB)
  // byte offsets into the workspace
  size_t off_qcount = 0, off_xcount = 0, off_xtotal = 0, off_qrow = 0, off_qmask = 0;
  size_t off_ktab = 0, off_krmask = 0, off_delta = 0;
  size_t off_clist = 0, off_nchunk = 0, off_part = 0, off_ptouch = 0;
  size_t off_gorder = 0, off_spre = 0, off_wstart = 0;
  size_t off_kbase = 0, off_korm = 0, off_cbase = 0, off_cmask = 0;
  size_t off_acc32 = 0;   // atomic dkv mode only: [NB * 64, 576] fp32 accumulator
  size_t off_pds = 0;     // stored-P mode only: [G, qcap, 2, 64] bf16 P and scale * dS
  size_t bytes = 0;
};

Plan make_plan(int64_t s_q, int64_t s_kv, int heads, int topk, bool backward, bool atomic = false,
               bool stored_p = false);

struct PlanArgs {
  const int32_t* idx;
  int64_t s_q, s_kv;
  int topk;
  int idx_shift;      // query row t reads index row t >> idx_shift (1: two rows per token)
  // kv groups: index row r belongs to kv group g = r % kv_groups, and its
  // valid value j (0 <= j < s_kv_idx) names flat kv row j * kv_groups + g of
  // the [s_kv_idx, kv_groups, 576] kv (s_kv = s_kv_idx * kv_groups rows).
  // The bitmaps, the union order and the kv blocks (ktab, krmask, kbase,
  // korm) use block row g * s_kv_idx + j instead, so that a 64-row block
  // holds one group's rows; qrow holds flat rows.
  int kv_groups;
  int64_t s_kv_idx;
  // group-major rows (0: token-major): row r is the (group, token) pair
  // (r / gmajor_s, r % gmajor_s), kv group r / gmajor_s, and its indices are
  // the caller's token-major index row caller_token(r, gmajor_s, kv_groups)
  int64_t gmajor_s;
  int64_t G, NB, qcap, rcap;
  int* qcount;        // [G]   union entries (main + extra) per group
  int* xcount;        // [G]   extra entries (repeated slots) per group
  int* xtotal;        // [1]   sum of xcount (written by the order kernel)
  int32_t* qrow;      // [G, qcap] flat kv row of each union entry
  uint8_t* qmask;     // [G, qcap] mask of the group's tokens that select it
  int2* ktab;         // [NB, G] (record start within the group, T) or (0, 0); may be null
  unsigned long long* krmask;  // [G, rcap] 64-bit row masks, T per (block, group) pair
  int* kbase;                  // [NB, G] first main union entry of the group in the block (with records)
  unsigned long long* korm;    // [NB, G] OR of the group's row masks for the block (with records)
};

// fp8 kv row record: e4m3 latent columns 0..511, then the fp32 scales of
// columns 128b .. 128b+127 (b = 0..3), then the bf16 rope columns 512..575.
constexpr int FP8_REC_BYTES = 656;
constexpr int FP8_SCALE_OFF = 512;
constexpr int FP8_ROPE_OFF = 528;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* kv;
  // fp8 kv (fp8 forward only; kv is then unused): FP8_REC_BYTES per row --
  // 512 e4m3 latent values, 4 fp32 scales (one per 128 columns), 64 bf16 rope
  const uint8_t* kv8;
  int64_t s_q, s_kv;
  float scale_log2;   // sm_scale * log2(e)
  int64_t G, qcap;
  const int* qcount;
  const int32_t* qrow;
  const uint8_t* qmask;
  const int* order;   // [G] groups by decreasing union size: workgroup i runs order[i]
  uint16_t* out;
  float* lse;
  // Several kv groups (pair_g > 1): the kernel's token tok is the (group,
  // token) pair g pair_s + s, and q, out and lse are the caller's token-major
  // rows (see caller_token).
  int64_t pair_s;
  int pair_g;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const uint16_t* out;
  const uint16_t* dout;
  const float* lse;
  int64_t s_q, s_kv;
  float scale, scale_log2;
  int64_t G, NB, qcap, rcap;
  int64_t NU;         // dkv units: kv blocks (NB) or, in the stored-P form, pairs of blocks
  int ub;             // kv blocks per dkv unit: 1, or 2 in the stored-P form
  const int* qcount;
  const int* xcount;
  const int* xtotal;
  const int32_t* qrow;
  const uint8_t* qmask;
  const int2* ktab;
  const unsigned long long* krmask;
  const int* gorder;  // [G] groups by decreasing union size (dq pass)
  // Several kv groups (pair_g > 1): q, out, dout and dq are the caller's
  // token-major rows (see caller_token); lse is a group-major copy.
  int64_t pair_s;
  int pair_g;
  // The dkv pass's kv blocks and finalize's rows are block rows: block row
  // b is row b % kvs of kv group b / kvs, flat row (b % kvs) * kvg + b / kvs
  // (kvg = 1: the same row).
  int kvg;
  int64_t kvs;
  int* spre;          // [NU + 1] dkv sub-chunks before each unit (exclusive prefix; [NU] = total)
  int* wstart;        // [DKV_WGS] first dkv unit of each dkv workgroup's range
  float* delta;       // [s_q * H] rowsum(dout * out), written by the dq pass
  int2* clist;        // [NU, G] per unit: (group, record start), compacted
  const int* kbase;   // [NB, G] from the planner (stored-P mode)
  const unsigned long long* korm;   // [NB, G] from the planner (stored-P mode)
  int* cbase;         // [NU, G, 2] parallel to clist: per block of the unit, the chunk's first
                      // union entry there (stored-P form)
  unsigned long long* cmask;   // [NU, G, 2] parallel to clist: per block, the rows the chunk selects
  uint16_t* pds;      // stored-P mode: [G, qcap, 2, 64] bf16 P and scale * dS per union entry and
                      // group row, written by the dq pass and read by the dkv pass; else null
  int* nchunk;        // [NU] entries of clist per unit
  float* part;        // [DKV_WGS + NU, 64 ub, 576] fp32 partial dkv per (workgroup w, unit u): slot w + u
  unsigned long long* ptouch;  // [DKV_WGS + NU, 2] rows each partial touched (per 64-row block)
  float* acc32;       // atomic mode: [NB * 64, 576] fp32 dkv accumulated with atomics; else null
  uint16_t* dq;
  uint16_t* dkv;      // may be null
  float* dkv_f32;     // may be null
  int accumulate;
};

struct TopkArgs {
  const float* logits;   // [s_q, ld] fp32, row s holds the logits of query s over kv rows 0..s_kv-1
  int64_t s_q, s_kv, ld;
  const int32_t* ks;     // [s_q] first kv row of each query's range
  const int32_t* ke;     // [s_q] one past its last
  int topk;
  int32_t* out;          // [s_q, topk]
};

// Pair-block permutation between token-major order (block s G + g) and
// group-major order (block g S + s) of S x G blocks of `block_bytes` bytes
// (a multiple of 4; of 16 for the 16-byte path): to_gmajor copies token-major
// src into group-major dst, else the reverse.
hipError_t launch_permute_pairs(const void* src, void* dst, int64_t S, int G, int64_t block_bytes,
                                bool to_gmajor, hipStream_t stream);
hipError_t launch_fill_u32(void* ptr, size_t n_words, uint32_t value, hipStream_t stream);
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);
hipError_t launch_plan(const PlanArgs& a, int heads, hipStream_t stream);
// fp8: 0 bf16 kv rows, 1 fp8 records (fp32 scales), 2 fp8 records with power-of-two scales
hipError_t launch_fwd(const FwdArgs& a, int heads, hipStream_t stream, int fp8 = 0);
hipError_t launch_bwd_dq(const BwdArgs& a, int heads, hipStream_t stream);
// Work order of the query groups: decreasing union size (largest first).
hipError_t launch_order_groups(const int* qcount, const int* xcount, int64_t G, int* order, int* xtotal,
                               hipStream_t stream);
// dkv pass: schedule (chunk lists and work order), main kernel, finalize.
// The chunk lists are built by the first workgroups of the dq launch; with no
// dq launch (s_q == 0) lists_built is false and a kernel of their own does it.
hipError_t launch_dkv_schedule(const BwdArgs& a, bool lists_built, hipStream_t stream);
hipError_t launch_bwd_dkv(const BwdArgs& a, int heads, hipStream_t stream);
hipError_t launch_dkv_finalize(const BwdArgs& a, int heads, hipStream_t stream);
// dkv split schedule: chunks a split covers at least, and the split count.
// The dkv pass runs DKV_WGS workgroups (one per CU of the part), each over an
// equal share of all sub-chunks in block order (stream-K style); a workgroup
// w that covers sub-chunks of block b leaves its partial in slot w + b.
constexpr int DKV_WGS = 256;
// Up to this many dkv units the dkv and finalize workgroups compute the
// sub-chunk prefix themselves (no prefix launch, spre / wstart unused).
constexpr int64_t DKV_INLINE_UNITS = 2048;
// Nonfinite diagnostics over n elements of es (2: bf16, 4: fp32) bytes at
// x: count the NaN / Inf entries, or replace them from ref (null: zero);
// the count is added into *count.
hipError_t launch_nonfinite(void* x, const void* ref, int64_t n, int es, bool replace,
                            unsigned long long* count, hipStream_t stream);
hipError_t launch_validate(const int32_t* idx, int64_t n, int64_t s_kv,
                           unsigned long long* n_bad, hipStream_t stream);

}  // namespace smla
