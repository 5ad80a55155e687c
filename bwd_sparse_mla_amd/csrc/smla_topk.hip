// Index production (gfx950): the top-k kv positions of each query's indexer
// logits, the step that makes the index rows the attention consumes.
//
// Query row s owns the key range [ks[s], ke[s]) (its sequence's start and its
// causal end; clipped to [0, s_kv)).  With n = the range's length and K the
// fixed width, the row's output is the min(K, n) positions with the largest
// logits (ties to the smaller position), ascending, then -1 up to K.  The cap
// and the -1 padding follow Megatron-Bridge PR #17, "GLM-5 DSA option:
// tilelang (2/2)", Bug fixes (a fixed-width top-k over a sequence shorter than
// the width fails; k is capped at the row length and the selection padded back
// to the width with -1).  The output order and the tie rule are this
// library's: the attention treats a row's slots as a set.
//
// One workgroup per query row.  A row no longer than K is the whole range.  A
// longer row finds the K-th largest key by an MSB-first radix select over
// order-preserving 32-bit keys (four 8-bit digits; per-wave LDS histograms),
// then writes, in position order, every key above it and the first keys equal
// to it.  The row's keys are read from HBM once and kept in LDS when they fit.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

constexpr int TOPK_THREADS = 256;
constexpr int TOPK_LDS_KEYS = 32768;   // rows up to this long keep their keys in LDS

// Unsigned keys that order like the floats (finite values); -0 and +0 get the
// same key, as they compare equal.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  b = b == 0x80000000u ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t keys[TOPK_LDS_KEYS];
  __shared__ int hist[4][256];
  __shared__ int scratch[8];
  __shared__ int s_digit, s_rank;

  const int64_t s = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int K = a.topk;
  const int64_t lo = max<int64_t>(0, a.ks[s]);
  const int64_t hi = min<int64_t>(a.s_kv, a.ke[s]);
  const int n = hi > lo ? (int)(hi - lo) : 0;
  int32_t* out = a.out + s * (int64_t)K;

  if (n <= K) {   // the whole range, then padding
    for (int i = tid; i < K; i += TOPK_THREADS) out[i] = i < n ? (int32_t)(lo + i) : -1;
    return;
  }

  const float* row = a.logits + s * a.ld + lo;
  const bool cached = n <= TOPK_LDS_KEYS;
  auto key_at = [&](int i) __attribute__((always_inline)) {
    return cached ? keys[i] : order_key(row[i]);
  };

  // Radix select: after the pass for digit d, `prefix` holds the K-th largest
  // key's digits above and at d, and `rank` its rank (1-based, from the top)
  // among the keys that share them.
  uint32_t prefix = 0, pmask = 0;
  int rank = K;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = tid; b < 4 * 256; b += TOPK_THREADS) (&hist[0][0])[b] = 0;
    __syncthreads();
    if (pass == 0) {
      for (int i = tid; i < n; i += TOPK_THREADS) {
        const uint32_t k = order_key(row[i]);
        if (cached) keys[i] = k;
        atomicAdd(&hist[wave][k >> 24], 1);
      }
    } else {
      for (int i = tid; i < n; i += TOPK_THREADS) {
        const uint32_t k = key_at(i);
        if ((k & pmask) == prefix) atomicAdd(&hist[wave][(k >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    // Thread t holds digit 255 - t: a scan from the top gives the count of
    // keys above each digit.
    const int d = 255 - tid;
    const int c = hist[0][d] + hist[1][d] + hist[2][d] + hist[3][d];
    int total;
    const int above = block_exclusive_scan256(c, scratch, &total);
    if (above < rank && rank <= above + c) {
      s_digit = d;
      s_rank = rank - above;
    }
    __syncthreads();
    prefix |= (uint32_t)s_digit << shift;
    pmask |= 255u << shift;
    rank = s_rank;
    __syncthreads();
  }

  // prefix is now the K-th largest key T: the K - rank keys above it and the
  // first `rank` keys equal to it (in position order) are the selection.
  const uint32_t T = prefix;
  const int C = (n + TOPK_THREADS - 1) / TOPK_THREADS;   // positions per thread, contiguous
  const int b0 = min(n, tid * C), b1 = min(n, b0 + C);
  int gt = 0, eq = 0;
  for (int i = b0; i < b1; ++i) {
    const uint32_t k = key_at(i);
    gt += k > T;
    eq += k == T;
  }
  int eq_total;
  const int eq_before = block_exclusive_scan256(eq, scratch, &eq_total);
  int take_eq = min(eq, max(0, rank - eq_before));
  int total_sel;
  int pos = block_exclusive_scan256(gt + take_eq, scratch, &total_sel);
  for (int i = b0; i < b1; ++i) {
    const uint32_t k = key_at(i);
    bool take = k > T;
    if (k == T && take_eq > 0) {
      take = true;
      --take_eq;
    }
    if (take && pos < K) out[pos++] = (int32_t)(lo + i);   // pos < K always: the counts sum to K
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.s_q == 0) return hipSuccess;
  topk_kernel<<<dim3((unsigned)a.s_q), dim3(TOPK_THREADS), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace smla
