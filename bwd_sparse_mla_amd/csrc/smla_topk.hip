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
// order-preserving 32-bit keys (digits of 10, 10, 10 and 2 bits; one LDS
// histogram of 1024 bins), then
// writes, in position order, every key above it and the first keys equal to
// it, each thread over its own contiguous run of positions.  The row's logits
// are read from HBM once, with 16-byte loads several in flight per thread, and
// their keys kept in LDS when the row fits the cache
// (sized at launch from s_kv, so short-context launches run several
// workgroups per CU).  The select stops early once the keys sharing the
// selected digits are exactly the ones still needed.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

constexpr int TOPK_THREADS = 256;
constexpr int TOPK_SMALL_CACHE = 8192;    // keys cached per row when s_kv <= 8192
constexpr int TOPK_LARGE_CACHE = 32768;   // otherwise rows up to this long are cached
constexpr int TOPK_LOADS = 8;             // 16-byte loads in flight per thread
constexpr int TOPK_BATCH = 8;             // keys read ahead per thread in the LDS passes
constexpr int TOPK_BINS = 1024;           // histogram bins: digits of up to 10 bits
// The radix digits, most significant first: the first one (sign, exponent and
// one mantissa bit) already spreads logits of one scale over many bins.
constexpr int TOPK_PASSES = 4;

// Unsigned keys that order like the floats (finite values); -0 and +0 get the
// same key, as they compare equal.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  b = b == 0x80000000u ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int CACHE>
__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t keys[CACHE + 8 + (CACHE + 8) / 32];
  __shared__ int hist[TOPK_BINS];
  __shared__ int scratch[8];
  __shared__ int s_digit, s_rank, s_count;

  const int64_t s = a.s_q - 1 - (int64_t)blockIdx.x;   // last rows first (on causal rows, the longest)
  const int tid = threadIdx.x;
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
  const bool cached = n <= CACHE;
  // Elements before the row's first 16-byte boundary are read one by one.
  // Key i is cached at c + c / 32 with c = i + pad (one spare word after every
  // 32 keys): a thread that walks 32 consecutive keys then sits on its own
  // bank, and coalesced walks stay conflict-free.
  const int head = min(n, (int)(((16u - ((uint32_t)reinterpret_cast<uintptr_t>(row) & 15u)) & 15u) >> 2));
  const int pad = (4 - head) & 3;
  auto cix = [&](int i) __attribute__((always_inline)) {
    const int c = i + pad;
    return c + (c >> 5);
  };
  auto key_at = [&](int i) __attribute__((always_inline)) {
    return cached ? keys[cix(i)] : order_key(row[i]);
  };

  for (int b = tid; b < TOPK_BINS; b += TOPK_THREADS) hist[b] = 0;
  __syncthreads();
  // Pass 0 reads the logits: the elements before the first 16-byte boundary
  // one by one, the body as float4 (TOPK_LOADS per thread in flight), the
  // tail one by one; each key is cached and counted by its top digit.
  auto first = [&](int i, float x) __attribute__((always_inline)) {
    const uint32_t k = order_key(x);
    if (cached) keys[cix(i)] = k;
    atomicAdd(&hist[k >> 22], 1);
  };
  if (tid < head) first(tid, row[tid]);
  const int nv4 = (n - head) >> 2;
  const float4* row4 = reinterpret_cast<const float4*>(row + head);
  for (int base = 0; base < nv4; base += TOPK_LOADS * TOPK_THREADS) {
    float4 v[TOPK_LOADS];
#pragma unroll
    for (int j = 0; j < TOPK_LOADS; ++j) {
      const int i = base + j * TOPK_THREADS + tid;
      v[j] = i < nv4 ? row4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < TOPK_LOADS; ++j) {
      const int i = base + j * TOPK_THREADS + tid;
      if (i < nv4) {
        const uint4 k = make_uint4(order_key(v[j].x), order_key(v[j].y), order_key(v[j].z),
                                   order_key(v[j].w));
        if (cached) {   // four keys inside one 32-key run: consecutive words
          uint32_t* kp = &keys[cix(head + 4 * i)];
          kp[0] = k.x;
          kp[1] = k.y;
          kp[2] = k.z;
          kp[3] = k.w;
        }
        atomicAdd(&hist[k.x >> 22], 1);
        atomicAdd(&hist[k.y >> 22], 1);
        atomicAdd(&hist[k.z >> 22], 1);
        atomicAdd(&hist[k.w >> 22], 1);
      }
    }
  }
  for (int i = head + 4 * nv4 + tid; i < n; i += TOPK_THREADS) first(i, row[i]);

  // Radix select: after the pass for digit d, `prefix` holds the K-th largest
  // key's digits above and at d (`pmask` marks them), and `rank` its rank
  // (1-based, from the top) among the keys that share them.  When exactly
  // `rank` keys share them, every one is taken and the select stops.
  uint32_t prefix = 0, pmask = 0;
  int rank = K;
#pragma unroll 1
  for (int pass = 0; pass < TOPK_PASSES; ++pass) {
    const int shift = pass < 3 ? 22 - 10 * pass : 0;     // digits [31:22], [21:12], [11:2], [1:0]
    const uint32_t dmask = pass < 3 ? 1023u : 3u;
    if (pass > 0) {
      for (int b = tid; b < TOPK_BINS; b += TOPK_THREADS) hist[b] = 0;
      __syncthreads();
      for (int base = 0; base < n; base += TOPK_BATCH * TOPK_THREADS) {
        uint32_t k[TOPK_BATCH];
#pragma unroll
        for (int j = 0; j < TOPK_BATCH; ++j) {
          const int i = base + j * TOPK_THREADS + tid;
          k[j] = i < n ? key_at(i) : 0u;
        }
#pragma unroll
        for (int j = 0; j < TOPK_BATCH; ++j) {
          const int i = base + j * TOPK_THREADS + tid;
          if (i < n && (k[j] & pmask) == prefix) atomicAdd(&hist[(k[j] >> shift) & dmask], 1);
        }
      }
    }
    __syncthreads();
    // Thread t holds digits 1023 - 4t - j (j = 0..3): a scan from the top
    // gives the count of keys above each digit.
    constexpr int PER = TOPK_BINS / TOPK_THREADS;
    int c[PER], csum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      c[j] = hist[TOPK_BINS - 1 - PER * tid - j];
      csum += c[j];
    }
    int total;
    int above = block_exclusive_scan256(csum, scratch, &total);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (above < rank && rank <= above + c[j]) {
        s_digit = TOPK_BINS - 1 - PER * tid - j;
        s_rank = rank - above;
        s_count = c[j];
      }
      above += c[j];
    }
    __syncthreads();
    prefix |= (uint32_t)s_digit << shift;
    pmask |= dmask << shift;
    rank = s_rank;
    const bool done = s_count == rank;
    __syncthreads();
    if (done) break;
  }

  // The selection: keys whose selected digits exceed the prefix, and the
  // first `rank` keys (in position order) whose digits equal it.  Thread t
  // takes positions [t C, (t+1) C): it counts both kinds, two block scans
  // give its output slot and its share of the equal keys, and it writes its
  // chosen positions in order.
  const int C = (n + TOPK_THREADS - 1) / TOPK_THREADS;
  const int b0 = min(n, tid * C), b1 = min(n, b0 + C);
  int gt = 0, eq = 0;
  for (int i0 = b0; i0 < b1; i0 += TOPK_BATCH) {
    uint32_t k[TOPK_BATCH];
#pragma unroll
    for (int j = 0; j < TOPK_BATCH; ++j) k[j] = i0 + j < b1 ? key_at(i0 + j) & pmask : 0u;
#pragma unroll
    for (int j = 0; j < TOPK_BATCH; ++j) {
      gt += i0 + j < b1 && k[j] > prefix;
      eq += i0 + j < b1 && k[j] == prefix;
    }
  }
  int eq_total;
  const int eq_before = block_exclusive_scan256(eq, scratch, &eq_total);
  int left = min(eq, max(0, rank - eq_before));   // equal keys this thread takes
  int sel_total;
  int pos = block_exclusive_scan256(gt + left, scratch, &sel_total);
  for (int i0 = b0; i0 < b1; i0 += TOPK_BATCH) {
    uint32_t k[TOPK_BATCH];
#pragma unroll
    for (int j = 0; j < TOPK_BATCH; ++j) k[j] = i0 + j < b1 ? key_at(i0 + j) & pmask : 0u;
#pragma unroll
    for (int j = 0; j < TOPK_BATCH; ++j) {
      if (i0 + j >= b1) continue;
      bool take = k[j] > prefix;
      if (k[j] == prefix && left > 0) {
        take = true;
        --left;
      }
      if (take && pos < K) out[pos++] = (int32_t)(lo + i0 + j);   // pos < K always: the counts sum to K
    }
  }
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  if (a.s_q == 0) return hipSuccess;
  if (a.s_kv <= TOPK_SMALL_CACHE)
    topk_kernel<TOPK_SMALL_CACHE><<<dim3((unsigned)a.s_q), dim3(TOPK_THREADS), 0, stream>>>(a);
  else
    topk_kernel<TOPK_LARGE_CACHE><<<dim3((unsigned)a.s_q), dim3(TOPK_THREADS), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace smla
