// Index planning for sparse-MLA attention (gfx950).
//
// The top-k index rows are turned into two structures that let the compute
// kernels share gathered KV tiles between query tokens:
//
//  * query-major: for every query group of T = 64/H consecutive tokens, the
//    union of the KV rows its tokens select (ascending), each with a T-bit
//    mask of the tokens that select it.  A token that lists a row more than
//    once gets one extra entry per repeat (mask = that token only), appended
//    after the union, so every slot stays its own softmax term.
//  * kv-major: for every (64-row KV block, query group) pair where some token
//    of the group selects a row of the block, T records -- one 64-bit row
//    mask per token of the group -- stored per group and indexed by a
//    [block, group] table.  Walking the table in group order visits the
//    records sorted by (block, token): a deterministic order for the per-row
//    dKV reduction.
//
// A slot is valid iff 0 <= index < s_kv; -1 (padding) and any other value are
// skipped, so padding never reaches memory (miles PR #2079 digest, "fix GLM-5
// sparse-MLA kernel -1 index OOB and NaN gradients", 实现拆解 item 1: -1 used
// to address the element before the KV buffer).
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

constexpr int WIN_BITS = 16384;            // kv rows per bitmap window
constexpr int WIN_WORDS = WIN_BITS / 32;   // 512: two per thread
constexpr int WIN_BLOCKS = WIN_BITS / 64;  // 256: one per thread
constexpr int XFLAG_WORDS = 4096;          // T * topk <= 8 * 16384 slots
constexpr int PLAN_LOADS = 64;             // index loads in flight per thread (a group's slots in one round at T K = 16384)

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

template <int T, bool KVG>
__global__ __launch_bounds__(256) void plan_kernel(PlanArgs a) {
  __shared__ unsigned bm[T][WIN_WORDS];      // per-token row bitmaps of one window
  __shared__ unsigned xflag[XFLAG_WORDS];    // slots that repeat an earlier slot's row
  __shared__ int scratch[8];
  __shared__ int s_lo, s_hi;
  __shared__ int64_t s_ixoff[T];             // group-major rows: each token's index row
  __shared__ int s_kg[T];                    // kv groups: each token's kv group
  __shared__ int s_rep;                      // window check: slots minus distinct rows

  // Index loads in flight per thread: with kv groups each load's address is
  // formed per slot, so fewer loads per thread keep three waves per SIMD.
  constexpr int NL = KVG ? PLAN_LOADS / 2 : PLAN_LOADS;
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int64_t t0 = g * T;
  const int nt = (int)min<int64_t>(T, a.s_q - t0);
  const int K = a.topk;
  const int nslots = nt * K;
  const int32_t* ix = a.idx + (t0 >> a.idx_shift) * K;   // shift > 0 only with T = 1
  const bool gmaj = KVG && a.gmajor_s > 0;
  // Group-local token of slot s (token t holds slots t K .. t K + K - 1;
  // K is uniform, so the division's reciprocal is formed once).
  auto tok_of = [&](int s) __attribute__((always_inline)) { return T == 1 ? 0 : s / K; };
  // kv group of token t (KVG): group-major rows are pairs g S + s (S =
  // gmajor_s), so from the first pair's (g0, r0) a token moves to the next
  // group each time r0 + t passes a multiple of S; token-major rows (T = 1)
  // have one group.  No divisions or LDS reads per slot.
  // (Pairs and tokens are below 2^31.)
  const int gS = gmaj ? (int)a.gmajor_s : 1;
  const int g0 = gmaj ? (int)(t0 / gS) : (KVG ? (int)((t0 >> a.idx_shift) % a.kv_groups) : 0);
  const int r0 = gmaj ? (int)(t0 - (int64_t)g0 * gS) : 0;
  auto group_of = [&](int t, int& r) __attribute__((always_inline)) {   // r: the pair's token
    int kg = g0;
    r = r0 + t;
    if (gmaj)
      while (r >= gS) {
        r -= gS;
        ++kg;
      }
    return kg;
  };
  // Index value of slot s of the group: the T index rows are consecutive,
  // except for group-major rows (kv groups), which read each token's row of
  // the caller's token-major indices (slot s - t K of row r kv_groups + kg).
  auto ixv = [&](int s) __attribute__((always_inline)) {
    if constexpr (KVG) {
      if (gmaj) {
        const int t = tok_of(s);
        int r;
        const int kg = group_of(t, r);
        return a.idx[((int64_t)r * a.kv_groups + kg - t) * K + s];
      }
    }
    return ix[s];
  };
  const int nxw = (nslots + 31) >> 5;
  const int skv = (int)a.s_kv;        // flat kv rows
  const int sidx = (int)a.s_kv_idx;   // valid index values: [0, sidx)
  const int kvg = a.kv_groups;
  // Rows of a valid value v of slot s (token t).  The bitmaps, the union order and
  // the kv blocks use block rows, in which each kv group's rows form one
  // range (row v of group g is g sidx + v), so a 64-row kv block holds one
  // group's rows; the union list stores the flat row of the [sidx, kvg,
  // 576] kv, v kvg + g, where the gathers read it.
  auto brow = [&](int v, int s) __attribute__((always_inline)) {   // v of slot s
    if constexpr (KVG) {
      int r;
      return group_of(tok_of(s), r) * sidx + v;
    } else {
      return v;
    }
  };
  auto frow = [&](int v, int t) __attribute__((always_inline)) {
    if constexpr (KVG) return v * kvg + s_kg[t];
    else return v;
  };

  if (tid == 0) {
    s_lo = 0x7fffffff;
    s_hi = -1;
  }
  if (gmaj && tid < nt) s_ixoff[tid] = caller_token(t0 + tid, a.gmajor_s, a.kv_groups) * K;
  if (KVG && tid < nt) {   // the (group, token) pair's kv group
    const int64_t r = t0 + tid;
    s_kg[tid] = gmaj ? (int)(r / a.gmajor_s) : (int)((r >> a.idx_shift) % kvg);
  }
  for (int w = tid; w < nxw; w += 256) xflag[w] = 0u;
  __syncthreads();

  // Span of the valid rows this group selects (one window covers every
  // valid row when s_kv <= WIN_BITS; the scan is skipped then, and with kv
  // groups the span is the block rows of the tokens' groups).
  int lo = 0, hi = skv - 1;
  if (KVG && skv <= WIN_BITS) {
    int gl = s_kg[0], gh = s_kg[0];
    for (int t = 1; t < nt; ++t) {
      gl = min(gl, s_kg[t]);
      gh = max(gh, s_kg[t]);
    }
    lo = gl * sidx;
    hi = min(skv, (gh + 1) * sidx) - 1;
  }
  if (skv > WIN_BITS) {
    lo = 0x7fffffff;
    hi = -1;
    for (int s0 = tid; s0 < nslots; s0 += 256 * NL) {   // NL loads in flight per thread
      int v[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) v[j] = s0 + 256 * j < nslots ? ixv(s0 + 256 * j) : -1;
#pragma unroll
      for (int j = 0; j < NL; ++j)
        if (v[j] >= 0 && v[j] < sidx) {
          const int m = brow(v[j], s0 + 256 * j);
          lo = min(lo, m);
          hi = max(hi, m);
        }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if ((tid & 63) == 0) {
      atomicMin(&s_lo, lo);
      atomicMax(&s_hi, hi);
    }
    __syncthreads();
    lo = s_lo;
    hi = s_hi;
  }

  int32_t* qrow = a.qrow + g * a.qcap;
  uint8_t* qmask = a.qmask + g * a.qcap;
  int qbase = 0, rbase = 0;
  if (a.ktab) {
    // This group's column of the [block, group] table is written whole (no
    // clearing pass before the planner): blocks the windows below do not
    // cover get (0, 0) here, the windows write every block they cover.
    const int64_t cover_lo = hi >= 0 ? (int64_t)(lo & ~63) >> 6 : a.NB;
    const int64_t cover_hi =
        hi >= 0 ? ((int64_t)(lo & ~63) + ((int64_t)(hi - (lo & ~63)) / WIN_BITS + 1) * WIN_BITS) >> 6 : a.NB;
    for (int64_t b = tid; b < a.NB; b += 256)
      if (b < cover_lo || b >= cover_hi) a.ktab[b * a.G + g] = make_int2(0, 0);
  }
  // Windows start on a 64-row block boundary so kv blocks never straddle two.
  for (int w0 = (hi >= 0 ? (lo & ~63) : 1); w0 <= hi; w0 += WIN_BITS) {
    const int qbase0 = qbase;   // union entries before this window
    // Bitmap pass: NL index loads in flight per thread before their
    // bitmap updates.  The first pass sets the bits with no-return atomics
    // and counts the window's valid slots; a token that lists a row twice
    // leaves fewer bits than slots, and only then does a second pass redo
    // the window with returning atomics that flag every slot whose row was
    // already set (the repeats).
    auto bitmap_pass = [&](auto RTN) __attribute__((always_inline)) {
      constexpr bool rtn = decltype(RTN)::value;
      for (int i = tid; i < T * WIN_WORDS; i += 256) (&bm[0][0])[i] = 0u;
      if (tid == 0) s_rep = 0;
      __syncthreads();
      int cnt = 0;
      for (int s0 = tid; s0 < nslots; s0 += 256 * NL) {
        int v[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int s = s0 + 256 * j;
          v[j] = s < nslots ? ixv(s) : -1;
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int s = s0 + 256 * j;
          const int m = v[j] >= 0 && v[j] < sidx ? brow(v[j], s) : -1;
          if (m >= w0 && m < w0 + WIN_BITS) {
            const int t = tok_of(s);
            const int bit = m - w0;
            const unsigned mb = 1u << (bit & 31);
            if constexpr (rtn) {
              const unsigned old = atomicOr(&bm[t][bit >> 5], mb);
              if (old & mb) atomicOr(&xflag[s >> 5], 1u << (s & 31));
            } else {
              __hip_atomic_fetch_or(&bm[t][bit >> 5], mb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
              ++cnt;
            }
          }
        }
      }
      __syncthreads();
      return cnt;
    };
    {
      int cnt = bitmap_pass(Int<0>{});
      for (int i = tid; i < T * WIN_WORDS; i += 256) cnt -= __popc((&bm[0][0])[i]);
      cnt = wave_inclusive_scan(cnt);   // lane 63: the wave's total
      if ((tid & 63) == 63 && cnt != 0) atomicAdd(&s_rep, cnt);
      __syncthreads();
      if (s_rep != 0) {   // (uniform) some token lists a row twice in this window
        __syncthreads();   // every thread has read s_rep before the clear
        bitmap_pass(Int<1>{});
      }
    }

    // Union entries, ascending row order.  Thread tid owns bytes tid + 256k
    // (k = 0..7) of the window's bitmap, so a contiguous union spreads over
    // many threads; each round k is one block-wide scan in row order.  Rounds
    // past the span's last row (2048 rows each) hold no set bit and are
    // skipped.
    const int rounds = min(WIN_WORDS * 4 / 256, ((hi - w0) >> 11) + 1);
#pragma unroll 1
    for (int k = 0; k < rounds; ++k) {
      const int byte = tid + 256 * k;
      const int w = byte >> 2, sh = 8 * (byte & 3);
      unsigned tb[T], u = 0;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        tb[t] = (bm[t][w] >> sh) & 0xFFu;
        u |= tb[t];
      }
      int total;
      int pos = qbase + block_exclusive_scan256(__popc(u), scratch, &total);
      const int row0 = w0 + 8 * byte;
      while (u) {
        const int b = __ffs(u) - 1;
        u &= u - 1;
        unsigned mask = 0;
#pragma unroll
        for (int t = 0; t < T; ++t) mask |= ((tb[t] >> b) & 1u) << t;
        if constexpr (KVG) {   // flat row of the block row (a selecting token's group)
          const int gk = s_kg[__ffs(mask) - 1];
          qrow[pos] = (row0 + b - gk * sidx) * kvg + gk;
        } else {
          qrow[pos] = row0 + b;
        }
        qmask[pos] = (uint8_t)mask;
        ++pos;
      }
      qbase += total;
    }

    if (a.ktab) {
      // kv-block records: thread tid owns block (w0 >> 6) + tid.  A block any
      // token of the group selects gets T records, one 64-bit row mask per
      // token of the group (zero for tokens that select none of its rows).
      unsigned long long mk[T], orm = 0ull;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        mk[t] = (unsigned long long)bm[t][2 * tid] |
                ((unsigned long long)bm[t][2 * tid + 1] << 32);
        orm |= mk[t];
      }
      const int any = orm != 0ull;
      int rtotal, etotal;
      const int rpos = rbase + block_exclusive_scan256(any ? T : 0, scratch, &rtotal);
      // The block's union entries follow those of the window's earlier
      // blocks (the union is in row order): its first entry index.
      const int epos = qbase0 + block_exclusive_scan256(__popcll(orm), scratch, &etotal);
      const int64_t b = (int64_t)(w0 >> 6) + tid;   // a set bit is a row < s_kv, so any => b < NB
      if (b < a.NB) a.ktab[b * a.G + g] = any ? make_int2(rpos, T) : make_int2(0, 0);
      if (any) {
        const int64_t r = g * a.rcap + rpos;
#pragma unroll
        for (int t = 0; t < T; ++t) a.krmask[r + t] = mk[t];
        a.kbase[b * a.G + g] = epos;
        a.korm[b * a.G + g] = orm;
      }
      rbase += rtotal;
    }
    __syncthreads();  // bm is cleared by the next window
  }

  // Which occurrence of a repeated (token, row) pair the atomics above flag
  // depends on the order they land in.  Make it canonical -- every occurrence
  // but the first in slot order -- so the extra entries, and the summation
  // order they imply, depend on the indices alone.  Only the first occurrence
  // can be flagged wrongly; the wave that owns its flag word hands the flag to
  // the one later occurrence the atomics left unflagged.  Flags of one pair
  // change only in that wave, and a flag set meanwhile in a word another wave
  // has already read belongs to a non-first occurrence, which needs no change.
  {
    int anyx = 0;
    for (int w = tid; w < nxw; w += 256) anyx |= (xflag[w] != 0u);
    if (__syncthreads_or(anyx)) {
      const int wv = tid >> 6, lane = tid & 63;
      // A wave reads 64 flag words at once and visits the nonzero ones.
      for (int w0 = 64 * wv; w0 < nxw; w0 += 256) {
        const unsigned fw = w0 + lane < nxw ? xflag[w0 + lane] : 0u;
        unsigned long long nz = __ballot(fw != 0u);
        while (nz) {
          const int wl = __ffsll((long long)nz) - 1;
          nz &= nz - 1;
          const int w = w0 + wl;
          unsigned f = (unsigned)__builtin_amdgcn_readlane((int)fw, wl);
          while (f) {
            const int b = __ffs(f) - 1;
            f &= f - 1;
            const int s = 32 * w + b;
            const int t = s / K, k = s - t * K;
            const int32_t* row = gmaj ? a.idx + s_ixoff[t] : ix + (int64_t)t * K;
            const int v = __builtin_amdgcn_readfirstlane(row[k]);
            // The row is scanned 512 slots per round (eight loads in flight per
            // lane), not 64: each round is one memory round trip.
            bool earlier = false;
            for (int i0 = 0; i0 < k && !earlier; i0 += 512) {
              int rv[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const int i = i0 + lane + 64 * j;
                rv[j] = i < k ? row[i] : ~v;
              }
              bool hit = false;
#pragma unroll
              for (int j = 0; j < 8; ++j) hit |= rv[j] == v;
              earlier = __ballot(hit) != 0ull;
            }
            if (earlier) continue;
            int later = -1;
            for (int i0 = k + 1; i0 < K && later < 0; i0 += 512) {
              int rv[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                const int i = i0 + lane + 64 * j;
                rv[j] = i < K ? row[i] : ~v;
              }
#pragma unroll
              for (int j = 0; j < 8; ++j) {   // in slot order: the first unflagged match
                const int si = min(t * K + i0 + lane + 64 * j, nslots - 1);   // (past the row: no hit)
                const bool hit = rv[j] == v && !((xflag[si >> 5] >> (si & 31)) & 1u);
                const unsigned long long bal = __ballot(hit);
                if (bal && later < 0) later = i0 + 64 * j + __ffsll((long long)bal) - 1;
              }
            }
            if (lane == 0 && later >= 0) {
              const int sx = t * K + later;
              atomicOr(&xflag[sx >> 5], 1u << (sx & 31));
              atomicAnd(&xflag[w], ~(1u << b));
            }
          }
        }
      }
      __syncthreads();
    }
  }

  // Repeated slots, in slot order: one extra union entry each.
  const int wpt = (nxw + 255) / 256;
  const int wb = min(nxw, tid * wpt), we = min(nxw, wb + wpt);
  int c = 0;
  for (int w = wb; w < we; ++w) c += __popc(xflag[w]);
  int xtot;
  int pos = qbase + block_exclusive_scan256(c, scratch, &xtot);
  for (int w = wb; w < we; ++w) {
    unsigned f = xflag[w];
    while (f) {
      const int b = __ffs(f) - 1;
      f &= f - 1;
      const int s = 32 * w + b;
      const int t = s / K;
      qrow[pos] = frow(ixv(s), t);
      qmask[pos] = (uint8_t)(1u << t);
      ++pos;
    }
  }
  if (tid == 0) {
    a.qcount[g] = qbase + xtot;
    a.xcount[g] = xtot;
  }
  // Zero the masks of the last tile's unused entries (up to the next multiple
  // of 64; qcap is a multiple of 64): the compute kernels copy masks in words.
  const int n_all = qbase + xtot;
  if (tid < 64 && n_all + tid < ((n_all + 63) & ~63)) qmask[n_all + tid] = 0;
}

// Work order of the query groups (largest union first) and the total count
// of extra entries (repeated slots) over all groups.
__global__ __launch_bounds__(256) void order_groups_kernel(const int* qcount, const int* xcount, int64_t G,
                                                           int* order, int* xtotal) {
  __shared__ int s_x[4];
  int x = 0;
  for (int64_t g = threadIdx.x; g < G; g += 256) x += xcount[g];
  x = wave_inclusive_scan(x);   // lane 63: the wave's total
  if ((threadIdx.x & 63) == 63) s_x[threadIdx.x >> 6] = x;
  order_by_cost(G, [&](int64_t g) { return (qcount[g] + 31) >> 5; }, order);   // syncs the block
  if (threadIdx.x == 0) *xtotal = s_x[0] + s_x[1] + s_x[2] + s_x[3];
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

__global__ void validate_kernel(const int32_t* idx, int64_t n, int64_t s_kv,
                                unsigned long long* n_bad) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  unsigned long long c = 0;
  for (; i < n; i += stride) {
    const int v = idx[i];
    c += (v != -1 && (v < 0 || v >= s_kv)) ? 1ull : 0ull;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if ((threadIdx.x & 63) == 0 && c) atomicAdd(n_bad, c);
}

}  // namespace

hipError_t launch_order_groups(const int* qcount, const int* xcount, int64_t G, int* order, int* xtotal,
                               hipStream_t stream) {
  if (G == 0) return hipSuccess;
  order_groups_kernel<<<1, 256, 0, stream>>>(qcount, xcount, G, order, xtotal);
  return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs& a, int heads, hipStream_t stream) {
  if (a.G == 0) return hipSuccess;
  dim3 grid((unsigned)a.G), block(256);
  const bool kvg = a.kv_groups > 1;
  switch (heads) {
    case 8: kvg ? plan_kernel<8, true><<<grid, block, 0, stream>>>(a) : plan_kernel<8, false><<<grid, block, 0, stream>>>(a); break;
    case 16: kvg ? plan_kernel<4, true><<<grid, block, 0, stream>>>(a) : plan_kernel<4, false><<<grid, block, 0, stream>>>(a); break;
    case 32: kvg ? plan_kernel<2, true><<<grid, block, 0, stream>>>(a) : plan_kernel<2, false><<<grid, block, 0, stream>>>(a); break;
    case 64: kvg ? plan_kernel<1, true><<<grid, block, 0, stream>>>(a) : plan_kernel<1, false><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename E>
__global__ __launch_bounds__(256) void permute_pairs_kernel(const E* src, E* dst, int64_t S, int G,
                                                            int64_t per, bool to_gmajor) {
  const int64_t n = S * G * per;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t u = i / per, c = i - u * per;   // group-major block u = g S + s
    const int64_t g = u / S, s = u - g * S;
    const int64_t t = s * G + g;                  // token-major block
    if (to_gmajor)
      dst[u * per + c] = src[t * per + c];
    else
      dst[t * per + c] = src[u * per + c];
  }
}

hipError_t launch_permute_pairs(const void* src, void* dst, int64_t S, int G, int64_t block_bytes,
                                bool to_gmajor, hipStream_t stream) {
  if (S == 0) return hipSuccess;
  if (block_bytes % 16 == 0) {
    const int64_t per = block_bytes / 16, n = S * G * per;
    const int64_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
    permute_pairs_kernel<uint4_t><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
        static_cast<const uint4_t*>(src), static_cast<uint4_t*>(dst), S, G, per, to_gmajor);
  } else {
    const int64_t per = block_bytes / 4, n = S * G * per;
    const int64_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
    permute_pairs_kernel<uint32_t><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
        static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), S, G, per, to_gmajor);
  }
  return hipGetLastError();
}

hipError_t launch_fill_u32(void* ptr, size_t n_words, uint32_t value, hipStream_t stream) {
  if (n_words == 0) return hipSuccess;
  size_t blocks = (n_words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_u32_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>((uint32_t*)ptr, n_words, value);
  return hipGetLastError();
}

hipError_t launch_validate(const int32_t* idx, int64_t n, int64_t s_kv,
                           unsigned long long* n_bad, hipStream_t stream) {
  hipError_t e = launch_fill_u32(n_bad, 2, 0u, stream);
  if (e != hipSuccess || n == 0) return e;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  validate_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(idx, n, s_kv, n_bad);
  return hipGetLastError();
}

}  // namespace smla
