// Nonfinite diagnostics (gfx950): count the NaN / Inf entries of a bf16 or
// fp32 buffer, and replace only those entries with a reference's values (or
// with zero).  These are the device-side pieces of the finite-check workflow
// in slime issue #2201, "GLM-5.2 SparseMLA TileLang backward returns NaN
// gradients from finite inputs" (Workarounds tested: check the kernel's dq /
// dkv for NaN / Inf, and when some are found, take the reference's values at
// those entries only; a variant that writes zeros there was the diagnostic
// confinement patch).  An entry is nonfinite when its exponent bits are all
// ones (IEEE-754 binary32 and bfloat16 alike).
//
// Both kernels stream the buffer once with 16-byte loads (a few in flight per
// thread); the replacement reads the reference only for 16-byte groups that
// hold a nonfinite entry and writes only those groups back.  The count is
// added into a caller's device uint64 with one atomic per wave that found any.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

constexpr int DIAG_THREADS = 256;
constexpr int DIAG_UNROLL = 4;   // 16-byte groups in flight per thread

// Nonfinite flags of the elements of one 16-byte group, as a bit mask
// (bit e for element e): 8 bf16 or 4 fp32.
template <int ES>
__device__ __forceinline__ unsigned nonfinite_mask(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  unsigned m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (ES == 2) {
      m |= ((w[j] & 0x7F80u) == 0x7F80u ? 1u : 0u) << (2 * j);
      m |= ((w[j] & 0x7F800000u) == 0x7F800000u ? 1u : 0u) << (2 * j + 1);
    } else {
      m |= ((w[j] & 0x7F800000u) == 0x7F800000u ? 1u : 0u) << j;
    }
  }
  return m;
}

template <int ES>
__device__ __forceinline__ bool nonfinite_scalar(const void* p, int64_t i) {
  if (ES == 2) return (reinterpret_cast<const uint16_t*>(p)[i] & 0x7F80u) == 0x7F80u;
  return (reinterpret_cast<const uint32_t*>(p)[i] & 0x7F800000u) == 0x7F800000u;
}

__device__ __forceinline__ void add_count(unsigned long long c, unsigned long long* count) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if ((threadIdx.x & 63) == 0 && c) atomicAdd(count, c);
}

// x: n elements of ES bytes, 16-byte aligned.  Groups of 16 bytes are
// handed out grid-stride, DIAG_UNROLL per thread per round; the last
// n mod (16 / ES) elements are checked one by one by the first workgroup.
template <int ES>
__global__ __launch_bounds__(DIAG_THREADS) void nonfinite_count_kernel(const void* x, int64_t n,
                                                                       unsigned long long* count) {
  constexpr int EPG = 16 / ES;
  const int64_t ng = n / EPG;
  const uint4* xg = reinterpret_cast<const uint4*>(x);
  const int64_t stride = (int64_t)gridDim.x * DIAG_THREADS;
  unsigned long long c = 0;
  for (int64_t g0 = (int64_t)blockIdx.x * DIAG_THREADS + threadIdx.x; g0 < ng; g0 += DIAG_UNROLL * stride) {
    uint4 v[DIAG_UNROLL];
#pragma unroll
    for (int u = 0; u < DIAG_UNROLL; ++u) {
      const int64_t g = g0 + u * stride;
      v[u] = g < ng ? xg[g] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < DIAG_UNROLL; ++u) c += __popc(nonfinite_mask<ES>(v[u]));
  }
  if (blockIdx.x == 0)
    for (int64_t i = ng * EPG + threadIdx.x; i < n; i += DIAG_THREADS) c += nonfinite_scalar<ES>(x, i);
  add_count(c, count);
}

// Where x is nonfinite, x := ref (ref null: +0); count the replaced entries.
template <int ES>
__global__ __launch_bounds__(DIAG_THREADS) void nonfinite_replace_kernel(void* x, const void* ref, int64_t n,
                                                                         unsigned long long* count) {
  constexpr int EPG = 16 / ES;
  const int64_t ng = n / EPG;
  uint4* xg = reinterpret_cast<uint4*>(x);
  const uint4* rg = reinterpret_cast<const uint4*>(ref);
  const int64_t stride = (int64_t)gridDim.x * DIAG_THREADS;
  unsigned long long c = 0;
  for (int64_t g0 = (int64_t)blockIdx.x * DIAG_THREADS + threadIdx.x; g0 < ng; g0 += DIAG_UNROLL * stride) {
    uint4 v[DIAG_UNROLL];
#pragma unroll
    for (int u = 0; u < DIAG_UNROLL; ++u) {
      const int64_t g = g0 + u * stride;
      v[u] = g < ng ? xg[g] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < DIAG_UNROLL; ++u) {
      const int64_t g = g0 + u * stride;
      const unsigned m = nonfinite_mask<ES>(v[u]);
      if (g < ng && m) {
        const uint4 r = rg ? rg[g] : make_uint4(0u, 0u, 0u, 0u);
        uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ES == 2) {
            const uint32_t keep = ((m >> (2 * j)) & 1u ? 0u : 0x0000FFFFu) |
                                  ((m >> (2 * j + 1)) & 1u ? 0u : 0xFFFF0000u);
            w[j] = (w[j] & keep) | (rw[j] & ~keep);
          } else {
            w[j] = (m >> j) & 1u ? rw[j] : w[j];
          }
        }
        xg[g] = make_uint4(w[0], w[1], w[2], w[3]);
        c += __popc(m);
      }
    }
  }
  if (blockIdx.x == 0)
    for (int64_t i = ng * EPG + threadIdx.x; i < n; i += DIAG_THREADS) {
      if (!nonfinite_scalar<ES>(x, i)) continue;
      if (ES == 2)
        reinterpret_cast<uint16_t*>(x)[i] = ref ? reinterpret_cast<const uint16_t*>(ref)[i] : (uint16_t)0;
      else
        reinterpret_cast<uint32_t*>(x)[i] = ref ? reinterpret_cast<const uint32_t*>(ref)[i] : 0u;
      ++c;
    }
  add_count(c, count);
}

unsigned diag_grid(int64_t n, int es) {
  const int64_t groups = n * es / 16;
  const int64_t per_wg = (int64_t)DIAG_THREADS * DIAG_UNROLL;
  const int64_t wgs = (groups + per_wg - 1) / per_wg;
  return (unsigned)(wgs < 1 ? 1 : wgs > 2048 ? 2048 : wgs);
}

}  // namespace

hipError_t launch_nonfinite(void* x, const void* ref, int64_t n, int es, bool replace,
                            unsigned long long* count, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const dim3 grid(diag_grid(n, es)), block(DIAG_THREADS);
  if (replace) {
    if (es == 2) nonfinite_replace_kernel<2><<<grid, block, 0, stream>>>(x, ref, n, count);
    else nonfinite_replace_kernel<4><<<grid, block, 0, stream>>>(x, ref, n, count);
  } else {
    if (es == 2) nonfinite_count_kernel<2><<<grid, block, 0, stream>>>(x, n, count);
    else nonfinite_count_kernel<4><<<grid, block, 0, stream>>>(x, n, count);
  }
  return hipGetLastError();
}

}  // namespace smla
