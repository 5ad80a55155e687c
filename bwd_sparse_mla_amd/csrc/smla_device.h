// Device-side building blocks shared by the sparse-MLA kernels (gfx950 / CDNA4).
//
// Matrix-core fragments follow the v_mfma_f32_16x16x32_bf16 lane layout
// (64 lanes; l = lane id, g = l >> 4, r = l & 15):
//   A [16 x 32]:  lane holds A[r][8g .. 8g+7]          (8 bf16, one 16-byte load)
//   B [32 x 16]:  lane holds B[8g .. 8g+7][r]
//   C [16 x 16]:  lane holds C[4g .. 4g+3][r]           (4 fp32)
// The transposing LDS read ds_read_b64_tr_b16 works on groups of 16 lanes:
// lane i of a group receives, as element j (j = 0..3), the 16-bit element
// (i & 3) of the 8 bytes addressed by lane (i >> 2) + 4j of the same group.
// So if lane i of a group addresses row k0 + (i >> 2) at columns
// n0 + 4(i & 3) .. +3, lane i receives rows k0 .. k0+3 of column n0 + i: a
// B fragment whose reduction index runs along stored rows, which is how V, K
// and Q/dO are consumed when the contraction runs over kv or query rows.
//
// Gathered tiles (kv rows, query rows) live in LDS row-major with swizzled
// 16-byte chunks.  A tile of R rows keeps the first 64 chunks of row r
// (columns 0..511) at r*1024 + 16 (c ^ swz_lo(r)) and, for 576-column rows,
// the 8 tail chunks (columns 512..575) at R*1024 + r*128 + 16 ((c-64) ^
// swz_hi(r)).  One direct global->LDS copy moves the first 1 KB of one row
// (a coalesced 1 KB read from a wave-uniform row address) or the tails of 8
// rows.  swz_lo(r) = r mod 16 and swz_hi(r) = (r / 2) mod 8.  The LDS serves a
// 16-byte read at full rate (about 220 B/clk per CU measured with 8 waves,
// against about 136 for other conflict-free-looking patterns) when every
// quad of lanes 4i .. 4i+3 lands in one aligned 64-byte bank group and the
// 16 lanes of a fragment read cover all 64 banks: a fragment read (16
// consecutive rows, one chunk) meets both with these XOR swizzles.
// Transposing 8-byte reads run at about 128 B/clk on any of the layouts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) short short8_t;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((ext_vector_type(4))) float float4_t;
typedef __attribute__((ext_vector_type(4))) unsigned uint4_t;
typedef short4_t __attribute__((address_space(3)))* lds_s4_ptr;
typedef void __attribute__((address_space(3)))* lds_void_ptr;

constexpr int D_V = 512;        // value (latent) width
constexpr int D_T = 64;         // rope tail width
constexpr int D_K = D_V + D_T;  // key width, 576
constexpr int ROW_CHUNKS = D_K / 8;          // 72 chunks of 16 bytes per kv/q row
constexpr int DO_CHUNKS = D_V / 8;           // 64 chunks per dout row
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float SUMEXP_FLOOR = 1e-30f;
// Running-max start: finite, so exp2(m_old - m_new) never sees inf - inf.
constexpr float M_INIT = -1e30f;
// Online softmax: the reference max of a row moves only when a new score
// exceeds it by more than this (log2 units); probabilities stay <= 2^8.
constexpr float RESCALE_SLACK = 8.f;

__device__ __forceinline__ float4_t mfma_bf16(short8_t a, short8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ unsigned short f2bf(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);
}
__device__ __forceinline__ unsigned pack_bf2(float lo, float hi) {
  return (unsigned)f2bf(lo) | ((unsigned)f2bf(hi) << 16);
}
__device__ __forceinline__ float bf2f(unsigned short b) {
  return __builtin_bit_cast(float, (unsigned)b << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 16-byte loads/stores.
__device__ __forceinline__ short8_t ld16_global(const void* p) {
  return *reinterpret_cast<const short8_t*>(p);
}
__device__ __forceinline__ short8_t ld16_lds(const void* p) {
  return *reinterpret_cast<const short8_t*>(p);
}

// Transposing LDS read of 8 bytes (see the header comment).
__device__ __forceinline__ short4_t ld_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_ptr)(lds_addr));
}

__device__ __forceinline__ int swz_lo(int r) { return r & 15; }
__device__ __forceinline__ int swz_hi(int r) { return (r >> 1) & 7; }

// Byte offset of chunk `chunk` (0..71) of row `row` in a swizzled tile of R rows.
template <int R>
__device__ __forceinline__ int rs_off(int row, int chunk) {
  return chunk < 64 ? row * 1024 + 16 * (chunk ^ swz_lo(row))
                    : R * 1024 + row * 128 + 16 * ((chunk - 64) ^ swz_hi(row));
}

// B fragment [32 x 16] with B[k][n] = tile[n0 + n][k0 + k] (the tile's rows
// are the fragment's columns): lane (g, r) reads chunk k0/8 + g of row n0 + r.
// (lane >> 4) & 3 rather than lane >> 4: kernels hide the lane id from the
// compiler on purpose, and the bound lets it resolve the main / tail choice
// of rs_off at compile time for a constant k0.
template <int R>
__device__ __forceinline__ short8_t ld_b_rs(const char* tile, int n0, int k0, int lane) {
  return ld16_lds(tile + rs_off<R>(n0 + (lane & 15), (k0 >> 3) + ((lane >> 4) & 3)));
}

// B fragment [32 x 16] with B[k][n] = tile[k0 + k][n0 + n] (reduction over
// the tile's rows; n0 a multiple of 16): two transposing reads give
// k = 8g .. 8g+3 and 8g+4 .. 8g+7 of lane column r.
template <int R>
__device__ __forceinline__ short8_t ld_bt_rs(const char* tile, int k0, int n0, int lane) {
  const int g = (lane >> 4) & 3, L = lane & 15;
  const int row = k0 + 8 * g + (L >> 2);
  const int chunk = (n0 >> 3) + ((L >> 1) & 1);
  const char* p = tile + (L & 1) * 8;
  short4_t lo = ld_tr16(p + rs_off<R>(row, chunk));
  short4_t hi = ld_tr16(p + rs_off<R>(row + 4, chunk));
  short8_t v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// ld_bt_rs for columns below 512 only (n0 + 16 <= 512): no tail addressing.
template <int R>
__device__ __forceinline__ short8_t ld_bt_rs_lo(const char* tile, int k0, int n0, int lane) {
  const int g = (lane >> 4) & 3, L = lane & 15;
  const int row = k0 + 8 * g + (L >> 2);
  const int chunk = (n0 >> 3) + ((L >> 1) & 1);
  const char* p = tile + (L & 1) * 8 + 16 * chunk;
  short4_t lo = ld_tr16(p + row * 1024 + 16 * ((chunk ^ swz_lo(row)) - chunk));
  short4_t hi = ld_tr16(p + (row + 4) * 1024 + 16 * ((chunk ^ swz_lo(row + 4)) - chunk));
  short8_t v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// Half h (0 or 1) of a pair of column blocks over columns n0 .. n0+31 (n0 a
// multiple of 32, n0 + 32 <= 512), rows k0 .. k0+31 as the reduction index:
// lane (g, L) holds rows k0 + 8g .. +7 of column n0 + 8 (L / 4) + 4h + L % 4.
// As the A operand of an MFMA (rows = these columns), output row 4g + i is
// column n0 + 8g + 4h + i, so a lane's outputs of the two halves are 8
// adjacent columns.
template <int R>
__device__ __forceinline__ short8_t ld_bt_rs_pair(const char* tile, int k0, int n0, int h, int lane) {
  const int g = (lane >> 4) & 3, L = lane & 15;
  const int row = k0 + 8 * g + (L >> 2);
  const int chunk = (n0 >> 3) + (L & 3);
  const char* p = tile + 8 * h + 16 * chunk;
  short4_t lo = ld_tr16(p + row * 1024 + 16 * ((chunk ^ swz_lo(row)) - chunk));
  short4_t hi = ld_tr16(p + (row + 4) * 1024 + 16 * ((chunk ^ swz_lo(row + 4)) - chunk));
  short8_t v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// ld_bt_rs for columns 512..575 only (n0 >= 512): tail addressing.
template <int R>
__device__ __forceinline__ short8_t ld_bt_rs_hi(const char* tile, int k0, int n0, int lane) {
  const int g = (lane >> 4) & 3, L = lane & 15;
  const int row = k0 + 8 * g + (L >> 2);
  const int ct = ((n0 - D_V) >> 3) + ((L >> 1) & 1);   // tail chunk, 0..7
  const char* p = tile + R * 1024 + (L & 1) * 8;
  short4_t lo = ld_tr16(p + row * 128 + 16 * (ct ^ swz_hi(row)));
  short4_t hi = ld_tr16(p + (row + 4) * 128 + 16 * (ct ^ swz_hi(row + 4)));
  short8_t v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return v;
}

// Asynchronous global -> LDS copies (global_load_lds): lane i writes
// lds_base + size*i; lds_base must be wave-uniform.  They are issued through
// inline asm on purpose: the compiler then inserts no vmcnt wait for them
// (its alias analysis cannot tell the next tile's buffer from the current
// one), so a prefetch overlaps the current tile.  Every consumer waits
// explicitly (wait_vmcnt0 + barrier) before it reads a copied buffer.  The
// "memory" clobber keeps the compiler from moving other memory accesses
// across a copy.  M0 carries the LDS address; nothing else in these kernels
// uses M0.
__device__ __forceinline__ uint32_t lds_offset(const void* lds_ptr) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)lds_ptr));
}
__device__ __forceinline__ void g2lds16(const void* gsrc, void* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gsrc), "s"(lds_offset(lds_base)) : "memory", "m0");
}
__device__ __forceinline__ void g2lds4(const void* gsrc, void* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gsrc), "s"(lds_offset(lds_base)) : "memory", "m0");
}
// 16-byte copy to LDS byte address lds_u32 (+ 16 per lane) from gsrc.
__device__ __forceinline__ void g2lds16_u(const void* gsrc, uint32_t lds_u32) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gsrc), "s"(lds_u32) : "memory", "m0");
}
// 16-byte copy from the wave-uniform base sbase plus a per-lane byte offset.
__device__ __forceinline__ void g2lds16_s(const void* sbase, uint32_t voff, uint32_t lds_u32) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_u32) : "memory", "m0");
}

// Compile-time loop: f(Int<0>{}), ..., f(Int<N-1>{}).
template <int I> struct Int { static constexpr int value = I; };
template <int I, int N, class F>
__device__ __forceinline__ void static_for_from(F& f) {
  if constexpr (I < N) {
    f(Int<I>{});
    static_for_from<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_from<0, N>(f); }

// s_waitcnt vmcnt(0) (other counters untouched).
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations
// (loads, stores and LDS copies alike; they complete in issue order) still
// outstanding.  The 6-bit count sits in bits 3:0 and 15:14; expcnt (6:4) and
// lgkmcnt (11:8) are left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Reductions across the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48)
// with the gfx950 row-swap instructions (VALU, no LDS round trip).
// v_permlane16_swap with both operands v gives (v of row 2k, v of row 2k+1)
// in rows 2k and 2k+1; v_permlane32_swap gives (v of lanes 0-31, v of lanes
// 32-63) in both halves.  Every lane combines the same pair in the same
// order, so all four lanes of a column get bitwise the same result.
__device__ __forceinline__ float max_rows(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_rows(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Exclusive prefix sum over a 256-thread block; returns this thread's
// exclusive prefix and writes the block total to *total.  `scratch` holds at
// least 8 ints of LDS.  Must be called by all threads.
// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), on
// the data-parallel-primitive lane moves: shifts by 1, 2, 4 and 8 within each
// row of 16 lanes (a lane shifted in from outside its row adds 0), then lane
// 15 added into row 1 and lane 47 into row 3, then lane 31 into rows 2 and 3.
// Six dependent adds instead of six LDS permutes.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
  return x;
}

__device__ __forceinline__ int block_exclusive_scan256(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int s = scratch[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Work order by decreasing cost (largest first), so the hardware's in-order
// workgroup dispatch approximates longest-processing-time scheduling: a
// counting sort on min(cost, ORDER_BUCKETS - 1).  Items of equal cost come in
// no particular order; each item writes its own outputs, so the order never
// changes a result.  One workgroup of 256 threads.
constexpr int ORDER_BUCKETS = 4096;
template <class Cost>
__device__ __forceinline__ void order_by_cost(int64_t n, Cost cost, int* order) {
  __shared__ int pos[ORDER_BUCKETS];
  __shared__ int scratch[8];
  const int tid = threadIdx.x;
  for (int b = tid; b < ORDER_BUCKETS; b += 256) pos[b] = 0;
  __syncthreads();
  for (int64_t i = tid; i < n; i += 256) atomicAdd(&pos[min(cost(i), ORDER_BUCKETS - 1)], 1);
  __syncthreads();
  // Thread t owns buckets 4095 - 16t down to 4080 - 16t (descending cost).
  int cnt[16], sum = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    cnt[k] = pos[ORDER_BUCKETS - 1 - 16 * tid - k];
    sum += cnt[k];
  }
  int total;
  int base = block_exclusive_scan256(sum, scratch, &total);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    pos[ORDER_BUCKETS - 1 - 16 * tid - k] = base;
    base += cnt[k];
  }
  __syncthreads();
  for (int64_t i = tid; i < n; i += 256) {
    const int slot = atomicAdd(&pos[min(cost(i), ORDER_BUCKETS - 1)], 1);
    order[slot] = (int)i;
  }
}

// Zeros that padding lanes of the LDS copies read from: a whole 576-column
// row, so a padding row of a tile holds true zeros and never reaches outside
// the inputs.
__device__ __attribute__((aligned(16))) const uint16_t g_zero_row[D_K] = {};
__device__ __forceinline__ const void* zero_row() { return g_zero_row; }

// Gathers rows into a swizzled tile of R rows whose rows have CH chunks (72:
// q / kv rows with their tail, 64: dout rows).  Wave wv copies the first 1 KB
// of rows R/4 * wv .. R/4 * wv + R/4 - 1 (one copy per row, from a
// wave-uniform row address) and the tails of rows 8j .. 8j+7 for j = wv,
// wv + 4, ... (one copy per 8 rows, per-lane row addresses).
//   gather_kv_rows: tile row r < count is kv row rows[r] (rows in LDS); rows
//     past count, and row indices outside [0, s_kv), read the zero row.
//   gather_seq_rows: tile row r < nvalid is row r of the contiguous rows at
//     `first`; rows past nvalid read the zero row.
template <int R, int CH>
__device__ __forceinline__ void gather_kv_rows(char* tile, const uint16_t* kv, int64_t s_kv,
                                               const int* rows, int count, int wv, int lane) {
  constexpr int PER = R / 4;
  const uint32_t base = lds_offset(tile);
  const int vrow = rows[PER * wv + (lane & (PER - 1))];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int r = PER * wv + i;
    const int row = __builtin_amdgcn_readlane(vrow, i);
    const bool ok = r < count && row >= 0 && row < s_kv;
    const uint16_t* src = ok ? kv + (int64_t)row * D_K : g_zero_row;
    g2lds16_s(src, 16u * (uint32_t)(lane ^ swz_lo(r)), base + 1024u * (uint32_t)r);
  }
  if constexpr (CH == ROW_CHUNKS) {
#pragma unroll
    for (int j = 0; j < R / 32; ++j) {
      const int jj = wv + 4 * j;
      const int r = 8 * jj + (lane >> 3);
      const int row = rows[r];
      const bool ok = r < count && row >= 0 && row < s_kv;
      const uint16_t* src = (ok ? kv + (int64_t)row * D_K : g_zero_row) + D_V + 8 * ((lane & 7) ^ swz_hi(r));
      g2lds16_u(src, base + (uint32_t)(R * 1024 + 1024 * jj));
    }
  }
}
template <int R, int CH>
__device__ __forceinline__ void gather_seq_rows(char* tile, const uint16_t* first, int nvalid,
                                                int wv, int lane) {
  constexpr int PER = R / 4;
  constexpr int W = CH * 8;  // elements per row
  const uint32_t base = lds_offset(tile);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int r = PER * wv + i;
    const uint16_t* src = r < nvalid ? first + (int64_t)r * W : g_zero_row;
    g2lds16_s(src, 16u * (uint32_t)(lane ^ swz_lo(r)), base + 1024u * (uint32_t)r);
  }
  if constexpr (CH == ROW_CHUNKS) {
#pragma unroll
    for (int j = 0; j < R / 32; ++j) {
      const int jj = wv + 4 * j;
      const int r = 8 * jj + (lane >> 3);
      const uint16_t* src = (r < nvalid ? first + (int64_t)r * W : g_zero_row) + D_V +
                            8 * ((lane & 7) ^ swz_hi(r));
      g2lds16_u(src, base + (uint32_t)(R * 1024 + 1024 * jj));
    }
  }
}

// gather_kv_rows for a workgroup of NW waves (NW >= 4, R / NW rows each):
// wave wv copies rows R/NW * wv .. +R/NW-1 (ROWS) and, for wv < R/8, the tails
// of rows 8 wv .. 8 wv + 7 (TAILS).
template <int R, int CH, int NW, bool ROWS = true, bool TAILS = true>
__device__ __forceinline__ void gather_kv_rows_nw(char* tile, const uint16_t* kv, int64_t s_kv,
                                                  const int* rows, int count, int wv, int lane) {
  constexpr int PER = R / NW;
  static_assert(PER >= 1 && (PER & (PER - 1)) == 0, "rows per wave must be a power of two");
  const uint32_t base = lds_offset(tile);
  if constexpr (ROWS) {
    const int vrow = rows[PER * wv + (lane & (PER - 1))];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int r = PER * wv + i;
      const int row = __builtin_amdgcn_readlane(vrow, i);
      const bool ok = r < count && (uint32_t)row < (uint32_t)s_kv;
      const uint16_t* src = (ok ? kv : g_zero_row) + (uint64_t)(uint32_t)(ok ? row : 0) * D_K;
      g2lds16_s(src, 16u * (uint32_t)(lane ^ swz_lo(r)), base + 1024u * (uint32_t)r);
    }
  }
  if constexpr (CH == ROW_CHUNKS && TAILS) {
    if (wv < R / 8) {
      const int r = 8 * wv + (lane >> 3);
      const int row = rows[r];
      const bool ok = r < count && (uint32_t)row < (uint32_t)s_kv;
      const uint16_t* src = (ok ? kv + (uint64_t)(uint32_t)row * D_K : g_zero_row) + D_V +
                            8 * ((lane & 7) ^ swz_hi(r));
      g2lds16_u(src, base + (uint32_t)(R * 1024 + 1024 * wv));
    }
  }
}

// The caller's token of a kernel token.  With several kv groups (G > 1) the
// kernels walk (group, token) pairs in group-major order, tok = g S + s, so
// that a query group holds one kv group's rows; the caller's rows are
// token-major, pair (s, g) at s G + g.  With one group the orders coincide.
// (Pairs number below 2^31: s_q < 2^24 tokens, G <= 64.)
__device__ __forceinline__ int64_t caller_token(int64_t tok, int64_t S, int G) {
  if (G <= 1) return tok;
  const uint32_t t = (uint32_t)tok, s = (uint32_t)S;
  const uint32_t g = t / s;
  return (int64_t)(t - g * s) * G + g;
}

// gather_seq_rows for a workgroup of NW waves over the kernel rows row0 ..
// row0 + nvalid - 1 of a tensor with H rows per token whose caller rows follow
// caller_token (S tokens per kv group, G groups): wave wv copies rows
// R/NW * wv .. +R/NW-1 and, for wv < R/8, the tails of rows 8 wv .. 8 wv + 7.
// (Each of those runs lies in one token: H is a multiple of R/NW and of 8.)
template <int R, int CH, int NW, int H>
__device__ __forceinline__ void gather_seq_rows_nw(char* tile, const uint16_t* src0, int64_t row0, int nvalid,
                                                   int64_t S, int G, int wv, int lane) {
  constexpr int PER = R / NW;
  constexpr int W = CH * 8;  // elements per row
  static_assert(H % PER == 0 && H % 8 == 0, "a wave's rows must lie in one token");
  const uint32_t base = lds_offset(tile);
  auto crow = [&](int64_t p) __attribute__((always_inline)) {   // caller row of kernel row p
    return caller_token(p / H, S, G) * H + p % H;
  };
  const uint16_t* first = src0 + crow(row0 + PER * wv) * W;   // the wave's rows PER wv ..
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int r = PER * wv + i;
    const bool ok = r < nvalid;
    const uint16_t* src = (ok ? first : g_zero_row) + (uint32_t)(ok ? i : 0) * (uint32_t)W;
    g2lds16_s(src, 16u * (uint32_t)(lane ^ swz_lo(r)), base + 1024u * (uint32_t)r);
  }
  if constexpr (CH == ROW_CHUNKS) {
    if (wv < R / 8) {
      const uint16_t* tfirst = src0 + crow(row0 + 8 * wv) * W;   // rows 8 wv .. 8 wv + 7
      const int r = 8 * wv + (lane >> 3);
      const bool ok = r < nvalid;
      const uint16_t* src = (ok ? tfirst + (uint32_t)(lane >> 3) * (uint32_t)W : g_zero_row) + D_V +
                            8 * ((lane & 7) ^ swz_hi(r));
      g2lds16_u(src, base + (uint32_t)(R * 1024 + 1024 * wv));
    }
  }
}

// Incremental form of the gathers: prepare once per tile, then issue copy J
// (a compile-time index) where it fits in the caller's instruction stream.
// For a kv gather of R rows, wave wv issues R/4 row copies (J < R/4) and
// R/32 tail copies (J = R/4 + j); a kv tile thus takes R/4 + R/32 copies per
// wave (18 for R = 64, 9 for R = 32).  The preparation forms every source
// address at once with vector instructions (lane i < R/4 holds the address of
// the wave's row i; rows past `count` and indices outside [0, s_kv) get the
// zero row), so a row copy is two lane reads, one XOR and the copy itself.
template <int R>
struct KvGather {
  uint64_t vaddr;           // lane i < R/4: source of tile row R/4 * wv + i
  uint32_t vswz;            // 16 (lane ^ swz_lo(R/4 * wv)): this lane's chunk in a row copy
  uint32_t lds_rows;        // LDS address of tile row R/4 * wv
  uint64_t vtail[R / 32];   // tail copy j: this lane's 16-byte source
  uint32_t lds_tail[R / 32];
};
template <int R>
__device__ __forceinline__ KvGather<R> kv_gather_prepare(char* tile, const uint16_t* kv, int64_t s_kv,
                                                         const int* rows, int count, int wv, int lane) {
  constexpr int PER = R / 4;
  static_assert(PER == 8 || PER == 16, "row copies per wave: 8 or 16");
  KvGather<R> g;
  const uint32_t base = lds_offset(tile);
  const uint64_t kva = reinterpret_cast<uint64_t>(kv);
  const uint64_t zero = reinterpret_cast<uint64_t>(g_zero_row);
  {
    const int r = PER * wv + (lane & (PER - 1));
    const int row = rows[r];
    const bool ok = r < count && (uint32_t)row < (uint32_t)s_kv;
    g.vaddr = ok ? kva + (uint64_t)(uint32_t)row * (2 * D_K) : zero;
  }
  // swz_lo(PER wv + J) = swz_lo(PER wv) ^ J for J < PER (PER wv mod 16 is 0 or 8)
  g.vswz = 16u * (uint32_t)(lane ^ ((PER * wv) & 15));
  g.lds_rows = base + 1024u * (uint32_t)(PER * wv);
#pragma unroll
  for (int j = 0; j < R / 32; ++j) {
    const int jj = wv + 4 * j;
    const int r = 8 * jj + (lane >> 3);
    const int row = rows[r];
    const bool ok = r < count && (uint32_t)row < (uint32_t)s_kv;
    g.vtail[j] = (ok ? kva + (uint64_t)(uint32_t)row * (2 * D_K) : zero) +
                 2u * (uint32_t)(D_V + 8 * ((lane & 7) ^ swz_hi(r)));
    g.lds_tail[j] = base + (uint32_t)(R * 1024 + 1024 * jj);
  }
  return g;
}
template <int R, int J>
__device__ __forceinline__ void kv_gather_copy(const KvGather<R>& g, int wv, int lane) {
  constexpr int PER = R / 4;
  if constexpr (J < PER) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)g.vaddr, J);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(g.vaddr >> 32), J);
    const void* src = reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
    g2lds16_s(src, g.vswz ^ (16u * J), g.lds_rows + 1024u * J);
  } else if constexpr (J < PER + R / 32) {
    constexpr int j = J - PER;
    g2lds16_u(reinterpret_cast<const void*>(g.vtail[j]), g.lds_tail[j]);
  }
}
// Copy J of a gather of R contiguous rows of CH chunks starting at `first`
// (rows >= nvalid read the zero row): J < R/4 row copies, then R/32 tail
// copies when CH = 72.
template <int R, int CH, int J>
__device__ __forceinline__ void seq_gather_copy(char* tile, const uint16_t* first, int nvalid,
                                                int wv, int lane) {
  constexpr int PER = R / 4;
  constexpr int W = CH * 8;
  const uint32_t base = lds_offset(tile);
  if constexpr (J < PER) {
    const int r = PER * wv + J;
    const bool ok = r < nvalid;
    const uint16_t* src = (ok ? first : g_zero_row) + (uint32_t)(ok ? r : 0) * (uint32_t)W;
    g2lds16_s(src, 16u * (uint32_t)(lane ^ swz_lo(r)), base + 1024u * (uint32_t)r);
  } else if constexpr (CH == ROW_CHUNKS && J < PER + R / 32) {
    constexpr int j = J - PER;
    const int jj = wv + 4 * j;
    const int r = 8 * jj + (lane >> 3);
    const bool ok = r < nvalid;
    const uint16_t* src = (ok ? first + (uint32_t)r * (uint32_t)W : g_zero_row) + D_V +
                          8 * ((lane & 7) ^ swz_hi(r));
    g2lds16_u(src, base + (uint32_t)(R * 1024 + 1024 * jj));
  }
}

// Bytes of swizzled tiles.
constexpr int KV64_TILE_BYTES = 64 * D_K * 2;   // 73728
constexpr int KV32_TILE_BYTES = 32 * D_K * 2;   // 36864

constexpr int DO32_TILE_BYTES = 32 * D_V * 2;   // 32768

// Copies `tile_rows` entries [first, first + tile_rows) of a query group's
// union (kv row indices, and token masks as 4-byte words of 4 entries each)
// into LDS with one direct copy each; rows at or past `count` read the zero
// chunk.  The planner zero-fills the masks from `count` up to the next
// multiple of 64 and `first` is a multiple of the tile size, so the mask
// words never carry stale entries.  Issued by wave `wv_rows` (rows) and wave
// `wv_mask` (masks) only.
__device__ __forceinline__ void copy_union_entries(int* rows_dst, unsigned char* mask_dst,
                                                   const int32_t* erow, const uint8_t* emask,
                                                   int first, int count, int tile_rows,
                                                   int wv, int wv_rows, int wv_mask, int lane) {
  const uint64_t zero = reinterpret_cast<uint64_t>(zero_row());
  if (rows_dst && wv == wv_rows) {
    const bool ok = lane < tile_rows && first + lane < count;
    g2lds4(reinterpret_cast<const void*>(ok ? reinterpret_cast<uint64_t>(erow + first + lane) : zero),
           rows_dst);
  }
  if (mask_dst && wv == wv_mask) {
    const bool ok = 4 * lane < tile_rows && first + 4 * lane < count;
    g2lds4(reinterpret_cast<const void*>(ok ? reinterpret_cast<uint64_t>(emask + first + 4 * lane) : zero),
           mask_dst);
  }
}

}  // namespace smla
