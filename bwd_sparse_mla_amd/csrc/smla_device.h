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
// Pointing lane L of a group at row 4*(L>>2 & 3)... of a row-major [k][n]
// tile (see tr_b_addr) turns row-major storage into a B fragment whose
// reduction index runs along rows, which is how V, K and Q/dO are consumed
// when the contraction runs over kv rows or query rows.
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
constexpr int TILE_STRIDE_CHUNKS = ROW_CHUNKS + 1;  // one 16-byte pad per LDS row
constexpr int TILE_STRIDE = TILE_STRIDE_CHUNKS * 16;  // 1168 bytes
constexpr int DO_CHUNKS = D_V / 8;           // 64 chunks per dout row
constexpr int DO_STRIDE_CHUNKS = DO_CHUNKS + 1;
constexpr int DO_STRIDE = DO_STRIDE_CHUNKS * 16;  // 1040 bytes
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float SUMEXP_FLOOR = 1e-30f;
// Running-max start: finite, so exp2(m_old - m_new) never sees inf - inf.
constexpr float M_INIT = -1e30f;

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

// B fragment [32 x 16] whose element (k, n) sits at row k0+k, column n0+n of a
// row-major LDS tile with `stride` bytes per row (bf16 elements).  Two
// transposing reads give k = 8g..8g+3 and 8g+4..8g+7 for lane column r.
__device__ __forceinline__ short8_t ld_b_tr(const char* tile, int stride, int k0, int n0, int lane) {
  const int g = lane >> 4, L = lane & 15;
  const int row = k0 + 8 * g + (L >> 2);
  const int col = n0 + 4 * (L & 3);
  const char* p0 = tile + row * stride + col * 2;
  short4_t lo = ld_tr16(p0);
  short4_t hi = ld_tr16(p0 + 4 * stride);
  short8_t r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
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

// s_waitcnt vmcnt(0) (other counters untouched).
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Reductions across the 16 lanes that share l >> 4 (one C-fragment row group).
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}

// Exclusive prefix sum over a 256-thread block; returns this thread's
// exclusive prefix and writes the block total to *total.  `scratch` holds at
// least 8 ints of LDS.  Must be called by all threads.
__device__ __forceinline__ int block_exclusive_scan256(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
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

// A zero 16-byte chunk that padding lanes of the LDS gathers copy from, so a
// padding row of a tile holds true zeros and never reaches outside the inputs.
__device__ __attribute__((aligned(16))) const unsigned g_zero16[4] = {0u, 0u, 0u, 0u};

// Bytes of an LDS tile of `rows` kv rows gathered by gather_kv_tile: the
// rows at TILE_STRIDE bytes (72 data chunks + 1 pad chunk each), rounded up to
// whole 1 KB copies.
__host__ __device__ constexpr int kv_tile_copies(int rows) {
  return (rows * TILE_STRIDE_CHUNKS + 63) / 64;
}
__host__ __device__ constexpr int kv_tile_bytes(int rows) { return kv_tile_copies(rows) * 1024; }

// Gathers `count` (>= 1) union rows, whose kv row indices sit in LDS at
// `rows` (entries 0..count-1), into an LDS tile of TILE_ROWS rows
// (kv_tile_bytes(TILE_ROWS) bytes) with direct global->LDS copies of 64 lanes
// x 16 bytes, copy i issued by wave i % 4.  Rows past `count`, pad chunks and
// the tail of the last copy read the zero chunk.  Every row index is clamped
// into [0, s_kv) before it forms an address, so no value in `rows` can reach
// outside kv.  All indices are read from LDS before the first copy and no
// memory read sits between copies, so the copies issue back to back.
// `wv` must be wave-uniform.
template <int TILE_ROWS>
__device__ __forceinline__ void gather_kv_tile(char* dst, const uint16_t* kv, int64_t s_kv,
                                               const int* rows, int count, int wv, int lane) {
  constexpr int NCOPY = kv_tile_copies(TILE_ROWS);
  constexpr int PER_WAVE = (NCOPY + 3) / 4;
  int rowv[PER_WAVE];
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int p = (wv + 4 * j) * 64 + lane;
    const int r = p / TILE_STRIDE_CHUNKS;
    rowv[j] = rows[r < count ? r : count - 1];
  }
  const uint64_t zero = reinterpret_cast<uint64_t>(g_zero16);
  const uint64_t base = reinterpret_cast<uint64_t>(kv);
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int i = wv + 4 * j;
    if (i < NCOPY) {
      const int p = i * 64 + lane;
      const int r = p / TILE_STRIDE_CHUNKS, c = p - r * TILE_STRIDE_CHUNKS;
      int64_t row = rowv[j];
      row = row < 0 ? 0 : (row >= s_kv ? s_kv - 1 : row);
      const uint64_t a = base + (uint64_t)(row * D_K + 8 * c) * 2u;
      g2lds16(reinterpret_cast<const void*>((c < ROW_CHUNKS && r < count) ? a : zero),
              dst + i * 1024);
    }
  }
}

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
  const uint64_t zero = reinterpret_cast<uint64_t>(g_zero16);
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
