// Sparse-MLA backward (gfx950): dq and dkv of the loss sum(dout * out), given
// the forward's out and lse, as the backward call on the pages receives them
// (slime issue #2201, "GLM-5.2 SparseMLA TileLang backward returns NaN
// gradients from finite inputs", section Suspected area).
//
// With z = scale q.k, p = exp(z - lse) and delta = rowsum(dout * out):
//   dp = dout . v,  ds = p (dp - delta),
//   dq[s,h]    = scale sum_j ds_j k_j
//   dkv[j]    += scale ds_j q[s,h]  (all 576 columns)  +  p_j dout[s,h]  (first 512)
//
// Two passes, neither uses atomics, both bitwise reproducible:
//  * dq pass, query-major (the forward's structure): per query group and
//    union tile, scores and dP share the K fragments read from LDS, then
//    dq += dS . K with K read once through transposing LDS reads.  It also
//    computes delta for its rows and leaves it in the workspace.
//  * dkv pass, kv-major: one workgroup per 64-row KV block keeps the block's
//    rows as MFMA fragments, walks the block's (token, row-mask) records in
//    (group, token) order, recomputes S^T, P^T, dP^T and dS^T for those
//    tokens' 64 query rows and accumulates dkv = dS^T . Q + P^T . dO in
//    registers; each dkv row is written exactly once.  This is the
//    sort-by-row segmented reduction: the records are the (token, slot)
//    pairs grouped by kv block, and the reduction runs on the matrix cores.
// Padding slots contribute nothing and write nothing: they are never part of
// a record or a union entry (miles PR #2079 digest, "fix GLM-5 sparse-MLA
// kernel -1 index OOB and NaN gradients", 实现拆解 item 3 -- there a clamped
// -1 added exact zeros into row 0; here it adds nothing anywhere).
#include <type_traits>

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

// Compacts each dkv unit's column of the [block, group] record table into
// the unit's chunk list (groups with records for the unit, ascending).  In
// the stored-P form a unit is a pair of blocks: a group with records in
// either block is a chunk, with, per block, its first union entry there and
// the rows it selects (zero where it has none).
// Exclusive prefix sum over a block of NT threads (a multiple of 64);
// returns this thread's exclusive prefix and writes the block total to
// *total.  `scratch` holds at least NT / 64 ints of LDS.  Must be called by
// all threads.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan_nt(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int s = scratch[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

template <int NT>
__device__ __forceinline__ void dkv_schedule_unit(const BwdArgs& a, int64_t unit) {
  __shared__ int scratch[NT / 64];
  const int tid = threadIdx.x;
  int base = 0;
  for (int64_t gb = 0; gb < a.G; gb += NT) {
    const int64_t g = gb + tid;
    int2 e = make_int2(0, 0), e1 = make_int2(0, 0);
    if (a.ub == 2) {
      if (g < a.G) e = a.ktab[(2 * unit) * a.G + g];
      if (g < a.G && 2 * unit + 1 < a.NB) e1 = a.ktab[(2 * unit + 1) * a.G + g];
    } else if (g < a.G) {
      e = a.ktab[unit * a.G + g];
    }
    const int nz = (e.y > 0 || e1.y > 0) ? 1 : 0;
    int total;
    const int pos = base + block_exclusive_scan_nt<NT>(nz, scratch, &total);
    if (nz) {
      a.clist[unit * a.G + pos] = make_int2((int)g, e.x);
      if (a.ub == 2) {   // stored-P form: per block, the first union entry and the rows
        const int64_t c = unit * a.G + pos;
        const int64_t k0 = (2 * unit) * a.G + g, k1 = (2 * unit + 1) * a.G + g;
        a.cbase[2 * c] = e.y > 0 ? a.kbase[k0] : 0;
        a.cmask[2 * c] = e.y > 0 ? a.korm[k0] : 0ull;
        a.cbase[2 * c + 1] = e1.y > 0 ? a.kbase[k1] : 0;
        a.cmask[2 * c + 1] = e1.y > 0 ? a.korm[k1] : 0ull;
      }
    }
    base += total;
  }
  if (tid == 0) a.nchunk[unit] = base;
}

__global__ __launch_bounds__(256) void dkv_schedule_kernel(BwdArgs a) {
  dkv_schedule_unit<256>(a, blockIdx.x);
}

// Flat kv row of block row b, and the block row of flat row f (b, f < 2^24).
__device__ __forceinline__ int64_t kv_flat_row(int64_t b, int kvg, int64_t kvs) {
  if (kvg == 1) return b;
  const uint32_t g = (uint32_t)b / (uint32_t)kvs;
  return (int64_t)((uint32_t)b - g * (uint32_t)kvs) * kvg + g;
}
__device__ __forceinline__ int64_t kv_block_row(int64_t f, int kvg, int64_t kvs) {
  if (kvg == 1) return f;
  const uint32_t v = (uint32_t)f / (uint32_t)kvg;
  return (int64_t)((uint32_t)f - v * (uint32_t)kvg) * kvs + v;
}

// ---------------------------------------------------------------------------
// dq pass
// ---------------------------------------------------------------------------
// Query group of T = 64/H tokens (64 rows), union tiles of 32 kv rows.  One
// workgroup of 8 waves, two roles one tile apart (two waves per SIMD, so one
// role's softmax, copies and LDS waits overlap the other's MFMAs):
//   score waves 0-3: wave w takes rows 16w .. 16w+15 of tile j: S^T = K Q^T
//       and dP^T = V dO^T sharing the K fragments (K from LDS as the A
//       operand, the wave's Q and dout rows held in registers as B operands,
//       36 + 32 MFMA 16x16x32), then P = exp(S - lse), dS = P (dP - delta)
//       to LDS (and, in the stored-P form, P and scale * dS staged in the
//       workspace's layout);
//   dq waves 4-7:    wave 4+c accumulates dq[64 rows, 128c .. 128c+127 and
//       tail block 512 + 16c] += dS . K for tile j - 1 (as dq^T = K^T dS^T,
//       K^T through transposing LDS reads as the A operand, 36 MFMA), writes
//       tile j - 1's staged P and dS out, and at the end stores its dq
//       columns straight from its registers (16-byte row pieces).
// One barrier per step: every wave waits for its copies, the workgroup syncs,
// then the dq waves issue the copies of tile j + 1 (8 kv rows and their
// tails per dq wave, the masks of tile j + 1 and the row indices of tile
// j + 2) and the roles work.  delta = rowsum(dout * out) is formed by the
// score waves from their dout registers in the prologue.
constexpr int DQ_TILE = 32;
constexpr int DQ_NW = 8;                 // waves per dq workgroup
constexpr int SDS = DQ_TILE + 8;         // dS row stride (bf16): 80 bytes, conflict-free reads

template <int H>
__global__ __launch_bounds__(DQ_NW * 64, 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int T = GROUP_ROWS / H;
  __shared__ __attribute__((aligned(16))) char sK[3][KV32_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned short sdS[2][GROUP_ROWS * SDS];
  __shared__ __attribute__((aligned(16))) unsigned char sMask[2][256];   // token masks (copied as words)
  __shared__ __attribute__((aligned(16))) int sRow[2][64];   // kv row indices of a tile's entries
  // stored-P form: a tile's P and scale * dS as [entry, {P, dS}, 64 rows]
  // bf16, the layout of the workspace, for one contiguous 8 KB copy out
  __shared__ __attribute__((aligned(16))) unsigned short sPDS[2][DQ_TILE * 2 * GROUP_ROWS];

  // The first NU workgroups build the dkv pass's chunk lists (they depend on
  // the plan only, so they run beside the dq work instead of in a launch of
  // their own).
  if ((int64_t)blockIdx.x < a.NU) {
    dkv_schedule_unit<DQ_NW * 64>(a, blockIdx.x);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool score_wave = wv < 4;
  const int lw = wv & 3;                   // index within the role
  const int g16 = lane >> 4, r16 = lane & 15;
  const int64_t grp = a.gorder[blockIdx.x - a.NU];
  const int64_t t0 = grp * T;
  const int n_ent = a.qcount[grp];
  const int32_t* erow = a.qrow + grp * a.qcap;
  const uint8_t* emask = a.qmask + grp * a.qcap;
  const int ntiles = (n_ent + DQ_TILE - 1) / DQ_TILE;
  const bool stored = a.pds != nullptr;
  auto tile_count = [&](int t) __attribute__((always_inline)) {
    return max(0, min(DQ_TILE, n_ent - t * DQ_TILE));
  };

  // Tile 0 is gathered at once by the dq waves, its row indices read straight
  // from the union list (so the gather overlaps the score waves' prologue
  // loads); the masks of tile 0 (wave 4) and the row indices of tile 1
  // (wave 5) go to LDS.
  copy_union_entries(nullptr, sMask[0], erow, emask, 0, n_ent, DQ_TILE, wv, -1, 4, lane);
  copy_union_entries(sRow[1], nullptr, erow, emask, DQ_TILE, n_ent, DQ_TILE, wv, 5, -1, lane);
  if (!score_wave && ntiles > 0) {
    const KvGather<DQ_TILE> g = kv_gather_prepare<DQ_TILE>(sK[0], a.kv, a.s_kv, erow, tile_count(0), lw, lane);
    static_for<DQ_TILE / 4 + 1>([&](auto J) __attribute__((always_inline)) {
      kv_gather_copy<DQ_TILE, decltype(J)::value>(g, lw, lane);
    });
  }

  // Copies of tile t into sK[t % 3] (its row indices in sRow[t & 1]), all by
  // the dq waves (the score waves carry more of a step's work): dq wave 4+c
  // copies the first 1 KB of rows 8c .. 8c+7 and their tails; wave 4 the
  // masks of tile t, wave 5 the row indices of tile t + 1.  Past the union
  // they read the zero row into buffers no live tile uses.
  auto issue = [&](int t) __attribute__((always_inline)) {
    const KvGather<DQ_TILE> g = kv_gather_prepare<DQ_TILE>(sK[t % 3], a.kv, a.s_kv, sRow[t & 1],
                                                           tile_count(t), lw, lane);
    static_for<DQ_TILE / 4 + 1>([&](auto J) __attribute__((always_inline)) {
      kv_gather_copy<DQ_TILE, decltype(J)::value>(g, lw, lane);
    });
    copy_union_entries(nullptr, sMask[t & 1], erow, emask, t * DQ_TILE, n_ent, DQ_TILE, wv, -1, 4, lane);
    copy_union_entries(sRow[(t + 1) & 1], nullptr, erow, emask, (t + 1) * DQ_TILE, n_ent, DQ_TILE, wv, 5,
                       -1, lane);
  };

  if (score_wave) {
    // Q and dout of row 16w + r as B fragments (k-step ks: columns 32 ks +
    // 8g .. +7), delta and lse of the row.
    const int rr = 16 * wv + r16;
    const int64_t tok = t0 + rr / H;
    const int tl = rr / H;                 // group-local token of the lane's row
    short8_t qf[18], df[16];
    float del, ls2 = 0.f;
    {
      short8_t of[16];
      if (tok < a.s_q) {
        const int64_t row = tok * H + rr % H;                                        // lse (group-major)
        const int64_t crw = caller_token(tok, a.pair_s, a.pair_g) * H + rr % H;   // q, dout, out
        const uint16_t* qp = a.q + crw * D_K + 8 * g16;
        const uint16_t* dp = a.dout + crw * D_V + 8 * g16;
        const uint16_t* op = a.out + crw * D_V + 8 * g16;
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) qf[ks] = ld16_global(qp + 32 * ks);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          df[ks] = ld16_global(dp + 32 * ks);
          of[ks] = ld16_global(op + 32 * ks);
        }
        ls2 = a.lse[row] * LOG2E;
      } else {
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) qf[ks] = (short8_t){0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          df[ks] = (short8_t){0, 0, 0, 0, 0, 0, 0, 0};
          of[ks] = (short8_t){0, 0, 0, 0, 0, 0, 0, 0};
        }
      }
      // delta = rowsum(dout * out): the lane's 128 columns, then the row's
      // four lanes (g = 0..3: lanes r, r + 16, r + 32, r + 48).
      float d = 0.f;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) d += bf2f((unsigned short)df[ks][j]) * bf2f((unsigned short)of[ks][j]);
      d = sum_rows(d);   // (d_r + d_r+16) + (d_r+32 + d_r+48)
      del = d;
      if (g16 == 0 && tok < a.s_q) a.delta[tok * H + rr % H] = d;
    }
    wait_vmcnt0();
    __syncthreads();   // tile 0, its masks and the row indices of tile 1

    for (int j = 0; j <= ntiles; ++j) {
      wait_vmcnt0();
      __syncthreads();
      if (j >= ntiles) continue;
      // Scores and dP of tile j: lane (g, r) holds kv entries 16 nt + 4g + i.
      const char* kt = sK[j % 3];
      const unsigned char* mkb = sMask[j & 1];
      float4_t s[2], dp[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        s[nt] = (float4_t){0.f, 0.f, 0.f, 0.f};
        dp[nt] = (float4_t){0.f, 0.f, 0.f, 0.f};
      }
      // K fragments KPF k-steps ahead of their MFMAs.
      constexpr int KPF = 3;
      short8_t kb[KPF + 1][2];
#pragma unroll
      for (int d = 0; d < KPF; ++d)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) kb[d][nt] = ld_b_rs<DQ_TILE>(kt, nt * 16, 32 * d, lane);
      static_for<18>([&](auto KS) __attribute__((always_inline)) {
        constexpr int ks = decltype(KS)::value;
        constexpr int cur = ks % (KPF + 1), nxt = (ks + KPF) % (KPF + 1);
        if constexpr (ks + KPF < 18) {
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) kb[nxt][nt] = ld_b_rs<DQ_TILE>(kt, nt * 16, 32 * (ks + KPF), lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          s[nt] = mfma_bf16(kb[cur][nt], qf[ks], s[nt]);
          if constexpr (ks < 16) dp[nt] = mfma_bf16(kb[cur][nt], df[ks], dp[nt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      unsigned short* pt = sPDS[j & 1];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const unsigned mk = *reinterpret_cast<const unsigned*>(mkb + nt * 16 + 4 * g16);
        float d[4], pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool v = (mk >> (8 * i + tl)) & 1u;
          pr[i] = v ? fast_exp2(s[nt][i] * a.scale_log2 - ls2) : 0.f;
          d[i] = pr[i] * (dp[nt][i] - del);
        }
        uint2 pk;
        pk.x = pack_bf2(d[0], d[1]);
        pk.y = pack_bf2(d[2], d[3]);
        *reinterpret_cast<uint2*>(&sdS[j & 1][rr * SDS + nt * 16 + 4 * g16]) = pk;
        if (stored) {
          // P and scale * dS of the lane's row for its four entries, staged
          // in the workspace's layout.
          unsigned short* st = pt + (nt * 16 + 4 * g16) * 2 * GROUP_ROWS + rr;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            st[i * 2 * GROUP_ROWS] = f2bf(pr[i]);
            st[i * 2 * GROUP_ROWS + GROUP_ROWS] = f2bf(d[i] * a.scale);
          }
        }
      }
    }
  } else {
    const int c = lw;   // column pairs 128c + 32m (blocks 2m, 2m + 1), tail block 512 + 16c
    float4_t acc[4][9];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int n = 0; n < 9; ++n) acc[rb][n] = (float4_t){0.f, 0.f, 0.f, 0.f};
    wait_vmcnt0();
    __syncthreads();

    for (int j = 0; j <= ntiles; ++j) {
      wait_vmcnt0();
      __syncthreads();
      if (j + 1 < ntiles) issue(j + 1);
      if (j == 0) continue;
      const int jj = j - 1;
      if (stored) {   // tile jj's P and dS: 32 entries x 256 bytes, contiguous in the workspace
        uint4_t* dst = reinterpret_cast<uint4_t*>(a.pds + (grp * a.qcap + jj * DQ_TILE) * 2 * GROUP_ROWS);
        const uint4_t* src = reinterpret_cast<const uint4_t*>(sPDS[jj & 1]);
        const int t4 = tid - 256;   // dq waves' thread index, 0..255
        dst[t4] = src[t4];
        dst[t4 + 256] = src[t4 + 256];
      }
      // dq^T += K^T . dS^T for tile jj: all 64 rows, the wave's column blocks
      // (K^T as the A operand, so a lane's outputs are adjacent columns of one
      // row: blocks 2m and 2m + 1 together hold 8 adjacent columns); the
      // transposed K fragments run two column blocks ahead of their MFMAs.
      const char* kt = sK[jj % 3];
      short8_t dsa[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) dsa[rb] = ld16_lds(&sdS[jj & 1][(16 * rb + r16) * SDS + 8 * g16]);
      auto kt_frag = [&](int n) __attribute__((always_inline)) {
        return n < 8 ? ld_bt_rs_pair<DQ_TILE>(kt, 0, 128 * c + 32 * (n >> 1), n & 1, lane)
                     : ld_bt_rs_hi<DQ_TILE>(kt, 0, D_V + 16 * c, lane);
      };
      constexpr int BPF = 2;
      short8_t bb[BPF + 1];
#pragma unroll
      for (int d = 0; d < BPF; ++d) bb[d] = kt_frag(d);
#pragma unroll
      for (int n = 0; n < 9; ++n) {
        if (n + BPF < 9) bb[(n + BPF) % (BPF + 1)] = kt_frag(n + BPF);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) acc[rb][n] = mfma_bf16(bb[n % (BPF + 1)], dsa[rb], acc[rb][n]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Epilogue: dq = scale * acc straight from the registers: lane (g, r)
    // holds columns 128c + 32m + 8g .. +7 (blocks 2m, 2m + 1) and tail
    // columns 512 + 16c + 4g .. +3 of rows 16 rb + r.
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int row = 16 * rb + r16;
      const int64_t tk = t0 + row / H;
      if (tk < a.s_q) {
        uint16_t* drow = a.dq + (caller_token(tk, a.pair_s, a.pair_g) * H + row % H) * D_K;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint4_t v;
          v[0] = pack_bf2(acc[rb][2 * m][0] * a.scale, acc[rb][2 * m][1] * a.scale);
          v[1] = pack_bf2(acc[rb][2 * m][2] * a.scale, acc[rb][2 * m][3] * a.scale);
          v[2] = pack_bf2(acc[rb][2 * m + 1][0] * a.scale, acc[rb][2 * m + 1][1] * a.scale);
          v[3] = pack_bf2(acc[rb][2 * m + 1][2] * a.scale, acc[rb][2 * m + 1][3] * a.scale);
          *reinterpret_cast<uint4_t*>(drow + 128 * c + 32 * m + 8 * g16) = v;
        }
        uint2 t;
        t.x = pack_bf2(acc[rb][8][0] * a.scale, acc[rb][8][1] * a.scale);
        t.y = pack_bf2(acc[rb][8][2] * a.scale, acc[rb][8][3] * a.scale);
        *reinterpret_cast<uint2*>(drow + D_V + 16 * c + 4 * g16) = t;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dkv pass
// ---------------------------------------------------------------------------
// kv-major: a kv block (64 rows) has a chunk list, one chunk per query group
// with records for the block (T tokens, 64 query rows, contiguous in q / dout
// / lse / delta); a chunk is processed as two sub-chunks of 32 query rows.
// DKV_WGS workgroups (one per CU) each take an equal share of all blocks'
// sub-chunks in block order (stream-K style: the work is even whatever the
// blocks' sizes), as one segment per block they meet.  A segment keeps the
// block's rows in registers, walks its sub-chunks double buffered (every
// step first issues the direct global->LDS copies of the next sub-chunk: Q,
// dout, its tokens' row masks, lse, delta -- all addresses computed, no
// memory read on the way -- then computes the current one), accumulates dkv
// in registers and writes an fp32 partial; dkv_finalize_kernel adds a
// block's partials in workgroup order.
constexpr int DKV_SUB = 32;                                 // query rows per sub-chunk

constexpr int DKV_NW = 8;                                   // waves per workgroup

// LDS of a dkv workgroup (double-buffered sub-chunks, P^T and dS^T tiles).
constexpr int DKV_SP = DKV_SUB + 8;  // P^T / dS^T row stride (bf16): 80 bytes
struct DkvLds {
  __attribute__((aligned(16))) char sQ[2][KV32_TILE_BYTES];
  __attribute__((aligned(16))) char sD[2][DO32_TILE_BYTES];
  __attribute__((aligned(16))) unsigned sM[2][64];   // T row masks (2 words each)
  __attribute__((aligned(16))) float sL[2][64];      // lse of the 32 rows
  __attribute__((aligned(16))) float sE[2][64];      // delta of the 32 rows
  __attribute__((aligned(16))) unsigned short sPT[TILE_KV * DKV_SP];
  __attribute__((aligned(16))) unsigned short sDST[TILE_KV * DKV_SP];
};

// Sub-chunks u0 .. u1-1 of kv block `blk` (sub-chunk u is query rows
// 32 (u & 1) .. +31 of the block's chunk u / 2); the fp32 partial dkv of the
// block's 64 rows goes to partial slot `slot`.
template <int H>
__device__ __forceinline__ void dkv_segment(const BwdArgs& a, int64_t blk, int u0, int u1, int64_t slot,
                                            DkvLds& lds) {
  constexpr int T = GROUP_ROWS / H;
  constexpr int SP = DKV_SP;
  auto& sQ = lds.sQ;
  auto& sD = lds.sD;
  auto& sM = lds.sM;
  auto& sL = lds.sL;
  auto& sE = lds.sE;
  auto& sPT = lds.sPT;
  auto& sDST = lds.sDST;
  const int tid = threadIdx.x, lane_id = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = a.nchunk[blk];
  const int64_t kb0 = blk * TILE_KV;
  const int64_t qrows = a.s_q * H;   // rows of q / dout / lse / delta

  // Scores / dP: wave w takes kv rows 16 (w & 3) + r (their K fragments stay
  // in registers: the B operand, K^T; the first 512 columns, ks < 16, are V
  // for dP) against query rows 16 (w >> 2) .. +15 of the sub-chunk.
  const int skb = wv & 3, sqh = wv >> 2;
  // dK / dV: wave w accumulates kv rows 32 (w & 1) .. +31 (two 16-row
  // blocks) x 9 column blocks of 16: 128 (w >> 1) .. +127 and tail columns
  // 512 + 16 (w >> 1) .. +15.
  const int drh = wv & 1, dcq = wv >> 1;
  short8_t kf[18];
  {
    const int64_t row = kb0 + 16 * skb + (lane_id & 15);
    if (row < a.s_kv) {
      const uint16_t* kr = a.kv + kv_flat_row(row, a.kvg, a.kvs) * D_K + 8 * (lane_id >> 4);
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) kf[ks] = ld16_global(kr + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) kf[ks] = (short8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  float4_t acc[2][9];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int n = 0; n < 9; ++n) acc[rb][n] = (float4_t){0.f, 0.f, 0.f, 0.f};
  unsigned long long touched = 0ull;

  const uint64_t zero = reinterpret_cast<uint64_t>(zero_row());
  // Sub-chunk u covers query rows 32 (u & 1) .. +31 of chunk u / 2 (a
  // query group); its buffers hold those rows of Q and dout as swizzled
  // 32-row tiles, the group's token masks for the block, and the rows' lse and
  // delta.  Every step first issues the copies of sub-chunk u+1 (4 Q rows,
  // one Q tail copy for waves 0-3, 4 dout rows and, for waves 5-7, the masks /
  // lse / delta) into the other buffer set.
  const int2* clist = a.clist + blk * a.G;
  int2 ce_cur = clist[u0 >> 1];                            // chunk of the current sub-chunk
  int2 ce_nxt = clist[min((u0 >> 1) + 1, nch - 1)];        // the chunk after it
  auto small_copy = [&](int2 ce, int64_t row0, unsigned* m_dst, float* l_dst, float* e_dst, int lane) __attribute__((always_inline)) {
    if (wv == 5) {
      const uint64_t src = reinterpret_cast<uint64_t>(a.krmask + (int64_t)ce.x * a.rcap + ce.y) + 4u * lane;
      g2lds4(reinterpret_cast<const void*>(lane < 2 * T ? src : zero), m_dst);
    } else if (wv == 6) {
      const uint64_t src = reinterpret_cast<uint64_t>(a.lse + row0 + lane);
      g2lds4(reinterpret_cast<const void*>((lane < DKV_SUB && row0 + lane < qrows) ? src : zero), l_dst);
    } else if (wv == 7) {
      const uint64_t src = reinterpret_cast<uint64_t>(a.delta + row0 + lane);
      g2lds4(reinterpret_cast<const void*>((lane < DKV_SUB && row0 + lane < qrows) ? src : zero), e_dst);
    }
  };
  auto rows_of = [&](int2 ce, int u, int64_t& row0, int& nvalid) __attribute__((always_inline)) {
    row0 = (int64_t)ce.x * GROUP_ROWS + DKV_SUB * (u & 1);
    nvalid = (int)max((int64_t)0, min((int64_t)DKV_SUB, qrows - row0));
  };

  auto step = [&](int u, const char* sq, const char* sd, const unsigned* sm, const float* sl,
                  const float* se, char* nq, char* nd, unsigned* nm, float* nl, float* ne) __attribute__((always_inline)) {
    wait_vmcnt0();
    __syncthreads();
    if (u + 1 < u1) {   // copies of sub-chunk u+1 into the other buffer set
      int lane = lane_id;
      asm volatile("" : "+v"(lane));   // offsets recomputed per sub-chunk, not kept live
      const int2 cen = (u & 1) ? ce_nxt : ce_cur;
      int64_t nrow0;
      int nvalid;
      rows_of(cen, u + 1, nrow0, nvalid);
      gather_seq_rows_nw<DKV_SUB, ROW_CHUNKS, DKV_NW, H>(nq, a.q, nrow0, nvalid, a.pair_s, a.pair_g, wv, lane);
      gather_seq_rows_nw<DKV_SUB, DO_CHUNKS, DKV_NW, H>(nd, a.dout, nrow0, nvalid, a.pair_s, a.pair_g, wv, lane);
      small_copy(cen, nrow0, nm, nl, ne, lane);
    }
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int g16 = lane >> 4, r16 = lane & 15;
    const int half = u & 1;
    // rows each token of the chunk selects; this sub-chunk's query rows are
    // 32*half .. 32*half+31 of the group, token slot = row / H
#pragma unroll
    for (int sl2 = 0; sl2 < T; ++sl2)
      touched |= (unsigned long long)sm[2 * sl2] | ((unsigned long long)sm[2 * sl2 + 1] << 32);

    // S and dP for query rows 16 sqh .. +15 (M) against kv rows 16 skb .. +15
    // (N): lane (g, r) holds query rows 16 sqh + 4g + i of kv row 16 skb + r.
    // Q / dout fragments run KPF k-steps ahead of their MFMAs.
    // Even and odd k-steps accumulate separately (four independent MFMA
    // chains of depth 9 instead of two of depth 18) and are added at the end.
    float4_t st2[2], dpt2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      st2[e] = (float4_t){0.f, 0.f, 0.f, 0.f};
      dpt2[e] = (float4_t){0.f, 0.f, 0.f, 0.f};
    }
    constexpr int KPF = 3;
    short8_t qb[KPF + 1], db[KPF + 1];
#pragma unroll
    for (int d = 0; d < KPF; ++d) {
      qb[d] = ld_b_rs<DKV_SUB>(sq, 16 * sqh, 32 * d, lane);
      db[d] = ld_b_rs<DKV_SUB>(sd, 16 * sqh, 32 * d, lane);
    }
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (ks + KPF < 18) {
        qb[(ks + KPF) % (KPF + 1)] = ld_b_rs<DKV_SUB>(sq, 16 * sqh, 32 * (ks + KPF), lane);
        if (ks + KPF < 16) db[(ks + KPF) % (KPF + 1)] = ld_b_rs<DKV_SUB>(sd, 16 * sqh, 32 * (ks + KPF), lane);
      }
      __builtin_amdgcn_sched_barrier(0);
      st2[ks & 1] = mfma_bf16(qb[ks % (KPF + 1)], kf[ks], st2[ks & 1]);
      if (ks < 16) dpt2[ks & 1] = mfma_bf16(db[ks % (KPF + 1)], kf[ks], dpt2[ks & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const float4_t st = st2[0] + st2[1], dpt = dpt2[0] + dpt2[1];
    {
      const int kvl = 16 * skb + r16;
      const int q0 = 16 * sqh + 4 * g16;            // first of the lane's 4 query rows
      const int slot = (DKV_SUB * half + q0) / H;   // one token for all 4 (H >= 4)
      const unsigned long long m =
          (unsigned long long)sm[2 * slot] | ((unsigned long long)sm[2 * slot + 1] << 32);
      const bool v = (m >> kvl) & 1ull;
      const float4_t l2 = *reinterpret_cast<const float4_t*>(sl + q0);
      const float4_t dl = *reinterpret_cast<const float4_t*>(se + q0);
      float p[4], ds[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = v ? fast_exp2(st[i] * a.scale_log2 - l2[i] * LOG2E) : 0.f;
        ds[i] = p[i] * (dpt[i] - dl[i]) * a.scale;
      }
      uint2 pk, dk;
      pk.x = pack_bf2(p[0], p[1]);
      pk.y = pack_bf2(p[2], p[3]);
      dk.x = pack_bf2(ds[0], ds[1]);
      dk.y = pack_bf2(ds[2], ds[3]);
      *reinterpret_cast<uint2*>(&sPT[kvl * SP + q0]) = pk;
      *reinterpret_cast<uint2*>(&sDST[kvl * SP + q0]) = dk;
    }
    __syncthreads();

    // dK / dV for kv rows 32 drh .. +31 and the wave's 9 column blocks:
    // blocks n < 8 are columns 128 dcq + 16 n (dK and dV), block 8 is tail
    // columns 512 + 16 dcq (dK only).  The transposed Q / dout fragments of
    // block n+1 are read before the MFMAs of block n.
    short8_t ad[2], ap[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      ad[rb] = ld16_lds(&sDST[(32 * drh + 16 * rb + r16) * SP + 8 * g16]);
      ap[rb] = ld16_lds(&sPT[(32 * drh + 16 * rb + r16) * SP + 8 * g16]);
    }
    const int col0 = 128 * dcq;
    short8_t bq = ld_bt_rs_lo<DKV_SUB>(sq, 0, col0, lane);
    short8_t bo = ld_bt_rs_lo<DKV_SUB>(sd, 0, col0, lane);
#pragma unroll
    for (int n = 0; n < 9; ++n) {
      short8_t bqn = bq, bon = bo;
      if (n + 1 < 8) {
        bqn = ld_bt_rs_lo<DKV_SUB>(sq, 0, col0 + 16 * (n + 1), lane);
        bon = ld_bt_rs_lo<DKV_SUB>(sd, 0, col0 + 16 * (n + 1), lane);
      } else if (n + 1 == 8) {
        bqn = ld_bt_rs_hi<DKV_SUB>(sq, 0, D_V + 16 * dcq, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) acc[rb][n] = mfma_bf16(ad[rb], bq, acc[rb][n]);
      if (n < 8) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) acc[rb][n] = mfma_bf16(ap[rb], bo, acc[rb][n]);
      }
      __builtin_amdgcn_sched_barrier(0);
      bq = bqn;
      bo = bon;
    }
    if (u & 1) {   // the next sub-chunk starts chunk u/2 + 1: load the one after it
      ce_cur = ce_nxt;
      if ((u >> 1) + 2 < nch) ce_nxt = clist[(u >> 1) + 2];
    }
  };

  {
    int64_t row0;
    int nvalid;
    rows_of(ce_cur, u0, row0, nvalid);
    gather_seq_rows_nw<DKV_SUB, ROW_CHUNKS, DKV_NW, H>(sQ[0], a.q, row0, nvalid, a.pair_s, a.pair_g, wv, lane_id);
    gather_seq_rows_nw<DKV_SUB, DO_CHUNKS, DKV_NW, H>(sD[0], a.dout, row0, nvalid, a.pair_s, a.pair_g, wv, lane_id);
    small_copy(ce_cur, row0, sM[0], sL[0], sE[0], lane_id);
  }
  for (int u = u0; u < u1; ++u) {
    const int b = (u - u0) & 1;
    step(u, sQ[b], sD[b], sM[b], sL[b], sE[b], sQ[b ^ 1], sD[b ^ 1], sM[b ^ 1], sL[b ^ 1], sE[b ^ 1]);
  }

  // Partial sum of the segment: rows 32 drh + 16 rb + 4 g + i, columns
  // 128 dcq + 16 n + r (n < 8) and 512 + 16 dcq + r (n = 8).  The atomic mode
  // adds it into the block's rows of the fp32 accumulator with no-return
  // fp32 atomics instead (the order the segments' adds land in varies, so
  // that mode is not bitwise reproducible).
  if (a.acc32) {
    const int g16 = lane_id >> 4, r16 = lane_id & 15;
    float* dst = a.acc32 + (kb0 + 32 * drh + 4 * g16) * D_K + r16;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 9; ++n)
          unsafeAtomicAdd(&dst[(16 * rb + i) * D_K + (n < 8 ? 128 * dcq + 16 * n : D_V + 16 * dcq)],
                          acc[rb][n][i]);
  } else {
    const int g16 = lane_id >> 4, r16 = lane_id & 15;
    float* dst = a.part + (slot * TILE_KV + 32 * drh + 4 * g16) * D_K + r16;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 9; ++n)
          dst[(16 * rb + i) * D_K + (n < 8 ? 128 * dcq + 16 * n : D_V + 16 * dcq)] = acc[rb][n][i];
  }
  if (tid == 0) a.ptouch[2 * slot] = touched;
}

// Stored-P form (SMLA_DKV_STORED_P): the dq pass has left P and scale * dS
// of every (union entry, query row) in the workspace, so the dkv pass does
// not recompute scores or dP, and its unit is a pair of kv blocks (128 rows):
// one copy of a sub-chunk's Q / dout then serves twice the rows.  A chunk is
// a query group with records in either block.  Per step: wait for the copies,
// stage the sub-chunk's 128 x 32 P^T / dS^T tiles from the workspace (thread
// t takes kv row t / 8 of each block and 8 query rows of P or dS; the union
// entry of a selected row is the chunk's first entry in that block plus the
// selected rows before it; other rows are zero), issue the next sub-chunk's
// copies (Q, dout into the other buffers; its P / dS pieces into
// registers), sync, and run the dK / dV contraction: wave w takes kv rows
// 64 (w & 1) .. +63 (four 16-row blocks) and the column blocks of w >> 1.
// P^T / dS^T tiles of the stored-P form: 128 kv rows x 32 query rows (bf16),
// 64 bytes per row, with 16-byte chunk c of row r at 64-byte group
// 4 (r / 4) + (c ^ (r / 4 mod 4)), slot r mod 4 (offsets in bf16 units).  A
// fragment read (16 rows, one chunk) then keeps each quad of lanes inside one
// aligned 64-byte bank group and 16 lanes on all 64 banks.
__device__ __forceinline__ int pt_off(int r, int c) {
  return 32 * (4 * (r >> 2) + (c ^ ((r >> 2) & 3))) + 8 * (r & 3);
}

struct DkvPairLds {
  __attribute__((aligned(16))) char sQ[2][KV32_TILE_BYTES];
  __attribute__((aligned(16))) char sD[2][DO32_TILE_BYTES];
  __attribute__((aligned(16))) unsigned short sPT[2 * TILE_KV * DKV_SUB];
  __attribute__((aligned(16))) unsigned short sDST[2 * TILE_KV * DKV_SUB];
};

template <int H>
__device__ __forceinline__ void dkv_segment_pair(const BwdArgs& a, int64_t unit, int u0, int u1,
                                                 int64_t slot, DkvPairLds& lds) {
  constexpr int UR = 2 * TILE_KV;   // kv rows per unit
  auto& sQ = lds.sQ;
  auto& sD = lds.sD;
  auto& sPT = lds.sPT;
  auto& sDST = lds.sDST;
  const int tid = threadIdx.x, lane_id = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = a.nchunk[unit];
  const int64_t kb0 = unit * UR;
  const int64_t qrows = a.s_q * H;
  const int drh = wv & 1, dcq = wv >> 1;
  float4_t acc[4][9];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int n = 0; n < 9; ++n) acc[rb][n] = (float4_t){0.f, 0.f, 0.f, 0.f};
  unsigned long long touched0 = 0ull, touched1 = 0ull;

  // Chunk c of the unit: group, and per block its first union entry and the
  // rows the group selects there (wave-uniform: scalar registers).
  const int64_t cu = unit * a.G;
  struct Chunk {
    int g, e0, e1;
    unsigned long long m0, m1;
  };
  auto uni64 = [](unsigned long long m) __attribute__((always_inline)) {
    // readfirstlane returns int: widen through unsigned, not by sign extension
    return (unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)m) |
           ((unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane((unsigned)(m >> 32)) << 32);
  };
  auto chunk = [&](int c) __attribute__((always_inline)) {
    Chunk ch;
    ch.g = __builtin_amdgcn_readfirstlane(a.clist[cu + c].x);
    ch.e0 = __builtin_amdgcn_readfirstlane(a.cbase[2 * (cu + c)]);
    ch.e1 = __builtin_amdgcn_readfirstlane(a.cbase[2 * (cu + c) + 1]);
    ch.m0 = uni64(a.cmask[2 * (cu + c)]);
    ch.m1 = uni64(a.cmask[2 * (cu + c) + 1]);
    return ch;
  };
  Chunk c_cur = chunk(u0 >> 1);                       // chunk of the current sub-chunk
  Chunk c_nxt = chunk(min((u0 >> 1) + 1, nch - 1));   // the chunk after it

  const int pr_row = tid >> 3, pr_part = tid & 7;
  const unsigned long long below = (1ull << pr_row) - 1ull;
  auto pds_load = [&](int g, int e0, unsigned long long m, int half) __attribute__((always_inline)) {
    short8_t v = (short8_t){0, 0, 0, 0, 0, 0, 0, 0};
    if ((m >> pr_row) & 1ull) {
      const int e = min(e0 + __popcll(m & below), (int)a.qcap - 1);
      v = ld16_global(a.pds + ((int64_t)g * a.qcap + e) * (2 * GROUP_ROWS) +
                      (pr_part >> 2) * GROUP_ROWS + DKV_SUB * half + 8 * (pr_part & 3));
    }
    return v;
  };
  auto copies = [&](int g, int u, char* nq, char* nd, int lane) __attribute__((always_inline)) {
    const int64_t row0 = (int64_t)g * GROUP_ROWS + DKV_SUB * (u & 1);
    const int nvalid = (int)max((int64_t)0, min((int64_t)DKV_SUB, qrows - row0));
    gather_seq_rows_nw<DKV_SUB, ROW_CHUNKS, DKV_NW, H>(nq, a.q, row0, nvalid, a.pair_s, a.pair_g, wv, lane);
    gather_seq_rows_nw<DKV_SUB, DO_CHUNKS, DKV_NW, H>(nd, a.dout, row0, nvalid, a.pair_s, a.pair_g, wv, lane);
  };

  copies(c_cur.g, u0, sQ[0], sD[0], lane_id);
  short8_t piece0 = pds_load(c_cur.g, c_cur.e0, c_cur.m0, u0 & 1);
  short8_t piece1 = pds_load(c_cur.g, c_cur.e1, c_cur.m1, u0 & 1);
  for (int u = u0; u < u1; ++u) {
    const int b = (u - u0) & 1;
    const char* sq = sQ[b];
    const char* sd = sD[b];
    wait_vmcnt0();
    __syncthreads();
    {
      unsigned short* st = pr_part < 4 ? sPT : sDST;
      *reinterpret_cast<short8_t*>(st + pt_off(pr_row, pr_part & 3)) = piece0;
      *reinterpret_cast<short8_t*>(st + pt_off(TILE_KV + pr_row, pr_part & 3)) = piece1;
    }
    touched0 |= c_cur.m0;
    touched1 |= c_cur.m1;
    if (u + 1 < u1) {   // the next sub-chunk: its Q / dout copies and its P / dS pieces
      int lane = lane_id;
      asm volatile("" : "+v"(lane));   // offsets recomputed per sub-chunk, not kept live
      const bool adv = (u & 1) != 0;
      const int gn = adv ? c_nxt.g : c_cur.g;
      copies(gn, u + 1, sQ[b ^ 1], sD[b ^ 1], lane);
      piece0 = pds_load(gn, adv ? c_nxt.e0 : c_cur.e0, adv ? c_nxt.m0 : c_cur.m0, (u + 1) & 1);
      piece1 = pds_load(gn, adv ? c_nxt.e1 : c_cur.e1, adv ? c_nxt.m1 : c_cur.m1, (u + 1) & 1);
    }
    __syncthreads();

    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int g16 = lane >> 4, r16 = lane & 15;
    short8_t ad[4], ap[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      ad[rb] = ld16_lds(&sDST[pt_off(64 * drh + 16 * rb + r16, g16)]);
      ap[rb] = ld16_lds(&sPT[pt_off(64 * drh + 16 * rb + r16, g16)]);
    }
    const int col0 = 128 * dcq;
    short8_t bq = ld_bt_rs_lo<DKV_SUB>(sq, 0, col0, lane);
    short8_t bo = ld_bt_rs_lo<DKV_SUB>(sd, 0, col0, lane);
#pragma unroll
    for (int n = 0; n < 9; ++n) {
      short8_t bqn = bq, bon = bo;
      if (n + 1 < 8) {
        bqn = ld_bt_rs_lo<DKV_SUB>(sq, 0, col0 + 16 * (n + 1), lane);
        bon = ld_bt_rs_lo<DKV_SUB>(sd, 0, col0 + 16 * (n + 1), lane);
      } else if (n + 1 == 8) {
        bqn = ld_bt_rs_hi<DKV_SUB>(sq, 0, D_V + 16 * dcq, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb][n] = mfma_bf16(ad[rb], bq, acc[rb][n]);
      if (n < 8) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) acc[rb][n] = mfma_bf16(ap[rb], bo, acc[rb][n]);
      }
      __builtin_amdgcn_sched_barrier(0);
      bq = bqn;
      bo = bon;
    }
    if (u & 1) {   // the next sub-chunk starts chunk u/2 + 1: load the one after it
      c_cur = c_nxt;
      if ((u >> 1) + 2 < nch) c_nxt = chunk((u >> 1) + 2);
    }
  }

  // Partial of the unit (rows 64 drh + 16 rb + 4 g + i); the atomic mode adds
  // it into the accumulator instead, rows of blocks past the last skipped.
  const int g16 = lane_id >> 4, r16 = lane_id & 15;
  if (a.acc32) {
    if (2 * unit + drh < a.NB) {
      float* dst = a.acc32 + (kb0 + 64 * drh + 4 * g16) * D_K + r16;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int n = 0; n < 9; ++n)
            unsafeAtomicAdd(&dst[(16 * rb + i) * D_K + (n < 8 ? 128 * dcq + 16 * n : D_V + 16 * dcq)],
                            acc[rb][n][i]);
    }
  } else {
    float* dst = a.part + (slot * UR + 64 * drh + 4 * g16) * D_K + r16;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 9; ++n)
          dst[(16 * rb + i) * D_K + (n < 8 ? 128 * dcq + 16 * n : D_V + 16 * dcq)] = acc[rb][n][i];
  }
  if (tid == 0) {
    a.ptouch[2 * slot] = touched0;
    a.ptouch[2 * slot + 1] = touched1;
  }
}

// Sub-chunk prefix of the dkv units computed by the calling workgroup (NT
// threads) instead of read from spre / wstart: with few units every
// workgroup redoing the scan costs less than a launch of its own.  Thread t
// sums units [t c, (t + 1) c), c = ceil(NU / NT); a block-wide exclusive scan
// of those sums gives each thread the prefix at its first unit.  Returns the
// total; with wg >= 0 also the unit whose sub-chunks [pre, pre + 2 nchunk)
// hold the first sub-chunk of dkv workgroup wg's range (min(total, wg per),
// per = max(1, ceil(total / DKV_WGS))) and its pre (unit -1 when the range is
// empty); with unit >= 0 the prefix at unit and at unit + 1.
struct UnitScan {
  int total;
  int t_unit, t_pre;   // unit holding workgroup wg's first sub-chunk, and its prefix
  int u_pre, u_end;    // prefix at `unit` and at unit + 1
};
template <int NT>
__device__ __forceinline__ UnitScan dkv_unit_scan(const BwdArgs& a, int wg, int64_t unit, int* red) {
  constexpr int NWV = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t cnt = (a.NU + NT - 1) / NT;
  const int64_t b0 = min<int64_t>(a.NU, tid * cnt), b1 = min<int64_t>(a.NU, b0 + cnt);
  int sum = 0;
  for (int64_t b = b0; b < b1; ++b) sum += 2 * a.nchunk[b];
  const int x = wave_inclusive_scan(sum);
  if (lane == 63) red[wv] = x;
  if (tid == 0) {
    red[NWV] = -1;
    red[NWV + 2] = 0;
    red[NWV + 3] = 0;
  }
  __syncthreads();
  int base = x - sum, total = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    if (w < wv) base += red[w];
    total += red[w];
  }
  const int target = wg >= 0 ? min(total, wg * max(1, (total + DKV_WGS - 1) / DKV_WGS)) : -1;
  if (target >= 0 && target < total && base <= target && target < base + sum) {
    int p = base;
    for (int64_t b = b0; b < b1; ++b) {
      const int v = 2 * a.nchunk[b];
      if (target < p + v) {
        red[NWV] = (int)b;
        red[NWV + 1] = p;
        break;
      }
      p += v;
    }
  }
  if (unit >= b0 && unit < b1) {
    int p = base;
    for (int64_t b = b0; b < unit; ++b) p += 2 * a.nchunk[b];
    red[NWV + 2] = p;
    red[NWV + 3] = p + 2 * a.nchunk[unit];
  }
  __syncthreads();
  UnitScan r;
  r.total = total;
  r.t_unit = red[NWV];
  r.t_pre = red[NWV + 1];
  r.u_pre = red[NWV + 2];
  r.u_end = red[NWV + 3];
  __syncthreads();   // red is reused by the caller
  return r;
}

// The dkv pass: workgroup w takes sub-chunks [w per, (w+1) per) of all
// blocks' sub-chunks in block order (per = ceil(total / DKV_WGS)), as one
// segment per block it meets, starting from block wstart[w] (with few units
// the workgroup finds its start and the prefix itself).
template <int H, bool PDS>
__global__ __launch_bounds__(DKV_NW * 64, 1) void bwd_dkv_kernel(BwdArgs a) {
  __shared__ std::conditional_t<PDS, DkvPairLds, DkvLds> lds;
  __shared__ int red[DKV_NW + 4];
  const bool inl = a.NU <= DKV_INLINE_UNITS;
  int total, per, lo, hi;
  int64_t blk0;
  int sb;
  if (inl) {
    const UnitScan us = dkv_unit_scan<DKV_NW * 64>(a, (int)blockIdx.x, -1, red);
    total = us.total;
    per = max(1, (total + DKV_WGS - 1) / DKV_WGS);
    lo = min(total, (int)blockIdx.x * per);
    hi = min(total, lo + per);
    if (lo >= hi) return;
    blk0 = us.t_unit;
    sb = us.t_pre;
  } else {
    total = a.spre[a.NU];
    per = max(1, (total + DKV_WGS - 1) / DKV_WGS);
    lo = min(total, (int)blockIdx.x * per);
    hi = min(total, lo + per);
    if (lo >= hi) return;
    blk0 = a.wstart[blockIdx.x];
    sb = a.spre[blk0];
  }
  for (int64_t blk = blk0; lo < hi; ++blk) {
    const int se = sb + 2 * a.nchunk[blk];
    if (se <= lo) {   // a block with no records
      sb = se;
      continue;
    }
    const int end = min(hi, se);
    if constexpr (PDS)
      dkv_segment_pair<H>(a, blk, lo - sb, end - sb, (int64_t)blockIdx.x + blk, lds);
    else
      dkv_segment<H>(a, blk, lo - sb, end - sb, (int64_t)blockIdx.x + blk, lds);
    lo = end;
    sb = se;
    __syncthreads();   // the next segment refills the LDS buffers
  }
}

// Sub-chunk prefix over the dkv units (spre[b] = sub-chunks of units before b,
// spre[NU] = total) and the first block of each dkv workgroup's range.  Two
// passes of the same scan: the second finds, for every block, the
// workgroups whose range starts inside it.
__global__ __launch_bounds__(256) void dkv_prefix_kernel(BwdArgs a) {
  __shared__ int scratch[8];
  __shared__ int s_total;
  int base = 0;
  for (int64_t b0 = 0; b0 < a.NU; b0 += 256) {
    const int64_t b = b0 + threadIdx.x;
    const int v = b < a.NU ? 2 * a.nchunk[b] : 0;
    int tot;
    const int pos = base + block_exclusive_scan256(v, scratch, &tot);
    if (b < a.NU) a.spre[b] = pos;
    base += tot;
  }
  if (threadIdx.x == 0) {
    a.spre[a.NU] = base;
    s_total = base;
  }
  __syncthreads();
  const int per = max(1, (s_total + DKV_WGS - 1) / DKV_WGS);
  base = 0;
  for (int64_t b0 = 0; b0 < a.NU; b0 += 256) {
    const int64_t b = b0 + threadIdx.x;
    const int v = b < a.NU ? 2 * a.nchunk[b] : 0;
    int tot;
    const int pos = base + block_exclusive_scan256(v, scratch, &tot);
    if (v > 0)
      for (int w = (pos + per - 1) / per; w < DKV_WGS && w * per < pos + v; ++w) a.wstart[w] = (int)b;
    base += tot;
  }
}

// Writes dkv for FIN_ROWS rows of a block (64 / FIN_ROWS workgroups per
// block): the block's partials added in workgroup order, plus -- only when
// some index row repeats an entry -- the extra slots' contributions, each
// computed directly in (group, slot) order.  Output semantics (bf16, fp32,
// accumulate, rows no slot selects) are applied here.  Bitwise reproducible.
constexpr int FIN_ROWS = 4;
constexpr int FIN_PARTS = TILE_KV / FIN_ROWS;   // workgroups per block
constexpr int FIN_XCAP = 512;   // extra slots listed per pass
constexpr int FIN_XB = 8;       // extra slots per batch
template <int H>
__global__ __launch_bounds__(256) void dkv_finalize_kernel(BwdArgs a) {
  constexpr int T = GROUP_ROWS / H;
  __shared__ float sX[FIN_ROWS * D_K];   // extra-slot contributions of the rows
  __shared__ int red_i[8];
  __shared__ int scr_i[8];
  __shared__ int64_t sXe[FIN_XCAP];      // listed extra slots (union entry index)
  __shared__ float sXc[FIN_XB][D_K];     // a batch's extras: contribution to their row
  __shared__ int sXr[FIN_XB];            // and that row's index among the workgroup's rows
  __shared__ unsigned s_xt;              // rows the extras touch
  const int tid = threadIdx.x;
  const int64_t blk = blockIdx.x / FIN_PARTS;
  const int part = blockIdx.x % FIN_PARTS;
  const int64_t r0 = blk * TILE_KV + FIN_ROWS * part;  // first row of this workgroup
  // The block's unit (the block itself, or its pair in the stored-P form)
  // and the unit's partials: slots w + unit of the workgroups w whose ranges
  // cover its sub-chunks, added in w order.
  const int64_t unit = blk / a.ub;
  const int hb = (int)(blk - unit * a.ub);   // the block's half of the unit
  int total, sb, se;
  if (a.NU <= DKV_INLINE_UNITS) {
    const UnitScan us = dkv_unit_scan<256>(a, -1, unit, red_i);
    total = us.total;
    sb = us.u_pre;
    se = us.u_end;
  } else {
    total = a.spre[a.NU];
    sb = a.spre[unit];
    se = a.spre[unit + 1];
  }
  const int per = max(1, (total + DKV_WGS - 1) / DKV_WGS);
  const int w0 = sb / per;
  const int nsplit = se > sb ? (se - 1) / per - w0 + 1 : 0;
  unsigned long long touched = 0ull;
  for (int sp = 0; sp < nsplit; ++sp) touched |= a.ptouch[2 * (w0 + sp + unit) + hb];
  touched = (touched >> (FIN_ROWS * part)) & ((1ull << FIN_ROWS) - 1ull);

  const bool extras = *a.xtotal > 0;
  if (extras) {
    // Extra slots whose row lies in r0 .. r0 + FIN_ROWS - 1, in (group, slot)
    // order.  Thread t scans groups t, t + 256, ... (a group's extras in slot
    // order); one block scan per round of 256 groups keeps the order.  Up to
    // FIN_XCAP matches are listed per pass (another pass takes the next ones),
    // and handled FIN_XB at a time: one wave per extra forms P and dS of every
    // head and the extra's contribution to its row, summed over the heads;
    // then every thread adds the batch's contributions to its columns in
    // extra order.
    if (tid == 0) s_xt = 0u;
    const int wv = tid >> 6, lane = tid & 63;
    float xa[FIN_ROWS][3];   // the terms of columns tid, tid + 256, tid + 512 (< 576) per row
#pragma unroll
    for (int r = 0; r < FIN_ROWS; ++r)
#pragma unroll
      for (int k = 0; k < 3; ++k) xa[r][k] = 0.f;
    int n_done = 0;
    for (;;) {
      int seen = 0;
      for (int64_t g0 = 0; g0 < a.G; g0 += 256) {
        const int64_t g = g0 + tid;
        int cnt = 0, xc = 0, n_main = 0;
        if (g < a.G) {
          xc = a.xcount[g];
          n_main = a.qcount[g] - xc;
          const int32_t* xr = a.qrow + g * a.qcap + n_main;
          for (int x0 = 0; x0 < xc; x0 += 8) {   // eight loads in flight
            int rr[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) rr[j] = x0 + j < xc ? xr[x0 + j] : -1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int64_t br = rr[j] >= 0 ? kv_block_row(rr[j], a.kvg, a.kvs) : -1;
              cnt += br >= r0 && br < r0 + FIN_ROWS && br < a.s_kv;
            }
          }
        }
        int tot;
        int m = seen + block_exclusive_scan256(cnt, scr_i, &tot);
        if (cnt > 0 && m + cnt > n_done && m < n_done + FIN_XCAP) {
          const int32_t* xr = a.qrow + g * a.qcap + n_main;
          for (int x0 = 0; x0 < xc; x0 += 8) {   // eight loads in flight
            int rr[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) rr[j] = x0 + j < xc ? xr[x0 + j] : -1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int64_t br = rr[j] >= 0 ? kv_block_row(rr[j], a.kvg, a.kvs) : -1;
              if (br >= r0 && br < r0 + FIN_ROWS && br < a.s_kv) {
                if (m >= n_done && m < n_done + FIN_XCAP) {
                  sXe[m - n_done] = g * a.qcap + n_main + x0 + j;
                  atomicOr(&s_xt, 1u << (int)(br - r0));
                }
                ++m;
              }
            }
          }
        }
        seen += tot;
      }
      __syncthreads();
      const int npass = min(FIN_XCAP, seen - n_done);
      for (int b0 = 0; b0 < npass; b0 += FIN_XB) {
        const int nb = min(FIN_XB, npass - b0);
        // Wave w takes extras w, w + 4, ... of the batch.  Eight heads of the
        // extra's token at a time: lane 8 hl + j takes head 8 hp + hl and the
        // 16-byte chunks j + 8 i of its q row (i < 9), dout row (i < 8) and
        // the kv row; the head's 8 lanes reduce q.k and dout.v, giving P and
        // scale * dS; then each chunk's terms dS q + P dout are summed over
        // the 8 heads by lanes 8 apart and added into sXc[e] (head passes in
        // order, so the sum order is fixed).
        for (int e = wv; e < nb; e += 4) {
          const int64_t ent = sXe[b0 + e];
          const int64_t row = a.qrow[ent];
          const int64_t g = ent / a.qcap;
          int64_t t = g * T + (__ffs((unsigned)a.qmask[ent]) - 1);
          t = t < 0 ? 0 : (t >= a.s_q ? a.s_q - 1 : t);
          if (lane == 0) sXr[e] = (int)(kv_block_row(row, a.kvg, a.kvs) - r0);
          const int j = lane & 7, hl = lane >> 3;
          const uint16_t* kr = a.kv + row * D_K + 8 * j;
          for (int hp = 0; hp < H / 8; ++hp) {
            const int h = 8 * hp + hl;
            const int64_t ct = caller_token(t, a.pair_s, a.pair_g);
            const uint16_t* qr = a.q + (ct * H + h) * D_K + 8 * j;
            const uint16_t* dr = a.dout + (ct * H + h) * D_V + 8 * j;
            const float lse2 = a.lse[t * H + h] * LOG2E, dl = a.delta[t * H + h];
            float z = 0.f, dp = 0.f;
#pragma unroll 3
            for (int i = 0; i < 9; ++i) {   // (three chunks' loads in flight: the kernel stays within 128 registers)
              const short8_t kc = ld16_global(kr + 64 * i);
              const short8_t qc = ld16_global(qr + 64 * i);
              short8_t dc = (short8_t){0, 0, 0, 0, 0, 0, 0, 0};
              if (i < 8) dc = ld16_global(dr + 64 * i);
#pragma unroll
              for (int x = 0; x < 8; ++x) {
                const float kx = bf2f((unsigned short)kc[x]);
                z += bf2f((unsigned short)qc[x]) * kx;
                if (i < 8) dp += bf2f((unsigned short)dc[x]) * kx;
              }
            }
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) {
              z += __shfl_xor(z, o);
              dp += __shfl_xor(dp, o);
            }
            const float pv = fast_exp2(z * a.scale_log2 - lse2);
            const float dsv = pv * (dp - dl) * a.scale;
#pragma unroll 3
            for (int i = 0; i < 9; ++i) {
              const short8_t qc = ld16_global(qr + 64 * i);
              short8_t dc = (short8_t){0, 0, 0, 0, 0, 0, 0, 0};
              if (i < 8) dc = ld16_global(dr + 64 * i);
              float cv[8];
#pragma unroll
              for (int x = 0; x < 8; ++x) {
                cv[x] = dsv * bf2f((unsigned short)qc[x]);
                if (i < 8) cv[x] += pv * bf2f((unsigned short)dc[x]);
              }
#pragma unroll
              for (int o = 8; o < 64; o <<= 1)
#pragma unroll
                for (int x = 0; x < 8; ++x) cv[x] += __shfl_xor(cv[x], o);
              if (hl == 0) {
                float* dst = &sXc[e][8 * (j + 8 * i)];
#pragma unroll
                for (int x = 0; x < 8; ++x) dst[x] = hp == 0 ? cv[x] : dst[x] + cv[x];
              }
            }
          }
        }
        __syncthreads();
        for (int e = 0; e < nb; ++e) {   // the batch's terms, in extra order
          const int rl = sXr[e];
#pragma unroll
          for (int r = 0; r < FIN_ROWS; ++r)
            if (rl == r)
#pragma unroll
              for (int k = 0; k < 3; ++k)
                if (tid + 256 * k < D_K) xa[r][k] += sXc[e][tid + 256 * k];
        }
        __syncthreads();
      }
      n_done += npass;
      if (n_done >= seen) break;
    }
#pragma unroll
    for (int r = 0; r < FIN_ROWS; ++r)
#pragma unroll
      for (int k = 0; k < 3; ++k)
        if (tid + 256 * k < D_K) sX[r * D_K + tid + 256 * k] = xa[r][k];
    touched |= (unsigned long long)s_xt;
    __syncthreads();
  }

  // Atomic mode: one source, the accumulator's rows of the block.
  const int64_t unit_rows = (int64_t)TILE_KV * a.ub;
  const float* src = a.acc32 ? a.acc32 + (blk * TILE_KV + FIN_ROWS * part) * D_K
                             : a.part + ((w0 + unit) * unit_rows + TILE_KV * hb + FIN_ROWS * part) * D_K;
  const int nsrc = a.acc32 ? (nsplit > 0 ? 1 : 0) : nsplit;
  constexpr int N4 = FIN_ROWS * D_K / 4;  // float4 elements of the rows
  constexpr int EPT = (N4 + 255) / 256;   // elements per thread
  const int64_t SPLIT = unit_rows * D_K;
  // Partials summed left to right in workgroup order.  All of a thread's
  // elements load their partials together, eight partials per round
  // (indices clamped into range, extra loads unused).  A block no record
  // touches has no partial: zeros.
  float4_t vs[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = min(tid + 256 * k, N4 - 1);
    vs[k] = nsrc > 0 ? *reinterpret_cast<const float4_t*>(src + 4 * e) : (float4_t){0.f, 0.f, 0.f, 0.f};
  }
  for (int sp = 1; sp < nsrc; sp += 8) {
    float4_t pp[EPT][8];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const float* pe = src + 4 * min(tid + 256 * k, N4 - 1);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pp[k][j] = *reinterpret_cast<const float4_t*>(pe + min(sp + j, nsrc - 1) * SPLIT);
    }
#pragma unroll
    for (int k = 0; k < EPT; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (sp + j < nsrc) vs[k] += pp[k][j];
  }
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int e = tid + 256 * k;
    if (e >= N4) break;
    float4_t v = vs[k];
    if (extras) v += *reinterpret_cast<const float4_t*>(sX + 4 * e);
    const int kvl = (4 * e) / D_K;
    const int col = (4 * e) % D_K;
    if (r0 + kvl >= a.s_kv) continue;
    const int64_t row = kv_flat_row(r0 + kvl, a.kvg, a.kvs);
    const bool hit = (touched >> kvl) & 1ull;
    if (a.dkv_f32) {
      float4_t* d = reinterpret_cast<float4_t*>(a.dkv_f32 + row * D_K + col);
      if (a.accumulate) {
        const float4_t old = *d;
        if (hit) {
          v = old + v;
          *d = v;
        } else {
          v = old;
        }
      } else {
        *d = v;
      }
    }
    if (a.dkv) {
      uint2 b;
      b.x = pack_bf2(v[0], v[1]);
      b.y = pack_bf2(v[2], v[3]);
      *reinterpret_cast<uint2*>(a.dkv + row * D_K + col) = b;
    }
  }
}

}  // namespace

hipError_t launch_bwd_dq(const BwdArgs& a, int heads, hipStream_t stream) {
  if (a.G == 0) return hipSuccess;
  dim3 grid((unsigned)(a.NU + a.G)), block(DQ_NW * 64);   // NU schedule workgroups, then the groups
  switch (heads) {
    case 8: bwd_dq_kernel<8><<<grid, block, 0, stream>>>(a); break;
    case 16: bwd_dq_kernel<16><<<grid, block, 0, stream>>>(a); break;
    case 32: bwd_dq_kernel<32><<<grid, block, 0, stream>>>(a); break;
    case 64: bwd_dq_kernel<64><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dkv_schedule(const BwdArgs& a, bool lists_built, hipStream_t stream) {
  if (a.NB == 0) return hipSuccess;
  if (!lists_built) {   // no dq launch built them (an empty query batch)
    dkv_schedule_kernel<<<dim3((unsigned)a.NU), dim3(256), 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.NU <= DKV_INLINE_UNITS) return hipSuccess;   // the dkv and finalize kernels scan themselves
  dkv_prefix_kernel<<<dim3(1), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkv(const BwdArgs& a, int heads, hipStream_t stream) {
  if (a.NB == 0) return hipSuccess;
  const dim3 grid((unsigned)DKV_WGS), block(DKV_NW * 64);
  const bool pds = a.pds != nullptr;
  switch (heads) {
    case 8: pds ? bwd_dkv_kernel<8, true><<<grid, block, 0, stream>>>(a)
                : bwd_dkv_kernel<8, false><<<grid, block, 0, stream>>>(a); break;
    case 16: pds ? bwd_dkv_kernel<16, true><<<grid, block, 0, stream>>>(a)
                 : bwd_dkv_kernel<16, false><<<grid, block, 0, stream>>>(a); break;
    case 32: pds ? bwd_dkv_kernel<32, true><<<grid, block, 0, stream>>>(a)
                 : bwd_dkv_kernel<32, false><<<grid, block, 0, stream>>>(a); break;
    case 64: pds ? bwd_dkv_kernel<64, true><<<grid, block, 0, stream>>>(a)
                 : bwd_dkv_kernel<64, false><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dkv_finalize(const BwdArgs& a, int heads, hipStream_t stream) {
  if (a.NB == 0) return hipSuccess;
  const dim3 grid((unsigned)(a.NB * FIN_PARTS)), block(256);
  switch (heads) {
    case 8: dkv_finalize_kernel<8><<<grid, block, 0, stream>>>(a); break;
    case 16: dkv_finalize_kernel<16><<<grid, block, 0, stream>>>(a); break;
    case 32: dkv_finalize_kernel<32><<<grid, block, 0, stream>>>(a); break;
    case 64: dkv_finalize_kernel<64><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace smla
