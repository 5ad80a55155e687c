// Sparse-MLA forward (gfx950): out = softmax(scale q.k) v over each token's
// selected KV rows, and the natural-log LSE per (token, head).
//
// One workgroup (4 waves) owns a query group: T = 64/H consecutive tokens,
// 64 query rows.  It walks the union of the group's selected KV rows in tiles
// of 64 rows, gathered into LDS with direct global->LDS copies (double
// buffered).  Per tile:
//   scores   wave w: rows 16w..16w+15 x 64 kv  (Q fragments in registers,
//            K read from LDS), 72 MFMA 16x16x32;
//   softmax  per row, base-2 exponent with scale*log2(e) folded in; entries
//            the row's token did not select get P = 0 by select;
//   PV       wave w: all 64 rows x output columns 128w..128w+127, V read once
//            per workgroup through transposing LDS reads, 64 MFMA.
// The running max starts at a finite -1e30, so a tile with no valid entry
// never forms exp(-inf - -inf); the final denominator is floored at 1e-30,
// a no-op on rows with a valid slot (their largest term is exp(0) = 1) that
// makes an all-padding row output exact zeros with LSE = ln(1e-30).  The
// floor and the exact-zero padding follow miles PR #2079 ("fix GLM-5
// sparse-MLA kernel -1 index OOB and NaN gradients", 实现拆解 item 2 and the
// forward key code snippet); padding rows of a tile are copied from a zero
// chunk, never from an address computed from -1.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

template <int H>
__global__ __launch_bounds__(256, 1) void fwd_kernel(FwdArgs a) {
  constexpr int T = GROUP_ROWS / H;
  // Double-buffered kv tiles: the next tile is copied while this one is used.
  __shared__ __attribute__((aligned(16))) char sK[2][KV64_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned short sP[GROUP_ROWS * 72];
  __shared__ __attribute__((aligned(16))) unsigned char sMask[2][256];   // token masks (copied as words)
  __shared__ __attribute__((aligned(16))) int sRow[2][64];   // kv row indices of a tile's entries
  __shared__ float sAlpha[GROUP_ROWS];
  __shared__ float sL[GROUP_ROWS];
  __shared__ int sRescale[4];   // per wave: some row of the wave moved its max

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int64_t grp = a.order[blockIdx.x];
  const int64_t t0 = grp * T;
  const int n_ent = a.qcount[grp];
  const int32_t* erow = a.qrow + grp * a.qcap;
  const uint8_t* emask = a.qmask + grp * a.qcap;
  const int ntiles = (n_ent + TILE_KV - 1) / TILE_KV;

  // Q fragments (A operand) of rows 16*wave + r16.
  short8_t qf[18];
  {
    const int rr = 16 * wave + r16;
    const int64_t tok = t0 + rr / H;
    if (tok < a.s_q) {
      const uint16_t* qrow = a.q + (tok * H + rr % H) * D_K + 8 * g16;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[ks] = ld16_global(qrow + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[ks] = (short8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  // Scores are computed transposed (S^T = K Q^T): lane (g, r) of wave w holds
  // row 16w + r of the group and kv entries 16nt + 4g + i.  Softmax state is
  // per lane (one row; the four lanes g = 0..3 of a row agree).
  const int tl = (16 * wave + r16) / H;  // group-local token of this lane's row
  // m_run is the max the probabilities are taken against: it only moves when
  // a row max exceeds it by more than RESCALE_SLACK (log2 units), so most
  // tiles need no rescaling of acc; p = exp2(z - m_run) <= 2^RESCALE_SLACK.
  float m_run = M_INIT, lsum = 0.f;
  float4_t acc[4][8];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[rb][n] = (float4_t){0.f, 0.f, 0.f, 0.f};

  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lane_id = lane;
  // kv rows of a tile (count entries at rows_t in LDS) into a swizzled tile:
  // 64 row copies and 8 tail copies, 18 per wave.
  auto gather = [&](char* kbuf, const int* rows_t, int count) __attribute__((always_inline)) {
    gather_kv_rows<TILE_KV, ROW_CHUNKS>(kbuf, a.kv, a.s_kv, rows_t, count, wv, lane_id);
  };
  // Tile t's kv rows are copied from rows_t (LDS); masks of tile t and row
  // indices of tile t+1 follow by direct copies, so nothing the copies need is
  // read from global memory between them.
  auto issue = [&](int tile, char* kbuf, const int* rows_t, unsigned char* mbuf, int* rows_t2) __attribute__((always_inline)) {
    gather(kbuf, rows_t, min(TILE_KV, n_ent - tile * TILE_KV));
    copy_union_entries(nullptr, mbuf, erow, emask, tile * TILE_KV, n_ent, TILE_KV, wv, 1, 1, lane);
    if (tile + 1 < ntiles)
      copy_union_entries(rows_t2, nullptr, erow, emask, (tile + 1) * TILE_KV, n_ent, TILE_KV, wv,
                         2, 2, lane);
  };

  // One tile: kt/mk hold it, knext/mnext receive the prefetch of the next.
  auto step = [&](int tile, const char* kt, const unsigned char* mkb, char* knext,
                  unsigned char* mnext, const int* rnext, int* rcur) __attribute__((always_inline)) {
    wait_vmcnt0();
    __syncthreads();
    // Prefetch the next tile into the other buffer (free: every wave has
    // passed the barrier above, so the previous tile's reads are done).
    if (tile + 1 < ntiles) issue(tile + 1, knext, rnext, mnext, rcur);
    // Lane-derived LDS offsets are recomputed per tile from an opaque copy of
    // the lane id rather than held in registers across the tile loop.
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int g16 = lane >> 4, r16 = lane & 15, wave = wv;
    float4_t s[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) s[nt] = (float4_t){0.f, 0.f, 0.f, 0.f};
    // K fragments one k-step ahead of the MFMAs that use them; the
    // scheduling barriers keep the compiler from sinking the reads onto
    // their uses (which serialises every read with its MFMA).
    short8_t kc[4], kn[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) kc[nt] = ld_b_rs<TILE_KV>(kt, nt * 16, 0, lane);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (ks + 1 < 18) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) kn[nt] = ld_b_rs<TILE_KV>(kt, nt * 16, 32 * (ks + 1), lane);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) s[nt] = mfma_bf16(kc[nt], qf[ks], s[nt]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) kc[nt] = kn[nt];
    }

    // Online softmax of this lane's row over the tile's 64 entries.
    float mx = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const unsigned mk = *reinterpret_cast<const unsigned*>(mkb + nt * 16 + 4 * g16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = (mk >> (8 * i + tl)) & 1u;
        const float x = v ? s[nt][i] * a.scale_log2 : -INFINITY;
        s[nt][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool move = mx > m_run + RESCALE_SLACK;
    float alpha = 1.f;
    if (move) {
      alpha = fast_exp2(m_run - mx);
      m_run = mx;
    }
    float rs = 0.f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(s[nt][i] - m_run);
        rs += p[i];
      }
      uint2 pk;
      pk.x = pack_bf2(p[0], p[1]);
      pk.y = pack_bf2(p[2], p[3]);
      *reinterpret_cast<uint2*>(&sP[(16 * wave + r16) * 72 + nt * 16 + 4 * g16]) = pk;
    }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    lsum = lsum * alpha + rs;
    if (g16 == 0) sAlpha[16 * wave + r16] = alpha;
    const bool wave_moved = __ballot(move) != 0ull;
    if (lane == 0) sRescale[wave] = wave_moved ? 1 : 0;
    __syncthreads();

    // PV: this wave's 128 output columns for all 64 rows.
    if (sRescale[0] | sRescale[1] | sRescale[2] | sRescale[3]) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = sAlpha[16 * rb + 4 * g16 + i];
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][n][i] *= al[i];
      }
    }
    short8_t pa[4][2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        pa[rb][k2] = ld16_lds(&sP[(16 * rb + r16) * 72 + 32 * k2 + 8 * g16]);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int col = 128 * wave + 16 * n;
      const short8_t b0 = ld_bt_rs_lo<TILE_KV>(kt, 0, col, lane);
      const short8_t b1 = ld_bt_rs_lo<TILE_KV>(kt, 32, col, lane);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        acc[rb][n] = mfma_bf16(pa[rb][0], b0, acc[rb][n]);
        acc[rb][n] = mfma_bf16(pa[rb][1], b1, acc[rb][n]);
      }
    }
  };

  if (ntiles > 0) {
    copy_union_entries(sRow[0], sMask[0], erow, emask, 0, n_ent, TILE_KV, wv, 0, 1, lane);
    if (ntiles > 1) copy_union_entries(sRow[1], nullptr, erow, emask, TILE_KV, n_ent, TILE_KV, wv, 2, 2, lane);
    wait_vmcnt0();
    __syncthreads();
    gather(sK[0], sRow[0], min(TILE_KV, n_ent));
  }
  for (int tile = 0; tile < ntiles; ++tile) {
    const int b = tile & 1;
    step(tile, sK[b], sMask[b], sK[b ^ 1], sMask[b ^ 1], sRow[b ^ 1], sRow[b]);
  }

  // Epilogue: LSE from the row owners, then normalised output through LDS.
  __syncthreads();
  if (g16 == 0) {
    const int rr = 16 * wave + r16;
    sL[rr] = lsum;
    const int64_t tok = t0 + rr / H;
    if (tok < a.s_q) {
      const float m_eff = lsum > 0.f ? m_run : 0.f;
      a.lse[tok * H + rr % H] = (m_eff + fast_log2(fmaxf(lsum, SUMEXP_FLOOR))) * LN2;
    }
  }
  __syncthreads();
  unsigned short* so = reinterpret_cast<unsigned short*>(sK[0]);  // [64][520]
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) inv[i] = 1.0f / fmaxf(sL[16 * rb + 4 * g16 + i], SUMEXP_FLOOR);
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        so[(16 * rb + 4 * g16 + i) * 520 + 128 * wave + 16 * n + r16] = f2bf(acc[rb][n][i] * inv[i]);
  }
  __syncthreads();
  for (int p = tid; p < GROUP_ROWS * 64; p += 256) {
    const int row = p >> 6, c = p & 63;
    const int64_t tok = t0 + row / H;
    if (tok < a.s_q)
      *reinterpret_cast<uint4_t*>(a.out + (tok * H + row % H) * D_V + 8 * c) =
          *reinterpret_cast<const uint4_t*>(so + row * 520 + 8 * c);
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int heads, hipStream_t stream) {
  if (a.G == 0) return hipSuccess;
  dim3 grid((unsigned)a.G), block(256);
  switch (heads) {
    case 8: fwd_kernel<8><<<grid, block, 0, stream>>>(a); break;
    case 16: fwd_kernel<16><<<grid, block, 0, stream>>>(a); break;
    case 32: fwd_kernel<32><<<grid, block, 0, stream>>>(a); break;
    case 64: fwd_kernel<64><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace smla
