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
  __shared__ __attribute__((aligned(16))) char sK[2][kv_tile_bytes(TILE_KV)];
  __shared__ __attribute__((aligned(16))) unsigned short sP[GROUP_ROWS * 72];
  __shared__ __attribute__((aligned(16))) unsigned char sMask[2][256];   // token masks (copied as words)
  __shared__ __attribute__((aligned(16))) int sRow[2][64];   // kv row indices of a tile's entries
  __shared__ float sAlpha[GROUP_ROWS];
  __shared__ float sL[GROUP_ROWS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int64_t grp = blockIdx.x;
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
  int tl[4];  // group-local token of this lane's C-fragment rows
#pragma unroll
  for (int i = 0; i < 4; ++i) tl[i] = (16 * wave + 4 * g16 + i) / H;

  float m2[4], lsum[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m2[i] = M_INIT;
    lsum[i] = 0.f;
  }
  float4_t acc[4][8];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[rb][n] = (float4_t){0.f, 0.f, 0.f, 0.f};

  // 64 rows x 73 chunks (72 data + 1 pad) = 73 copies of 64 lanes x 16 bytes.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // Tile t's kv rows are copied from rows_t (LDS); masks of tile t+1 and row
  // indices of tile t+2 follow by direct copies, so nothing the copies need is
  // read from global memory between them.
  auto issue = [&](int tile, char* kbuf, const int* rows_t, unsigned char* mbuf, int* rows_t2) __attribute__((always_inline)) {
    gather_kv_tile<TILE_KV>(kbuf, a.kv, a.s_kv, rows_t, min(TILE_KV, n_ent - tile * TILE_KV), wv,
                            lane);
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
    float4_t s[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) s[nt] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const short8_t b = ld16_lds(kt + (nt * 16 + r16) * TILE_STRIDE + (4 * ks + g16) * 16);
        s[nt] = mfma_bf16(qf[ks], b, s[nt]);
      }
    }

    int mk[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) mk[nt] = mkb[nt * 16 + r16];
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bool v = (mk[nt] >> tl[i]) & 1;
        const float x = v ? s[nt][i] * a.scale_log2 : -INFINITY;
        s[nt][i] = x;
        mx = fmaxf(mx, x);
      }
      mx = max16(mx);
      const float mn = fmaxf(m2[i], mx);
      alpha[i] = fast_exp2(m2[i] - mn);
      m2[i] = mn;
      float rs = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float p = fast_exp2(s[nt][i] - mn);
        s[nt][i] = p;
        rs += p;
      }
      lsum[i] = lsum[i] * alpha[i] + sum16(rs);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sP[(16 * wave + 4 * g16 + i) * 72 + nt * 16 + r16] = f2bf(s[nt][i]);
    if (r16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sAlpha[16 * wave + 4 * g16 + i] = alpha[i];
    }
    __syncthreads();

    // PV: this wave's 128 output columns for all 64 rows.
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
    short8_t pa[4][2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        pa[rb][k2] = ld16_lds(&sP[(16 * rb + r16) * 72 + 32 * k2 + 8 * g16]);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int col = 128 * wave + 16 * n;
      const short8_t b0 = ld_b_tr(kt, TILE_STRIDE, 0, col, lane);
      const short8_t b1 = ld_b_tr(kt, TILE_STRIDE, 32, col, lane);
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
    gather_kv_tile<TILE_KV>(sK[0], a.kv, a.s_kv, sRow[0], min(TILE_KV, n_ent), wv, lane);
  }
  for (int tile = 0; tile < ntiles; ++tile) {
    const int b = tile & 1;
    step(tile, sK[b], sMask[b], sK[b ^ 1], sMask[b ^ 1], sRow[b ^ 1], sRow[b]);
  }

  // Epilogue: LSE from the row owners, then normalised output through LDS.
  __syncthreads();
  if (r16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * wave + 4 * g16 + i;
      sL[rr] = lsum[i];
      const int64_t tok = t0 + rr / H;
      if (tok < a.s_q) {
        const float m_eff = lsum[i] > 0.f ? m2[i] : 0.f;
        a.lse[tok * H + rr % H] = (m_eff + fast_log2(fmaxf(lsum[i], SUMEXP_FLOOR))) * LN2;
      }
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
