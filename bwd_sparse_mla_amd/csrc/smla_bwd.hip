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
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

// ---------------------------------------------------------------------------
// dq pass
// ---------------------------------------------------------------------------
template <int H>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int T = GROUP_ROWS / H;
  __shared__ __attribute__((aligned(16))) char sK[2][TILE_KV * TILE_STRIDE];
  __shared__ __attribute__((aligned(16))) unsigned short sdS[GROUP_ROWS * 72];
  __shared__ int sMask[2][TILE_KV];
  __shared__ float sDelta[GROUP_ROWS];
  __shared__ float sLse2[GROUP_ROWS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int64_t grp = blockIdx.x;
  const int64_t t0 = grp * T;
  const int n_ent = a.qcount[grp];
  const int32_t* erow = a.qrow + grp * a.qcap;
  const uint8_t* emask = a.qmask + grp * a.qcap;
  const int ntiles = (n_ent + TILE_KV - 1) / TILE_KV;

  // delta = rowsum(dout * out) for the group's 64 rows (4 threads per row).
  {
    const int row = tid >> 2, part = tid & 3;
    const int64_t tok = t0 + row / H;
    float d = 0.f;
    if (tok < a.s_q) {
      const int64_t o = (tok * H + row % H) * D_V + 128 * part;
#pragma unroll 4
      for (int c = 0; c < 16; ++c) {
        const short8_t x = ld16_global(a.dout + o + 8 * c);
        const short8_t y = ld16_global(a.out + o + 8 * c);
#pragma unroll
        for (int j = 0; j < 8; ++j) d += bf2f((unsigned short)x[j]) * bf2f((unsigned short)y[j]);
      }
    }
    d += __shfl_xor(d, 1);
    d += __shfl_xor(d, 2);
    if (part == 0) {
      sDelta[row] = d;
      float l2 = 0.f;
      if (tok < a.s_q) {
        a.delta[tok * H + row % H] = d;
        l2 = a.lse[tok * H + row % H] * LOG2E;
      }
      sLse2[row] = l2;
    }
  }

  short8_t qf[18], dof[16];
  {
    const int rr = 16 * wave + r16;
    const int64_t tok = t0 + rr / H;
    if (tok < a.s_q) {
      const uint16_t* qrow = a.q + (tok * H + rr % H) * D_K + 8 * g16;
      const uint16_t* drow = a.dout + (tok * H + rr % H) * D_V + 8 * g16;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[ks] = ld16_global(qrow + 32 * ks);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) dof[ks] = ld16_global(drow + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) qf[ks] = (short8_t){0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) dof[ks] = (short8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  __syncthreads();
  int tl[4];
  float del[4], ls2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = 16 * wave + 4 * g16 + i;
    tl[i] = rr / H;
    del[i] = sDelta[rr];
    ls2[i] = sLse2[rr];
  }

  float4_t acc[4][9];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int n = 0; n < 9; ++n) acc[rb][n] = (float4_t){0.f, 0.f, 0.f, 0.f};

  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int tile, int buf) {
    gather_kv_tile<TILE_KV>(sK[buf], a.kv, a.s_kv, erow, tile * TILE_KV,
                            min(TILE_KV, n_ent - tile * TILE_KV), wv, lane);
    if (tid < TILE_KV) {
      const int e = tile * TILE_KV + tid;
      sMask[buf][tid] = e < n_ent ? (int)emask[e] : 0;
    }
  };

  if (ntiles > 0) issue(0, 0);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    wait_vmcnt0();
    __syncthreads();
    const char* kt = sK[buf];

    float4_t s[4], dp[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      s[nt] = (float4_t){0.f, 0.f, 0.f, 0.f};
      dp[nt] = (float4_t){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const short8_t b = ld16_lds(kt + (nt * 16 + r16) * TILE_STRIDE + (4 * ks + g16) * 16);
        s[nt] = mfma_bf16(qf[ks], b, s[nt]);
        if (ks < 16) dp[nt] = mfma_bf16(dof[ks], b, dp[nt]);
      }
    }
    if (tile + 1 < ntiles) issue(tile + 1, buf ^ 1);

#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int mk = sMask[buf][nt * 16 + r16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = (mk >> tl[i]) & 1;
        const float p = v ? fast_exp2(s[nt][i] * a.scale_log2 - ls2[i]) : 0.f;
        const float ds = p * (dp[nt][i] - del[i]);
        sdS[(16 * wave + 4 * g16 + i) * 72 + nt * 16 + r16] = f2bf(ds);
      }
    }
    __syncthreads();

    short8_t da[4][2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        da[rb][k2] = ld16_lds(&sdS[(16 * rb + r16) * 72 + 32 * k2 + 8 * g16]);
#pragma unroll
    for (int n = 0; n < 9; ++n) {
      const int col = 144 * wave + 16 * n;
      const short8_t b0 = ld_b_tr(kt, TILE_STRIDE, 0, col, lane);
      const short8_t b1 = ld_b_tr(kt, TILE_STRIDE, 32, col, lane);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        acc[rb][n] = mfma_bf16(da[rb][0], b0, acc[rb][n]);
        acc[rb][n] = mfma_bf16(da[rb][1], b1, acc[rb][n]);
      }
    }
  }

  // Epilogue: dq = scale * acc through LDS, 16-byte stores.
  __syncthreads();
  unsigned short* so = reinterpret_cast<unsigned short*>(sK[0]);  // [64][584]
  constexpr int SO = TILE_STRIDE / 2;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int n = 0; n < 9; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        so[(16 * rb + 4 * g16 + i) * SO + 144 * wave + 16 * n + r16] = f2bf(acc[rb][n][i] * a.scale);
  __syncthreads();
  for (int p = tid; p < GROUP_ROWS * ROW_CHUNKS; p += 256) {
    const int row = p / ROW_CHUNKS, c = p - row * ROW_CHUNKS;
    const int64_t tok = t0 + row / H;
    if (tok < a.s_q)
      *reinterpret_cast<uint4_t*>(a.dq + (tok * H + row % H) * D_K + 8 * c) =
          *reinterpret_cast<const uint4_t*>(so + row * SO + 8 * c);
  }
}

// ---------------------------------------------------------------------------
// dkv pass
// ---------------------------------------------------------------------------
template <int H>
__global__ __launch_bounds__(256, 1) void bwd_dkv_kernel(BwdArgs a) {
  constexpr int T = GROUP_ROWS / H;   // token slots per chunk = tokens per group
  __shared__ __attribute__((aligned(16))) char sQ[GROUP_ROWS * TILE_STRIDE];
  __shared__ __attribute__((aligned(16))) char sDO[GROUP_ROWS * DO_STRIDE];
  __shared__ __attribute__((aligned(16))) unsigned short sPT[TILE_KV * 72];
  __shared__ __attribute__((aligned(16))) unsigned short sDST[TILE_KV * 72];
  __shared__ int2 sTab[256];
  __shared__ unsigned long long sMask[T];
  __shared__ int sTok[T];
  __shared__ float sLse2[GROUP_ROWS];
  __shared__ float sDel[GROUP_ROWS];
  __shared__ int scratch[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g16 = lane >> 4, r16 = lane & 15;
  const int64_t blk = blockIdx.x;
  const int64_t kb0 = blk * TILE_KV;

  // This wave's 16 kv rows as A fragments (K for S^T; their first 512
  // columns, ks < 16, are V for dP^T).
  short8_t kf[18];
  {
    const int64_t row = kb0 + 16 * wave + r16;
    if (row < a.s_kv) {
      const uint16_t* kr = a.kv + row * D_K + 8 * g16;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) kf[ks] = ld16_global(kr + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) kf[ks] = (short8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  float4_t acc[4][9];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int n = 0; n < 9; ++n) acc[rb][n] = (float4_t){0.f, 0.f, 0.f, 0.f};
  unsigned long long touched = 0ull;

  // One chunk: up to T token slots (sTok/sMask filled, cnt slots valid).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // Token of a chunk slot, clamped into [0, s_q) before it forms an address.
  auto slot_token = [&](int slot) -> int64_t {
    int64_t t = sTok[slot];
    return t < 0 ? 0 : (t >= a.s_q ? a.s_q - 1 : t);
  };
  auto process_chunk = [&](int cnt) {
    // Q rows of the chunk: 64 rows x 73 chunks = 73 copies; dO: 64 x 65 = 65.
#pragma unroll
    for (int j = 0; j < (TILE_STRIDE_CHUNKS + 3) / 4; ++j) {
      const int i = wv + 4 * j;
      if (i < TILE_STRIDE_CHUNKS) {
        const int p = i * 64 + lane;
        const int row = p / TILE_STRIDE_CHUNKS, c = p - row * TILE_STRIDE_CHUNKS;
        const int slot = row / H;
        const void* src = g_zero16;
        if (c < ROW_CHUNKS && slot < cnt)
          src = a.q + (slot_token(slot) * H + row % H) * D_K + 8 * c;
        g2lds16(src, sQ + i * 1024);
      }
    }
#pragma unroll
    for (int j = 0; j < (DO_STRIDE_CHUNKS + 3) / 4; ++j) {
      const int i = wv + 4 * j;
      if (i < DO_STRIDE_CHUNKS) {
        const int p = i * 64 + lane;
        const int row = p / DO_STRIDE_CHUNKS, c = p - row * DO_STRIDE_CHUNKS;
        const int slot = row / H;
        const void* src = g_zero16;
        if (c < DO_CHUNKS && slot < cnt)
          src = a.dout + (slot_token(slot) * H + row % H) * D_V + 8 * c;
        g2lds16(src, sDO + i * 1024);
      }
    }
    if (tid < GROUP_ROWS) {
      const int slot = tid / H;
      float l2 = 0.f, dl = 0.f;
      if (slot < cnt) {
        const int64_t r = slot_token(slot) * H + tid % H;
        l2 = a.lse[r] * LOG2E;
        dl = a.delta[r];
      }
      sLse2[tid] = l2;
      sDel[tid] = dl;
    }
    wait_vmcnt0();
    __syncthreads();

    float4_t st[4], dpt[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      st[nt] = (float4_t){0.f, 0.f, 0.f, 0.f};
      dpt[nt] = (float4_t){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const short8_t b = ld16_lds(sQ + (nt * 16 + r16) * TILE_STRIDE + (4 * ks + g16) * 16);
        st[nt] = mfma_bf16(kf[ks], b, st[nt]);
        if (ks < 16) {
          const short8_t b2 = ld16_lds(sDO + (nt * 16 + r16) * DO_STRIDE + (4 * ks + g16) * 16);
          dpt[nt] = mfma_bf16(kf[ks], b2, dpt[nt]);
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int q = nt * 16 + r16;
      const int slot = q / H;
      const unsigned long long m = slot < cnt ? sMask[slot] : 0ull;
      const float l2 = sLse2[q], dl = sDel[q];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kvl = 16 * wave + 4 * g16 + i;
        const bool v = (m >> kvl) & 1ull;
        const float p = v ? fast_exp2(st[nt][i] * a.scale_log2 - l2) : 0.f;
        const float ds = p * (dpt[nt][i] - dl) * a.scale;
        sPT[kvl * 72 + q] = f2bf(p);
        sDST[kvl * 72 + q] = f2bf(ds);
      }
    }
    __syncthreads();

    short8_t ad[4][2], ap[4][2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        ad[rb][k2] = ld16_lds(&sDST[(16 * rb + r16) * 72 + 32 * k2 + 8 * g16]);
        ap[rb][k2] = ld16_lds(&sPT[(16 * rb + r16) * 72 + 32 * k2 + 8 * g16]);
      }
#pragma unroll
    for (int n = 0; n < 9; ++n) {
      const int col = 144 * wave + 16 * n;
      const short8_t bq0 = ld_b_tr(sQ, TILE_STRIDE, 0, col, lane);
      const short8_t bq1 = ld_b_tr(sQ, TILE_STRIDE, 32, col, lane);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        acc[rb][n] = mfma_bf16(ad[rb][0], bq0, acc[rb][n]);
        acc[rb][n] = mfma_bf16(ad[rb][1], bq1, acc[rb][n]);
      }
      if (col < D_V) {
        const short8_t bo0 = ld_b_tr(sDO, DO_STRIDE, 0, col, lane);
        const short8_t bo1 = ld_b_tr(sDO, DO_STRIDE, 32, col, lane);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          acc[rb][n] = mfma_bf16(ap[rb][0], bo0, acc[rb][n]);
          acc[rb][n] = mfma_bf16(ap[rb][1], bo1, acc[rb][n]);
        }
      }
    }
    __syncthreads();  // sQ / sDO / sPT / sDST are refilled by the next chunk
  };

  // Records of this block, group by group (ascending group, then token).
  for (int64_t gb = 0; gb < a.G; gb += 256) {
    if (gb + tid < a.G) sTab[tid] = a.ktab[blk * a.G + gb + tid];
    else sTab[tid] = make_int2(0, 0);
    __syncthreads();
    const int ng = (int)min<int64_t>(256, a.G - gb);
    for (int j = 0; j < ng; ++j) {
      const int2 e = sTab[j];
      if (e.y == 0) continue;
      const int64_t base = (gb + j) * a.rcap + e.x;
      if (tid < e.y) {
        sTok[tid] = a.krtok[base + tid];
        sMask[tid] = a.krmask[base + tid];
      }
      __syncthreads();
      for (int c = 0; c < e.y; ++c) touched |= sMask[c];
      process_chunk(e.y);
    }
    __syncthreads();  // sTab is reloaded
  }

  // Repeated slots (rare): one single-row record each, in group/slot order.
  if (*a.xtotal > 0) {
    int fill = 0;
    for (int64_t g = 0; g < a.G; ++g) {
      const int xc = a.xcount[g];
      if (xc == 0) continue;
      const int n_main = a.qcount[g] - xc;
      const int32_t* xrow = a.qrow + g * a.qcap + n_main;
      const uint8_t* xmask = a.qmask + g * a.qcap + n_main;
      for (int x0 = 0; x0 < xc; x0 += 256) {
        const int x = x0 + tid;
        int match = 0, tok = 0;
        unsigned long long bit = 0ull;
        if (x < xc) {
          const int64_t row = xrow[x];
          if (row >= kb0 && row < kb0 + TILE_KV) {
            match = 1;
            tok = (int)(g * T + (__ffs((unsigned)xmask[x]) - 1));
            bit = 1ull << (row - kb0);
          }
        }
        int total;
        const int pos = block_exclusive_scan256(match, scratch, &total);
        for (int done = 0; done < total;) {
          const int take = min(T - fill, total - done);
          if (match && pos >= done && pos < done + take) {
            sTok[fill + pos - done] = tok;
            sMask[fill + pos - done] = bit;
          }
          fill += take;
          done += take;
          __syncthreads();
          if (fill == T) {
            for (int c = 0; c < T; ++c) touched |= sMask[c];
            process_chunk(T);
            fill = 0;
          }
        }
      }
    }
    if (fill > 0) {
      for (int c = 0; c < fill; ++c) touched |= sMask[c];
      process_chunk(fill);
    }
  }

  // Epilogue: each dkv row of the block is written once.
  unsigned short* so = reinterpret_cast<unsigned short*>(sQ);  // [64][584]
  constexpr int SO = TILE_STRIDE / 2;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kvl = 16 * rb + 4 * g16 + i;
      const int64_t row = kb0 + kvl;
      const bool hit = (touched >> kvl) & 1ull;
#pragma unroll
      for (int n = 0; n < 9; ++n) {
        const int col = 144 * wave + 16 * n + r16;
        float v = acc[rb][n][i];
        if (row < a.s_kv && a.dkv_f32) {
          float* dst = a.dkv_f32 + row * D_K + col;
          if (a.accumulate) {
            const float old = *dst;
            if (hit) {
              v = old + v;
              *dst = v;
            } else {
              v = old;
            }
          } else {
            *dst = v;
          }
        }
        so[kvl * SO + col] = f2bf(v);
      }
    }
  if (a.dkv) {
    __syncthreads();
    for (int p = tid; p < TILE_KV * ROW_CHUNKS; p += 256) {
      const int kvl = p / ROW_CHUNKS, c = p - kvl * ROW_CHUNKS;
      const int64_t row = kb0 + kvl;
      if (row < a.s_kv)
        *reinterpret_cast<uint4_t*>(a.dkv + row * D_K + 8 * c) =
            *reinterpret_cast<const uint4_t*>(so + kvl * SO + 8 * c);
    }
  }
}

}  // namespace

hipError_t launch_bwd_dq(const BwdArgs& a, int heads, hipStream_t stream) {
  if (a.G == 0) return hipSuccess;
  dim3 grid((unsigned)a.G), block(256);
  switch (heads) {
    case 8: bwd_dq_kernel<8><<<grid, block, 0, stream>>>(a); break;
    case 16: bwd_dq_kernel<16><<<grid, block, 0, stream>>>(a); break;
    case 32: bwd_dq_kernel<32><<<grid, block, 0, stream>>>(a); break;
    case 64: bwd_dq_kernel<64><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkv(const BwdArgs& a, int heads, hipStream_t stream) {
  if (a.NB == 0) return hipSuccess;
  dim3 grid((unsigned)a.NB), block(256);
  switch (heads) {
    case 8: bwd_dkv_kernel<8><<<grid, block, 0, stream>>>(a); break;
    case 16: bwd_dkv_kernel<16><<<grid, block, 0, stream>>>(a); break;
    case 32: bwd_dkv_kernel<32><<<grid, block, 0, stream>>>(a); break;
    case 64: bwd_dkv_kernel<64><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace smla
