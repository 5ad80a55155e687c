// Sparse-MLA forward (gfx950): out = softmax(scale q.k) v over each token's
// selected KV rows, and the natural-log LSE per (token, head).
//
// One workgroup of 8 waves owns a query group: T = 64/H consecutive tokens,
// 64 query rows.  It walks the union of the group's selected KV rows in tiles
// of 32 rows, gathered into LDS with direct global->LDS copies two tiles
// ahead of their use (four buffers), and splits the work in two roles that
// run one tile apart:
//   score waves 0-3: wave w scores rows 16w..16w+15 against the tile
//            (S^T = K Q^T: K from LDS as the A operand, the wave's Q rows
//            held in registers as the B operand, 36 MFMA 16x16x32), then the
//            row softmax, and leaves P (bf16) and the rescale factors in LDS;
//   PV waves 4-7:    wave 4+c accumulates out[:, 128c .. 128c+127] for all 64
//            rows from the previous tile's P and V (32 MFMA, as out^T = V^T
//            P^T so that a lane holds adjacent columns of one row, stored
//            straight from the registers at the end).
// Per step every wave waits for the copies it issued two steps before (its
// copies of the previous step may still be in flight) and the workgroup syncs
// once; then the copies of tile j+2 are issued (8-9 per PV wave, one per
// score wave) and the PV waves take tile j-1 while the score waves take tile
// j.  Two waves share each SIMD, so one's softmax, copies and LDS waits
// overlap the other's MFMAs.
//
// The running max starts at a finite -1e30, so a tile with no valid entry
// never forms exp(-inf - -inf); the final denominator is floored at 1e-30, a
// no-op on rows with a valid slot (their largest term is exp(0) = 1) that
// makes an all-padding row output exact zeros with LSE = ln(1e-30).  The
// floor and the exact-zero padding follow miles PR #2079 ("fix GLM-5
// sparse-MLA kernel -1 index OOB and NaN gradients", 实现拆解 item 2 and the
// forward key code snippet); padding rows of a tile are copied from a zero
// row, never from an address computed from -1.
//
// fp8 kv variant (FP8): kv rows are records of 512 e4m3 latent values, four
// fp32 scales (one per 128 columns) and the 64 bf16 rope columns.  The
// latent bytes and scales of a tile are copied directly into an LDS staging
// buffer two tiles ahead (two buffers); a step before the tile is used, every
// wave converts 4 of its rows (value = e4m3 * scale, rounded to bf16) from
// the staging buffer into the same swizzled bf16 tile, right after the
// step's barrier.  The score waves copy
// the rope tails directly into the tile.  Everything downstream of the tile
// is the bf16 kernel's.
#include "smla_device.h"
#include "smla_internal.h"

namespace smla {

namespace {

constexpr int FT = 32;                // kv rows per tile
constexpr int FNB = 3;                // kv tile buffers
constexpr int FNW = 8;                // waves per workgroup
constexpr int SPS = FT + 8;           // P row stride (bf16): 80 bytes

// fp8 staging buffer of one tile: latent bytes [FT][512], then 16 bytes of
// scales per row for 64 rows (rows FT..63 are copies of the zero row, so the
// scale copy is one full-wave instruction).
constexpr int SF_LATENT = FT * FP8_SCALE_OFF;
constexpr int SF_BYTES = SF_LATENT + 64 * 16;

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, float sc) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);   // OCP e4m3 -> fp32 (exact)
  return pack_bf2(f[0] * sc, f[1] * sc);
}
// The same for a power-of-two scale, in one instruction: the scaled
// conversion applies only the scale's exponent, which is the whole scale
// when it is a power of two (the product is then exact in bf16).
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2_pow2(uint32_t w, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, HI));
}

// FP8: 0 bf16 kv rows; 1 fp8 records with fp32 scales; 2 fp8 records whose
// scales are powers of two.
template <int H, int FP8>
__global__ __launch_bounds__(FNW * 64, 1) void fwd_kernel(FwdArgs a) {
  constexpr int T = GROUP_ROWS / H;
  // bf16 kv: four tile buffers (tiles j-1 .. j+2: copies run two tiles
  // ahead); fp8 kv: three (its staging buffers take the rest of the LDS)
  constexpr int NBUF = FP8 ? FNB : FNB + 1;
  __shared__ __attribute__((aligned(16))) char sK[NBUF][KV32_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sF[2][FP8 ? SF_BYTES : 16];   // fp8 staging
  __shared__ __attribute__((aligned(16))) unsigned short sP[2][GROUP_ROWS * SPS];
  __shared__ __attribute__((aligned(16))) unsigned char sMask[NBUF][256];  // token masks (word copies)
  __shared__ __attribute__((aligned(16))) int sRow[NBUF][64];             // kv rows of a tile's entries
  __shared__ float sAlpha[2][GROUP_ROWS];                               // rescale factor per row
  __shared__ int sMoved[2][4];                                          // per score wave: a max moved
  __shared__ float sL[GROUP_ROWS];

  const int tid = threadIdx.x, lane_id = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool score_wave = wv < 4;
  const int64_t grp = a.order[blockIdx.x];
  const int64_t t0 = grp * T;
  const int n_ent = a.qcount[grp];
  const int32_t* erow = a.qrow + grp * a.qcap;
  const uint8_t* emask = a.qmask + grp * a.qcap;
  const int ntiles = (n_ent + FT - 1) / FT;

  // One register array serves both roles: a score wave keeps its 18 Q
  // fragments in the first 18 entries, a PV wave accumulates its 64 x 128
  // output block in all 32 (so the workgroup fits two waves per SIMD).
  float4_t acc[4][8];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[rb][n] = (float4_t){0.f, 0.f, 0.f, 0.f};
  if (score_wave) {
    const int r16 = lane_id & 15, g16 = lane_id >> 4;
    const int rr = 16 * wv + r16;
    const int64_t tok = t0 + rr / H;
    if (tok < a.s_q) {
      const uint16_t* qrow = a.q + (caller_token(tok, a.pair_s, a.pair_g) * H + rr % H) * D_K + 8 * g16;
#pragma unroll
      for (int ks = 0; ks < 18; ++ks)
        acc[ks >> 3][ks & 7] = __builtin_bit_cast(float4_t, ld16_global(qrow + 32 * ks));
    }
  }
  // Score-wave state: this lane's row is 16w + (lane & 15); the four lanes
  // g = 0..3 of a row hold kv entries 16nt + 4g + i and agree on m_run and
  // lsum.  m_run only moves when a row max exceeds it by more than
  // RESCALE_SLACK (log2 units), so most tiles leave the PV accumulators alone.
  const int tl = (16 * wv + (lane_id & 15)) / H;
  float m_run = M_INIT, lsum = 0.f;

  // Copies of tile t (its rows' indices are in sRow[t % NBUF]): the first 1 KB
  // of 8 kv rows per PV wave, the rope tails of 8 rows per score wave (the
  // score waves carry more of the per-tile work), the token masks by wave 4,
  // the row indices of tile t + 2 by wave 5.  Per call each wave issues a
  // fixed number of copies (bf16 kv: score waves 1, waves 4 and 5 nine,
  // waves 6 and 7 eight; past the union they copy zero rows), which the
  // counted waits of the main loop rely on.
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int b = t % NBUF;
    if constexpr (FP8) {
      if (score_wave && wv < FT / 8) {   // rope tails of rows 8 wv .. 8 wv + 7
        const int r = 8 * wv + (lane_id >> 3);
        const int row = sRow[b][r];
        const bool ok = r < min(FT, n_ent - t * FT) && (uint32_t)row < (uint32_t)a.s_kv;
        const uint8_t* rec = ok ? a.kv8 + (uint64_t)(uint32_t)row * FP8_REC_BYTES
                                : reinterpret_cast<const uint8_t*>(zero_row());
        g2lds16_u(rec + FP8_ROPE_OFF + 16 * ((lane_id & 7) ^ swz_hi(r)),
                  lds_offset(sK[b]) + (uint32_t)(FT * 1024 + 1024 * wv));
      }
    } else {
      // the rope tails of rows 8 w .. 8 w + 7 (score wave w), the first 1 KB
      // of rows 8 c .. 8 c + 7 (PV wave 4 + c)
      const int lw = score_wave ? wv : wv - 4;
      const KvGather<FT> g =
          kv_gather_prepare<FT>(sK[b], a.kv, a.s_kv, sRow[b], min(FT, n_ent - t * FT), lw, lane_id);
      if (score_wave) {
        kv_gather_copy<FT, FT / 4>(g, lw, lane_id);
      } else {
        static_for<FT / 4>([&](auto J) __attribute__((always_inline)) {
          kv_gather_copy<FT, decltype(J)::value>(g, lw, lane_id);
        });
      }
    }
    copy_union_entries(nullptr, sMask[b], erow, emask, t * FT, n_ent, FT, wv, 5, 4, lane_id);
    // Row indices of tile t + 2, the tile the copies two steps on need (the
    // copies run two tiles ahead of their use, for fp8 kv the staging
    // loads).  The buffer it lands in is read by no wave during this step.
    const int ti = t + 2;
    if (!FP8 || ti < ntiles)
      copy_union_entries(sRow[ti % NBUF], nullptr, erow, emask, ti * FT, n_ent, FT, wv, 5, 4,
                         lane_id);
  };

  // fp8 staging copies of tile t into sF[t & 1]: wave w copies the latent
  // bytes of rows 4w .. 4w+3 (two rows per copy: lanes 0-31 and 32-63, 16
  // bytes each), wave 7 the 16 scale bytes of rows 0..63.  Rows past the
  // tile's count, and indices outside [0, s_kv), read the zero row (all-zero
  // bytes: value 0, scale 0).
  auto fp8_stage = [&](int t) __attribute__((always_inline)) {
    const int b = t % NBUF;
    const int count = min(FT, n_ent - t * FT);
    const uint32_t st = lds_offset(sF[t & 1]);
    const int half = lane_id >> 5, m = lane_id & 31;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 4 * wv + 2 * p + half;
      const int row = sRow[b][r];
      const bool ok = r < count && (uint32_t)row < (uint32_t)a.s_kv;
      const uint8_t* rec = ok ? a.kv8 + (uint64_t)(uint32_t)row * FP8_REC_BYTES
                              : reinterpret_cast<const uint8_t*>(zero_row());
      g2lds16_u(rec + 16 * m, st + (uint32_t)(1024 * (2 * wv + p)));   // row r at 512 r
    }
    if (wv == FNW - 1) {
      const int r = lane_id;
      const int row = sRow[b][r];
      const bool ok = r < count && (uint32_t)row < (uint32_t)a.s_kv;
      const uint8_t* rec = ok ? a.kv8 + (uint64_t)(uint32_t)row * FP8_REC_BYTES
                              : reinterpret_cast<const uint8_t*>(zero_row());
      g2lds16_u(rec + FP8_SCALE_OFF, st + (uint32_t)SF_LATENT);
    }
  };
  // Conversion of tile t's staged rows 4w .. 4w+3 (wave w) into sK[t % 3]:
  // in pair p, lane l takes bytes 16 (l mod 32) .. +15 of row 4w + 2p + l/32,
  // which become bf16 chunks 2 (l mod 32) and 2 (l mod 32) + 1 of the row.
  auto fp8_convert = [&](int t) __attribute__((always_inline)) {
    const unsigned char* st = sF[t & 1];
    char* tile = sK[t % NBUF];
    const int half = lane_id >> 5, m = lane_id & 31;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int r = 4 * wv + 2 * p + half;
      const uint4_t v = *reinterpret_cast<const uint4_t*>(st + FP8_SCALE_OFF * r + 16 * m);
      const float sc = *reinterpret_cast<const float*>(st + SF_LATENT + 16 * r + 4 * (m >> 3));
      uint4_t w0, w1;
      if constexpr (FP8 == 2) {
        w0[0] = fp8x2_to_bf16x2_pow2<false>(v[0], sc);
        w0[1] = fp8x2_to_bf16x2_pow2<true>(v[0], sc);
        w0[2] = fp8x2_to_bf16x2_pow2<false>(v[1], sc);
        w0[3] = fp8x2_to_bf16x2_pow2<true>(v[1], sc);
        w1[0] = fp8x2_to_bf16x2_pow2<false>(v[2], sc);
        w1[1] = fp8x2_to_bf16x2_pow2<true>(v[2], sc);
        w1[2] = fp8x2_to_bf16x2_pow2<false>(v[3], sc);
        w1[3] = fp8x2_to_bf16x2_pow2<true>(v[3], sc);
      } else {
        w0[0] = fp8x2_to_bf16x2<false>(v[0], sc);
        w0[1] = fp8x2_to_bf16x2<true>(v[0], sc);
        w0[2] = fp8x2_to_bf16x2<false>(v[1], sc);
        w0[3] = fp8x2_to_bf16x2<true>(v[1], sc);
        w1[0] = fp8x2_to_bf16x2<false>(v[2], sc);
        w1[1] = fp8x2_to_bf16x2<true>(v[2], sc);
        w1[2] = fp8x2_to_bf16x2<false>(v[3], sc);
        w1[3] = fp8x2_to_bf16x2<true>(v[3], sc);
      }
      *reinterpret_cast<uint4_t*>(tile + 1024 * r + 16 * ((2 * m) ^ swz_lo(r))) = w0;
      *reinterpret_cast<uint4_t*>(tile + 1024 * r + 16 * ((2 * m + 1) ^ swz_lo(r))) = w1;
    }
  };

  // Scores and softmax of tile t (score waves).
  auto score = [&](int t) __attribute__((always_inline)) {
    const char* kt = sK[t % NBUF];
    const unsigned char* mkb = sMask[t % NBUF];
    int lane = lane_id;
    asm volatile("" : "+v"(lane));   // offsets recomputed per tile, not kept live
    const int g16 = lane >> 4, r16 = lane & 15;
    float4_t s[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) s[nt] = (float4_t){0.f, 0.f, 0.f, 0.f};
    // K fragments run KPF k-steps ahead of their MFMAs (a ring of KPF + 1
    // register sets); the scheduling barriers keep the reads from sinking
    // onto their uses.
    constexpr int KPF = 3;
    short8_t kb[KPF + 1][2];
#pragma unroll
    for (int d = 0; d < KPF; ++d)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) kb[d][nt] = ld_b_rs<FT>(kt, nt * 16, 32 * d, lane);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (ks + KPF < 18) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          kb[(ks + KPF) % (KPF + 1)][nt] = ld_b_rs<FT>(kt, nt * 16, 32 * (ks + KPF), lane);
      }
      __builtin_amdgcn_sched_barrier(0);
      const short8_t qf = __builtin_bit_cast(short8_t, acc[ks >> 3][ks & 7]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) s[nt] = mfma_bf16(kb[ks % (KPF + 1)][nt], qf, s[nt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const unsigned mk = *reinterpret_cast<const unsigned*>(mkb + nt * 16 + 4 * g16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = (mk >> (8 * i + tl)) & 1u;
        const float x = v ? s[nt][i] * a.scale_log2 : -INFINITY;
        s[nt][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = max_rows(mx);
    const bool move = mx > m_run + RESCALE_SLACK;
    float alpha = 1.f;
    if (move) {
      alpha = fast_exp2(m_run - mx);
      m_run = mx;
    }
    unsigned short* pt = sP[t & 1];
    float rs = 0.f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(s[nt][i] - m_run);
        rs += p[i];
      }
      uint2 pk;
      pk.x = pack_bf2(p[0], p[1]);
      pk.y = pack_bf2(p[2], p[3]);
      *reinterpret_cast<uint2*>(&pt[(16 * wv + r16) * SPS + nt * 16 + 4 * g16]) = pk;
    }
    rs = sum_rows(rs);
    lsum = lsum * alpha + rs;
    if (g16 == 0) sAlpha[t & 1][16 * wv + r16] = alpha;
    const bool moved = __ballot(move) != 0ull;
    if (lane == 0) sMoved[t & 1][wv] = moved ? 1 : 0;
  };

  // PV of tile t (PV waves): columns 128c .. 128c+127 for all 64 rows.
  auto pv = [&](int t) __attribute__((always_inline)) {
    const int c = wv - 4;
    const char* vt = sK[t % NBUF];
    const unsigned short* pt = sP[t & 1];
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int g16 = lane >> 4, r16 = lane & 15;
    const int* mv = sMoved[t & 1];
    if (mv[0] | mv[1] | mv[2] | mv[3]) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const float al = sAlpha[t & 1][16 * rb + r16];
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][n][i] *= al;
      }
    }
    short8_t pa[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) pa[rb] = ld16_lds(&pt[(16 * rb + r16) * SPS + 8 * g16]);
    // out^T += V^T P^T (V^T as the A operand): lane (g, r) accumulates row
    // 16 rb + r, columns 128c + 32m + 8g + 4h .. +3 in block n = 2m + h, so
    // blocks 2m and 2m + 1 hold 8 adjacent columns of one row.
    constexpr int VPF = 2;   // V fragments this many n-tiles ahead
    short8_t vb[VPF + 1];
#pragma unroll
    for (int d = 0; d < VPF; ++d) vb[d] = ld_bt_rs_pair<FT>(vt, 0, 128 * c + 32 * (d >> 1), d & 1, lane);
    static_for<8>([&](auto N) __attribute__((always_inline)) {
      constexpr int n = decltype(N)::value;
      if constexpr (n + VPF < 8)
        vb[(n + VPF) % (VPF + 1)] = ld_bt_rs_pair<FT>(vt, 0, 128 * c + 32 * ((n + VPF) >> 1), (n + VPF) & 1, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[rb][n] = mfma_bf16(vb[n % (VPF + 1)], pa[rb], acc[rb][n]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  if (ntiles > 0) {
    copy_union_entries(sRow[0], nullptr, erow, emask, 0, n_ent, FT, wv, 5, 4, lane_id);
    copy_union_entries(sRow[1], nullptr, erow, emask, FT, n_ent, FT, wv, 5, 4, lane_id);
    wait_vmcnt0();
    __syncthreads();
    issue(0);
    if constexpr (FP8) {   // tiles 0 and 1 staged, tile 0 converted
      fp8_stage(0);
      if (ntiles > 1) fp8_stage(1);
      wait_vmcnt0();
      __syncthreads();
      fp8_convert(0);
    } else {
      issue(1);            // (tile 2's and 3's row indices come with these)
    }
  }
  // Step j: the score waves take tile j, the PV waves tile j - 1; the next
  // tile's copies go into a buffer no wave reads in this step.  The two roles run
  // separate loops (so each keeps only its own state in registers) with the
  // same count of workgroup barriers, one per step.  fp8: tile j + 2 is
  // staged (into the staging buffer tile j left; its indices landed at this
  // step's barrier) and, before its role's work, every wave converts its rows
  // of tile j + 1 (staged a step ago) into the buffer tile j - 2 used.
  if constexpr (!FP8) {
    // bf16 kv: step j issues tile j + 2 (into the buffer of tile j - 2) and
    // waits at its start only for what step j - 2 and earlier issued -- the
    // wave's own copies of step j - 1 (a fixed count per wave) may still be
    // in flight -- so a tile's gather has two steps to land.
    if (ntiles > 0) {
      if (score_wave) {
        for (int j = 0; j <= ntiles; ++j) {
          if (j == 0) wait_vmcnt0(); else wait_vmcnt<1>();
          __syncthreads();
          issue(j + 2);
          if (j < ntiles) score(j);
        }
      } else {
        for (int j = 0; j <= ntiles; ++j) {
          if (j == 0) {
            wait_vmcnt0();
          } else if (wv == 4 || wv == 5) {
            wait_vmcnt<FT / 4 + 1>();
          } else {
            wait_vmcnt<FT / 4>();
          }
          __syncthreads();
          issue(j + 2);
          if (j >= 1) pv(j - 1);
        }
      }
    }
  } else if (score_wave) {
    for (int j = 0; j <= ntiles; ++j) {
      wait_vmcnt0();
      __syncthreads();
      if (j + 1 < ntiles) issue(j + 1);
      if (j + 2 < ntiles) fp8_stage(j + 2);
      if (j + 1 < ntiles) fp8_convert(j + 1);
      if (j < ntiles) score(j);
    }
  } else {
    for (int j = 0; j <= ntiles; ++j) {
      wait_vmcnt0();
      __syncthreads();
      if (j + 1 < ntiles) issue(j + 1);
      if (j + 2 < ntiles) fp8_stage(j + 2);
      if (j + 1 < ntiles) fp8_convert(j + 1);
      if (j >= 1) pv(j - 1);
    }
  }

  // Epilogue: LSE from the score waves; the PV waves normalise their rows'
  // columns and store them straight from their registers (16-byte pieces).
  wait_vmcnt0();
  if (score_wave && (lane_id >> 4) == 0) {
    const int rr = 16 * wv + (lane_id & 15);
    sL[rr] = lsum;
    const int64_t tok = t0 + rr / H;
    if (tok < a.s_q) {
      const float m_eff = lsum > 0.f ? m_run : 0.f;
      a.lse[caller_token(tok, a.pair_s, a.pair_g) * H + rr % H] =
          (m_eff + fast_log2(fmaxf(lsum, SUMEXP_FLOOR))) * LN2;
    }
  }
  __syncthreads();
  if (!score_wave) {
    const int c = wv - 4, g16 = lane_id >> 4, r16 = lane_id & 15;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int row = 16 * rb + r16;
      const int64_t tok = t0 + row / H;
      const float inv = 1.0f / fmaxf(sL[row], SUMEXP_FLOOR);
      if (tok < a.s_q) {
        uint16_t* orow = a.out + (caller_token(tok, a.pair_s, a.pair_g) * H + row % H) * D_V + 128 * c + 8 * g16;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint4_t v;
          v[0] = pack_bf2(acc[rb][2 * m][0] * inv, acc[rb][2 * m][1] * inv);
          v[1] = pack_bf2(acc[rb][2 * m][2] * inv, acc[rb][2 * m][3] * inv);
          v[2] = pack_bf2(acc[rb][2 * m + 1][0] * inv, acc[rb][2 * m + 1][1] * inv);
          v[3] = pack_bf2(acc[rb][2 * m + 1][2] * inv, acc[rb][2 * m + 1][3] * inv);
          *reinterpret_cast<uint4_t*>(orow + 32 * m) = v;
        }
      }
    }
  }
}

}  // namespace

template <int FP8>
hipError_t launch_fwd_t(const FwdArgs& a, int heads, hipStream_t stream) {
  dim3 grid((unsigned)a.G), block(FNW * 64);
  switch (heads) {
    case 8: fwd_kernel<8, FP8><<<grid, block, 0, stream>>>(a); break;
    case 16: fwd_kernel<16, FP8><<<grid, block, 0, stream>>>(a); break;
    case 32: fwd_kernel<32, FP8><<<grid, block, 0, stream>>>(a); break;
    case 64: fwd_kernel<64, FP8><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int heads, hipStream_t stream, int fp8) {
  if (a.G == 0) return hipSuccess;
  switch (fp8) {
    case 0: return launch_fwd_t<0>(a, heads, stream);
    case 1: return launch_fwd_t<1>(a, heads, stream);
    case 2: return launch_fwd_t<2>(a, heads, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace smla
