// Forward attention kernels for gfx950.
//
// Method ("FlashAttention 为什么不需要存下注意力矩阵" §03 3.2; "FlashAttention V1 技术深度解析" §3.2):
// stream K/V tiles past a resident block of queries, keeping per query row a running maximum m,
// a running sum l and an unnormalised output accumulator O, rescaled by exp(m_old - m_new)
// whenever the maximum grows; at the end O / l is the softmax-weighted sum and m + log l the
// logsumexp. Masked scores are -inf and K/V tiles entirely above the causal diagonal are never
// visited (same page, §03 3.2 last paragraph and §04 4.5).
//
// Loop order: each workgroup owns a query tile for its whole life and loops over K/V tiles
// (queries outer, keys inner), so m, l and O never leave registers. The pages' own V1 order
// (K/V outer, with O, l, m round-tripped to HBM per K/V block) is not used.
//
// gfx950 mapping (16-bit inputs):
//   * the score tile is computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: each lane
//     then owns one query (its accumulator column) and 16 keys, so row max / row sum are
//     in-lane plus one exchange between the two wave halves, and m, l, corr are lane-local;
//   * K rows are placed in LDS in a permuted order so that a lane's 16 accumulator slots are
//     keys {16*(i/8) + 8*g + i%8}: the probabilities then feed the P·V MFMA directly as its
//     B operand (no LDS round trip); V stays in key order in LDS and its transposed operand is
//     read with ds_read_b64_tr_b16;
//   * exp2 with scale*log2(e) folded into one FMA per score;
//   * K/V tiles hold fwd_tile_keys<D, IS_BF16, CAUSAL>() keys (a table per head dim, dtype and
//     causality written by the tuner; 64 for block-sparse masks);
//   * K and V tiles are double-buffered in LDS (one barrier per K/V tile) and filled by direct
//     buffer->LDS loads, issued for the next tile before the current tile's math: no staging
//     registers, no LDS write instructions. Tile rows are unpadded and swizzled (swz_off), which
//     keeps both the row reads of K and the transposed reads of V free of bank conflicts;
//   * workgroups are ordered longest-first for causal masks and grouped per XCD so that the
//     query tiles of one (b, h) share an L2;
//   * plain attention at d <= 128 runs fwd16pp_kernel: two groups of four waves that alternate
//     a softmax phase and an MFMA phase, one phase apart, so that each SIMD always holds one wave
//     of each kind, when its grid is large enough to fill the chip. Smaller grids, dropout,
//     block-sparse masks and d = 256 run fwd16_kernel (one group).
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_tune.h"

namespace fa {

// ----------------------------------------------------------------------------------------
// Workgroup -> (b*h, query tile) map. Workgroups are dispatched round-robin over the 8 XCDs
// (blockIdx % 8). When B*H is a multiple of 8, each XCD gets a contiguous set of heads, and
// within an XCD the longest query tiles (causal: the last ones) are dispatched first. With
// `fold` (a causal grid that is resident all at once, two workgroups per CU), the first half of
// the order still runs longest-first and takes the first slot of each CU, while the second half
// runs shortest-first: the second slot of the CU that got query tile T-1-t gets tile t, so every
// CU holds about the same number of key tiles (tile t of a causal head visits t+1 of them).
// ----------------------------------------------------------------------------------------
__device__ __forceinline__ int causal_tile(int t, int n_tiles, bool fold) {
  const int half = (n_tiles + 1) >> 1;
  return (fold && t >= half) ? t - half : n_tiles - 1 - t;
}

__device__ __forceinline__ void map_block(int bid, int n_tiles, int bh_total, bool causal,
                                          bool fold, int& bh, int& tile) {
  int t;
  if ((bh_total & 7) == 0) {
    const int xcd = bid & 7;
    const int slot = bid >> 3;
    const int heads_per_xcd = bh_total >> 3;
    t = slot / heads_per_xcd;
    bh = xcd * heads_per_xcd + (slot - t * heads_per_xcd);
  } else {
    t = bid / bh_total;
    bh = bid - t * bh_total;
  }
  tile = causal ? causal_tile(t, n_tiles, fold) : t;
}

// Key held by LDS row R (0..31 within a 32-key block) of a K tile: rows are filled so that
// accumulator row r = 8a + 4b + c of the S^T MFMA holds key 16*(a/2) + 8*b + 4*(a%2) + c, which
// makes accumulator slot i of lane group g hold key 16*(i/8) + 8*g + i%8 (contiguous runs of 8
// that feed the P.V MFMA directly).
__device__ __forceinline__ int key_of_krow(int R) {
  return 16 * (R >> 4) + 8 * ((R >> 2) & 1) + 4 * ((R >> 3) & 1) + (R & 3);
}

// Tile shape of the 16-bit forward kernel: QB 32-query blocks per wave, BC keys per K/V tile
// (from the tuning table; block-sparse instances use 64, half a mask block).
template <int D, int QB, int BC_>
struct Fwd16 {
  static constexpr int NW = 4;            // waves per workgroup
  static constexpr int NT = NW * 64;      // threads
  static constexpr int BR = NW * QB * 32; // query rows per workgroup
  static constexpr int BC = BC_;          // keys per K/V tile
  static constexpr int KB = BC / 32;      // 32-key MFMA blocks per tile
  static constexpr int KS = D / 16;       // contraction steps of S^T = K Q^T
  static constexpr int DB = D / 32;       // 32-row blocks of O^T
  static constexpr int KROW = D;          // K and V tile rows in LDS: swizzled, no padding
  static constexpr int KTILE = BC * KROW;
  static constexpr int LD_INSTR = BC * D * 2 / 1024;  // 1 KB direct loads per tile and tensor
  static constexpr int STAGE = 2 * KTILE;  // K then V, elements per LDS stage
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static_assert(LD_INSTR % NW == 0, "each wave issues whole 1 KB loads");
};

template <int D, bool IS_BF16, bool CAUSAL, bool SPARSE>
constexpr int fwd_bc() {
  return SPARSE ? 64 : fwd_tile_keys<D, IS_BF16, CAUSAL>();
}

// Queries per wave (32 per MFMA column block). Two blocks halve the LDS reads per MFMA but, at
// 227 VGPRs, allow only 2 waves per SIMD and give half as many workgroups for the causal
// schedule; measured at B=2 H=16 N=4096 d=64 causal, one block per wave is 17% faster.
template <int D>
constexpr int fwd_qb() {
  return 1;
}

// Waves per SIMD the register allocation must allow: 2, except at d = 256, whose 32-query
// output accumulator alone is 128 registers (one wave then uses the whole file, AGPRs included).
template <int D>
constexpr int fwd_min_waves() {
  return D >= 256 ? 1 : 2;
}

template <int D, bool IS_BF16, bool O_F32, bool CAUSAL, int QB, bool DROP, bool SPARSE>
__global__ __launch_bounds__(256, fwd_min_waves<D>()) void fwd16_kernel(FwdArgs a) {
  using C = Fwd16<D, QB, fwd_bc<D, IS_BF16, CAUSAL, SPARSE>()>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int r = lane & 31;
  // Queries are rows 0 .. N-1 of Q and sit at positions qoff .. qoff + N - 1 of the key sequence
  // (N keys and qoff = 0 unless the caller gave a longer K/V, Nk = N + qoff keys).
  const int N = a.N;
  const int Nk = a.Nk;
  const int qoff = a.qoff;

  int bh, tile;
  map_block(blockIdx.x, a.n_tiles, a.bh, CAUSAL, a.fold != 0, bh, tile);
  const size_t head_off = (size_t)bh * N * D;
  const size_t kv_off = (size_t)bh * Nk * D;
  const auto qrs = make_rsrc(static_cast<const uint16_t*>(a.q) + head_off, (uint32_t)N * D * 2);
  const auto krs = make_rsrc(static_cast<const uint16_t*>(a.k) + kv_off, (uint32_t)Nk * D * 2);
  const auto vrs = make_rsrc(static_cast<const uint16_t*>(a.v) + kv_off, (uint32_t)Nk * D * 2);

  const int qt0 = tile * C::BR;
  const int qw0 = qt0 + wave * QB * 32;  // first query of this wave

  // Q fragments (B operand of S^T = K Q^T): query qw0 + 32*qb + r, d = 16*ks + 8*g .. +8.
  // Rows beyond N read as zeros. A negative scale is folded into Q by flipping its sign bits
  // (exact), so the math below only ever sees c = |scale| * log2(e) > 0 and a row maximum.
  const uint32_t qsign = a.c < 0.f ? 0x80008000u : 0u;
  Frag16 qf[QB][C::KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      qf[qb][ks].w = buf_ld16(qrs, (uint32_t)((qw0 + qb * 32 + r) * D + ks * 16 + g * 8) * 2);
      qf[qb][ks].w ^= qsign;
    }

  f32x16 oacc[C::DB][QB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][qb][i] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -3.0e38f;
    l_run[qb] = 0.f;
  }

  // |scale| * log2(e); never 0 (the host maps scale 0 to a tiny value).
  const float c = __builtin_fabsf(a.c);

  const int kv_end = CAUSAL ? min(Nk, qt0 + qoff + C::BR) : Nk;
  const int n_kt = (kv_end + C::BC - 1) / C::BC;

  // Block-sparse: the K/V tiles this query tile visits are those whose 128-key block is live in
  // its row of the block mask (the query tile is exactly one 128-row block). They are compacted
  // into a list in LDS after the two stages; tiles past the list's end map past kv_end.
  int n_live = n_kt;
  const uint16_t* live_list = nullptr;
  if constexpr (SPARSE) {
    static_assert(C::BR == kSparseBlock && 2 * C::BC == kSparseBlock, "tile / block mismatch");
    uint16_t* list = smem + 2 * C::STAGE;
    const uint8_t* mrow = a.sparse.mask +
        ((size_t)(a.sparse.mask_heads == 1 ? 0 : bh) * a.sparse.nb + tile) * a.sparse.nb;
    n_live = build_live_list(list, reinterpret_cast<int*>(list + kSparseListMax), n_kt,
                             [&](int t) { return mrow[t >> 1] != 0; });
    live_list = list;
  }
  auto tile_j0 = [&](int n) -> int {
    if constexpr (SPARSE) return n < n_live ? (int)live_list[n] * C::BC : n_kt * C::BC;
    return n * C::BC;
  };

  // Global -> LDS staging of one K/V tile by direct (LDS-destination) buffer loads: wave w
  // issues the 1 KB loads t = w, w + 4, ... of each tensor; lane l of load t deposits 16 bytes at
  // element 512 t + 8 l of the tile, i.e. LDS row R = (512 t + 8 l) / D, physical chunk p. That
  // slot holds logical chunk p ^ swz<D>(R) of the key stored on row R: key R for V, and for K the
  // key given by key_of_krow. Keys beyond N read as zeros.
  constexpr int LPW = C::LD_INSTR / C::NW;  // loads per wave and tensor
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int e = (wave + i * C::NW) * 512 + lane * 8;
    const int R = e / D, pch = (e % D) >> 3;
    const int cch = pch ^ swz<D>(R);
    const int kkey = (R & ~31) + key_of_krow(R & 31);
    koff[i] = (uint32_t)(kkey * D + cch * 8) * 2;
    voff[i] = (uint32_t)(R * D + cch * 8) * 2;
  }
  auto issue_tile = [&](int stage, int j0) {
    uint16_t* ks_ = smem + stage * C::STAGE;
    uint16_t* vs_ = ks_ + C::KTILE;
    const uint32_t base = (uint32_t)j0 * D * 2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int t = wave + i * C::NW;
      buf_ld16_lds(krs, base + koff[i], ks_ + t * 512);
      buf_ld16_lds(vrs, base + voff[i], vs_ + t * 512);
    }
  };

  // Math of one K/V tile already in LDS stage `stage`.
  auto tile_math = [&](int stage, int j0) {
      const bool wave_live = (j0 < kv_end) && (!CAUSAL || (j0 <= qw0 + qoff + QB * 32 - 1));
      if (wave_live) {
        const uint16_t* ks_ = smem + stage * C::STAGE;
        const uint16_t* vs_ = ks_ + C::KTILE;

        // ---- S^T = K Q^T ---------------------------------------------------------------
        f32x16 sacc[C::KB][QB];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[kb][qb][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) {
            Frag16 kf;
            kf.w = *reinterpret_cast<const u32x4*>(ks_ + swz_off<D>(kb * 32 + r, ks * 16 + g * 8));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              sacc[kb][qb] = mfma32x32x16<IS_BF16>(kf, qf[qb][ks], sacc[kb][qb]);
          }
        }

        // ---- mask: keys beyond Nk, and keys after the query on causal diagonal tiles ---------
        const bool need_mask = (j0 + C::BC > Nk) || (CAUSAL && (j0 + C::BC - 1 > qw0 + qoff));
        if (need_mask) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int qpos = qw0 + qb * 32 + r + qoff;
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int key = j0 + kb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
                const bool dead = (key >= Nk) || (CAUSAL && key > qpos);
                sacc[kb][qb][i] = dead ? -INFINITY : sacc[kb][qb][i];
              }
          }
        }

        // ---- online softmax (log2 domain): m, l, corr per query (lane-local) ----------------
        Frag16 pf[C::KB][2][QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float red = sacc[0][qb][0];
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) red = vmax(red, sacc[kb][qb][i]);
          red = halves_max(red);
          const float m_blk = red * c;  // -inf when the whole tile is masked for this query
          // Exact running maximum: the largest weight of each row is then exp2(0) = 1, which
          // bf16/fp16 hold exactly. (Deferring the rescale until the maximum grows by a margin
          // saves the multiplies below but leaves that weight at 2^x with a rounding error of
          // up to 2^-9, which measurably degrades O, and through D = rowsum(dO * O) the
          // gradients, on peaked rows.)
          const float m_new = vmax(m_run[qb], m_blk);
          const float corr = fast_exp2(m_run[qb] - m_new);
          m_run[qb] = m_new;
          l_run[qb] *= corr;
          // Unconditional rescale: a branch here would split the tile's math into separate
          // basic blocks and keep the scheduler from overlapping MFMA and VALU work.
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][qb][i] *= corr;
          const float m_ref = m_run[qb];
          float lsum = -0.f;  // -0 + x = x exactly, so the first add folds away
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              float p[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                p[e] = fast_exp2(__builtin_fmaf(sacc[kb][qb][h * 8 + e], c, -m_ref));
                lsum += p[e];  // fp32 row sum: the LSE needs it to well below bf16 precision
              }
              if constexpr (DROP) {
                // Dropout on the probabilities that multiply V (the row sum above keeps every
                // probability: the softmax is normalised before dropout). This lane's 8 keys
                // form one aligned group of 8, i.e. one Philox block.
                const uint32_t grp = (uint32_t)(j0 + kb * 32 + h * 16 + g * 8) >> 3;
                const uint32_t bits = keep_bits8(a.drop, grp, (uint32_t)(qw0 + qb * 32 + r),
                                                 (uint32_t)bh);
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] = ((bits >> e) & 1u) ? p[e] : 0.f;
              }
              pf[kb][h][qb].w = u32x4{pack2<IS_BF16>(p[0], p[1]), pack2<IS_BF16>(p[2], p[3]),
                                      pack2<IS_BF16>(p[4], p[5]), pack2<IS_BF16>(p[6], p[7])};
            }
          }
          l_run[qb] += lsum;
        }

      // ---- O^T += V^T P^T -----------------------------------------------------------------
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
              // A operand V^T: lane (g, r) needs V[kb*32 + 16h + 8g + s][32*db + r], s = 0..7.
              Frag16 vf;
              const int row = kb * 32 + h * 16 + g * 8;
              vf.w = lds_tr_frag_swz<D>(vs_, row, row + 4, db * 32);
#pragma unroll
              for (int qb = 0; qb < QB; ++qb)
                oacc[db][qb] = mfma32x32x16<IS_BF16>(vf, pf[kb][h][qb], oacc[db][qb]);
            }
          }
        }
      }

  };

  // n_kt >= 1 always (N >= 1). The prologue stages tile 0; the explicit wait retires the Q loads
  // before the loop; tile 1 is then in flight when the loop starts.
  issue_tile(0, tile_j0(0));
  wait_vmem_all();
  __syncthreads();

  // Iteration jt: start the direct loads of tile jt+1 into the other stage (its previous tile's
  // math ended before the last barrier), do the math of tile jt, wait for the loads, barrier.
  // After the last tile nothing is loaded or waited for: on small grids the memory latency of a
  // load whose data is never used would sit on the critical path of every workgroup.
  for (int jt = 0; jt < n_live; jt += 2) {
    const bool more1 = jt + 1 < n_live;
    if (more1) issue_tile(1, tile_j0(jt + 1));
    tile_math(0, tile_j0(jt));
    if (!more1) break;
    wait_vmem_all();
    __syncthreads();
    const bool more2 = jt + 2 < n_live;
    if (more2) issue_tile(0, tile_j0(jt + 2));
    tile_math(1, tile_j0(jt + 1));
    if (!more2) break;
    wait_vmem_all();
    __syncthreads();
  }

  // ---- epilogue: O / l, LSE = (m + log2 l) * ln 2 -------------------------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qw0 + qb * 32 + r;
    const float l_tot = halves_sum(l_run[qb]);
    // With dropout, kept probabilities are scaled by 1 / keep rate. A row that saw no key at all
    // (possible only with a block mask) has l = 0: its output is 0 and its LSE -inf.
    const bool empty = SPARSE && l_tot == 0.f;
    const float inv = empty ? 0.f : (DROP ? a.drop.keep_scale : 1.f) / l_tot;
    if (qrow < N) {
      if (g == 0)
        a.lse[(size_t)bh * N + qrow] = empty ? -INFINITY : (m_run[qb] + fast_log2(l_tot)) * kLn2;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          const int d0 = db * 32 + blk * 8 + g * 4;
          const float o0 = oacc[db][qb][blk * 4 + 0] * inv;
          const float o1 = oacc[db][qb][blk * 4 + 1] * inv;
          const float o2 = oacc[db][qb][blk * 4 + 2] * inv;
          const float o3 = oacc[db][qb][blk * 4 + 3] * inv;
          if constexpr (O_F32) {
            float* dst = static_cast<float*>(a.o) + head_off + (size_t)qrow * D + d0;
            *reinterpret_cast<f32x4*>(dst) = f32x4{o0, o1, o2, o3};
          } else {
            uint16_t* dst = static_cast<uint16_t*>(a.o) + head_off + (size_t)qrow * D + d0;
            *reinterpret_cast<u32x2*>(dst) = u32x2{pack2<IS_BF16>(o0, o1), pack2<IS_BF16>(o2, o3)};
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------------------
// Two-group variant for plain attention: 8 waves (256 queries, 32 per wave) per workgroup in two
// groups of four; waves w and w + 4 share a SIMD. Each wave alternates two phases per K/V tile:
//   V phase (vector ALU): mask, online softmax of its score tile S_t -> P_t, rescale of O;
//   M phase (matrix cores + LDS): O += V_t P_t, then S_{t+1} = K_{t+1} Q^T.
// Group 1 runs one phase behind group 0 and every phase ends with a workgroup barrier, so on each
// SIMD one wave is in its M phase while the other is in its V phase: the exp / FMA stream of one
// wave issues alongside the MFMA stream of the other.
// LDS holds two K and two V stages (tile t in stage t mod 2). With phase 2t the V phase of group
// 0 for tile t (and the M phase of group 1 for tile t-1):
//   K_t is read in phases 2t-1 and 2t; V_t in phases 2t+1 and 2t+2;
//   group 0 issues K_{t+1} in phase 2t (its stage last held K_{t-1}, read up to phase 2t-2) and
//   waits for it at the end of that phase; group 1 issues V_{t+1} in phase 2t+1 (stage of
//   V_{t-1}, read up to phase 2t) and waits for it at the end of phase 2t+2.
// ----------------------------------------------------------------------------------------
constexpr int kPpRows = 256;  // queries per workgroup of the two-group kernel (8 waves x 32)

template <int D, int BC_>
struct FwdPP {
  static constexpr int NW = 8;
  static constexpr int NT = NW * 64;
  static constexpr int BR = kPpRows;
  static constexpr int BC = BC_;
  static constexpr int KB = BC / 32;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int KTILE = BC * D;
  static constexpr int LD_INSTR = BC * D * 2 / 1024;  // 1 KB direct loads per tile and tensor
  static constexpr int LPW = LD_INSTR / 4;            // per wave of one group
  static constexpr int LDS_BYTES = 4 * KTILE * 2;
  static_assert(LD_INSTR % 4 == 0, "each wave of a group issues whole 1 KB loads");
};

template <int D, bool IS_BF16, bool O_F32, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd16pp_kernel(FwdArgs a) {
  using C = FwdPP<D, fwd_tile_keys<D, IS_BF16, CAUSAL>()>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wg = wave & 3;  // index within the group
  const int g = lane >> 5;
  const int r = lane & 31;
  const int N = a.N;
  const int Nk = a.Nk;
  const int qoff = a.qoff;

  int bh, tile;
  map_block(blockIdx.x, a.n_tiles, a.bh, CAUSAL, a.fold != 0, bh, tile);
  const size_t head_off = (size_t)bh * N * D;
  const size_t kv_off = (size_t)bh * Nk * D;
  const auto qrs = make_rsrc(static_cast<const uint16_t*>(a.q) + head_off, (uint32_t)N * D * 2);
  const auto krs = make_rsrc(static_cast<const uint16_t*>(a.k) + kv_off, (uint32_t)Nk * D * 2);
  const auto vrs = make_rsrc(static_cast<const uint16_t*>(a.v) + kv_off, (uint32_t)Nk * D * 2);

  const int qt0 = tile * C::BR;
  const int qw0 = qt0 + wave * 32;

  const uint32_t qsign = a.c < 0.f ? 0x80008000u : 0u;
  Frag16 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qf[ks].w = buf_ld16(qrs, (uint32_t)((qw0 + r) * D + ks * 16 + g * 8) * 2);
    qf[ks].w ^= qsign;
  }

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -3.0e38f, l_run = 0.f;
  const float c = __builtin_fabsf(a.c);

  const int kv_end = CAUSAL ? min(Nk, qt0 + qoff + C::BR) : Nk;
  const int n_kt = (kv_end + C::BC - 1) / C::BC;

  uint16_t* const k_st = smem;
  uint16_t* const v_st = smem + 2 * C::KTILE;

  // Direct loads of one tile by the four waves of a group (group 0 loads K, group 1 V): wave wg
  // issues 1 KB loads t = wg, wg + 4, ...; lane l of load t fills element 512 t + 8 l of the tile
  // (swizzled rows; K rows in key_of_krow order).
  uint32_t loff[C::LPW];
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int e = (wg + i * 4) * 512 + lane * 8;
    const int R = e / D, pch = (e % D) >> 3;
    const int cch = pch ^ swz<D>(R);
    const int key = grp == 0 ? (R & ~31) + key_of_krow(R & 31) : R;
    loff[i] = (uint32_t)(key * D + cch * 8) * 2;
  }
  auto load_k = [&](int stage, int t) {
    uint16_t* dst = k_st + stage * C::KTILE;
    const uint32_t base = (uint32_t)(t * C::BC) * D * 2;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) buf_ld16_lds(krs, base + loff[i], dst + (wg + i * 4) * 512);
  };
  auto load_v = [&](int stage, int t) {
    uint16_t* dst = v_st + stage * C::KTILE;
    const uint32_t base = (uint32_t)(t * C::BC) * D * 2;
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) buf_ld16_lds(vrs, base + loff[i], dst + (wg + i * 4) * 512);
  };

  // Every wave processes every tile of the workgroup: a tile entirely after a wave's queries is
  // masked to -inf, which leaves m, l and O exactly unchanged (tile 0 is never of that kind, so
  // m is finite from the first tile on). This costs at most one tile per wave and keeps the
  // phases branch-free.
  f32x16 s[C::KB];
  Frag16 pf[C::KB][2];
  float corr_pend = 1.f;  // rescale factor of tile t's softmax, applied to O in its M phase

  // M phase of tile t: O = corr * O + V_t P_t (V stage t % 2), then S_{t+1} (K stage (t + 1) % 2)
  // if t + 1 < n_s. The rescale of O sits here rather than in the softmax phase, which is the
  // longer of the two (measured 2% faster); the order of the arithmetic on O is unchanged.
  auto m_phase = [&](int t, int vstage, int kstage, int n_s) {
    if (t >= 0) {
      const uint16_t* vs_ = v_st + vstage * C::KTILE;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= corr_pend;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = kb * 32 + h * 16 + g * 8;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            Frag16 vf;
            vf.w = lds_tr_frag_swz<D>(vs_, row, row + 4, db * 32);
            oacc[db] = mfma32x32x16<IS_BF16>(vf, pf[kb][h], oacc[db]);
          }
        }
    }
    if (t + 1 < n_s) {
      const uint16_t* ks_ = k_st + kstage * C::KTILE;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      // Fragment f = (ks, kb) of K, read fwd_pre<D>() fragments ahead of its MFMA.
      read_ahead<C::KS * C::KB, fwd_pre<D>()>(
          [&](int f) {
            const int ks = f / C::KB, kb = f % C::KB;
            return *reinterpret_cast<const u32x4*>(ks_ +
                                                   swz_off<D>(kb * 32 + r, ks * 16 + g * 8));
          },
          [&](int f, const Frag16& kf) {
            const int ks = f / C::KB, kb = f % C::KB;
            s[kb] = mfma32x32x16<IS_BF16>(kf, qf[ks], s[kb]);
          });
    }
  };

  // V phase of tile t: mask, online softmax (the rescale of O is left to the M phase).
  auto v_phase = [&](int t) {
    const int j0 = t * C::BC;
    if ((j0 + C::BC > Nk) || (CAUSAL && (j0 + C::BC - 1 > qw0 + qoff))) {
      // Slot i of block kb holds key j0 + g*8 + ci, ci = 32kb + 16(i/8) + i%8 (a constant); the
      // key is dead past Nk - 1 and, when causal, past this lane's query position. One bound per
      // tile keeps the comparisons against immediates.
      int bound = Nk - 1 - j0 - g * 8;
      if (CAUSAL) bound = min(bound, qw0 + r + qoff - j0 - g * 8);
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ci = kb * 32 + (i >> 3) * 16 + (i & 7);
          s[kb][i] = ci > bound ? -INFINITY : s[kb][i];
        }
    }
    // Row maximum as four independent chains (a single chain would serialise ~32 dependent
    // max3 instructions while this wave is the only VALU issuer on its SIMD).
    float red4[4] = {s[0][0], s[0][1], s[0][2], s[0][3]};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int i = (kb == 0 ? 4 : 0); i < 16; ++i) red4[i & 3] = vmax(red4[i & 3], s[kb][i]);
    const float red = halves_max(vmax(vmax(red4[0], red4[1]), vmax(red4[2], red4[3])));
    const float m_new = vmax(m_run, red * c);
    const float corr = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= corr;
    corr_pend = corr;
    // Row sum. bf16: the unrounded fp32 probabilities (a bf16 rounding of a dominant weight would
    // show in log l beyond the LSE tolerance). fp16: the probabilities as rounded for the P.V
    // product, two per v_dot2c_f32_f16 in four chains; an fp16 rounding (2^-11 relative) stays
    // well inside that tolerance, and O is then normalised by the sum of exactly the weights
    // that multiplied V.
    float lsum = -0.f;  // -0 + x = x exactly, so the first add folds away
    float lpart[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(__builtin_fmaf(s[kb][h * 8 + e], c, -m_new));
          if constexpr (IS_BF16) lsum += p[e];
        }
        pf[kb][h].w = u32x4{pack2<IS_BF16>(p[0], p[1]), pack2<IS_BF16>(p[2], p[3]),
                            pack2<IS_BF16>(p[4], p[5]), pack2<IS_BF16>(p[6], p[7])};
        if constexpr (!IS_BF16) {
#pragma unroll
          for (int j = 0; j < 4; ++j) lpart[j] = add_pair_f16(pf[kb][h].w[j], lpart[j]);
        }
      }
    if constexpr (!IS_BF16) lsum = (lpart[0] + lpart[1]) + (lpart[2] + lpart[3]);
    l_run += lsum;
  };

  // Prologue: K_0 (group 0) and V_0 (group 1); then group 0 computes S_0.
  if (grp == 0) load_k(0, 0);
  else load_v(0, 0);
  wait_vmem_all();
  __syncthreads();

  // Causal: group 0's queries end at qt0 + 127, so the tiles from n_math on (keys past
  // qt0 + qoff + 127) hold no key any of its waves may see; they would leave its m, l and O
  // unchanged. Group 0 computes only the tiles before n_math, then for the others still issues
  // the K loads that group 1 needs and takes part in the same barriers, in the same order.
  const int n_math = (CAUSAL && grp == 0) ? min(n_kt, (qt0 + qoff + 127) / C::BC + 1) : n_kt;

  if (grp == 0) {
    m_phase(-1, 1, 0, n_math);
    wg_barrier();
    for (int t = 0; t < n_math; t += 2) {
      if (t + 1 < n_kt) load_k(1, t + 1);
      v_phase(t);
      wait_vmem_all();
      wg_barrier();
      m_phase(t, 0, 1, n_math);
      wg_barrier();
      if (t + 1 >= n_math) break;
      if (t + 2 < n_kt) load_k(0, t + 2);
      v_phase(t + 1);
      wait_vmem_all();
      wg_barrier();
      m_phase(t + 1, 1, 0, n_math);
      wg_barrier();
    }
    for (int u = n_math; u < n_kt; ++u) {
      if (u + 1 < n_kt) load_k((u + 1) & 1, u + 1);
      wait_vmem_all();
      wg_barrier();
      wg_barrier();
    }
  } else {
    wg_barrier();
    for (int t = 0; t < n_kt; t += 2) {
      m_phase(t - 1, 1, 0, n_kt);
      wait_vmem_all();
      wg_barrier();
      if (t + 1 < n_kt) load_v(1, t + 1);
      v_phase(t);
      wg_barrier();
      if (t + 1 >= n_kt) break;
      m_phase(t, 0, 1, n_kt);
      wait_vmem_all();
      wg_barrier();
      if (t + 2 < n_kt) load_v(0, t + 2);
      v_phase(t + 1);
      wg_barrier();
    }
    // P.V of the last tile (its V stage is not the target of the load still in flight).
    if (n_kt & 1) m_phase(n_kt - 1, 0, 1, n_kt);
    else m_phase(n_kt - 1, 1, 0, n_kt);
    wait_vmem_all();
  }

// Epilogue: O / l, LSE = (m + log2 l) * ln 2.
  const int qrow = qw0 + r;
  const float l_tot = halves_sum(l_run);
  const float inv = 1.f / l_tot;
  if (qrow < N) {
    if (g == 0) a.lse[(size_t)bh * N + qrow] = (m_run + fast_log2(l_tot)) * kLn2;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int d0 = db * 32 + blk * 8 + g * 4;
        const float o0 = oacc[db][blk * 4 + 0] * inv;
        const float o1 = oacc[db][blk * 4 + 1] * inv;
        const float o2 = oacc[db][blk * 4 + 2] * inv;
        const float o3 = oacc[db][blk * 4 + 3] * inv;
        if constexpr (O_F32) {
          float* dst = static_cast<float*>(a.o) + head_off + (size_t)qrow * D + d0;
          *reinterpret_cast<f32x4*>(dst) = f32x4{o0, o1, o2, o3};
        } else {
          uint16_t* dst = static_cast<uint16_t*>(a.o) + head_off + (size_t)qrow * D + d0;
          *reinterpret_cast<u32x2*>(dst) = u32x2{pack2<IS_BF16>(o0, o1), pack2<IS_BF16>(o2, o3)};
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------------------
// fp32 inputs: the same recurrence on true-fp32 MFMA (v_mfma_f32_32x32x2_f32). One wave owns
// 32 queries, K/V tiles of 32 keys are staged in LDS in natural [key][d] layout (one float per
// lane per operand, so no transposition is needed).
// ----------------------------------------------------------------------------------------
template <int D, bool CAUSAL>
struct Fwd32 {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BR = NW * 32;
  static constexpr int BC = 32;
  static constexpr int DB = D / 32;
  static constexpr int ROW = D + 1;  // padded row stride (floats)
  static constexpr int TILE = BC * ROW;
  static constexpr int LDS_BYTES = 2 * TILE * 4;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd32_kernel(FwdArgs a) {
  using C = Fwd32<D, CAUSAL>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem16[];
  float* smem = reinterpret_cast<float*>(smem16);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int r = lane & 31;
  const int N = a.N;

  int bh, tile;
  map_block(blockIdx.x, a.n_tiles, a.bh, CAUSAL, a.fold != 0, bh, tile);
  const size_t head_off = (size_t)bh * N * D;
  const float* __restrict__ qh = static_cast<const float*>(a.q) + head_off;
  const float* __restrict__ kh = static_cast<const float*>(a.k) + head_off;
  const float* __restrict__ vh = static_cast<const float*>(a.v) + head_off;

  const int qt0 = tile * C::BR;
  const int qw0 = qt0 + wave * 32;
  const int qrow = qw0 + r;

  // Q (B operand): query qrow, d = 2*ks + g.
  float qf[D / 2];
#pragma unroll
  for (int ks = 0; ks < D / 2; ++ks) qf[ks] = (qrow < N) ? qh[(size_t)qrow * D + 2 * ks + g] : 0.f;

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -3.0e38f, l_run = 0.f;

  const float c = a.c;
  const bool c_pos = c > 0.f;
  const float masked = c_pos ? -INFINITY : INFINITY;
  const int kv_end = CAUSAL ? min(N, qt0 + C::BR) : N;
  const int n_kt = (kv_end + C::BC - 1) / C::BC;

  for (int jt = 0; jt < n_kt; ++jt) {
    const int j0 = jt * C::BC;
    float* ks_ = smem;
    float* vs_ = smem + C::TILE;
    __syncthreads();
    for (int e = tid; e < C::BC * D; e += C::NT) {
      const int key = e / D, dd = e % D;
      const int gk = j0 + key;
      ks_[key * C::ROW + dd] = (gk < N) ? kh[(size_t)gk * D + dd] : 0.f;
      vs_[key * C::ROW + dd] = (gk < N) ? vh[(size_t)gk * D + dd] : 0.f;
    }
    __syncthreads();
    if (CAUSAL && j0 > qw0 + 31) continue;

    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(ks_[r * C::ROW + 2 * ks + g], qf[ks], sacc, 0,
                                                  0, 0);
    // accumulator slot i holds key j0 + 8*(i/4) + 4*g + i%4 for query qrow
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = j0 + (i >> 2) * 8 + g * 4 + (i & 3);
      if (key >= N || (CAUSAL && key > qrow)) sacc[i] = masked;
    }
    float red = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) red = c_pos ? fmaxf(red, sacc[i]) : fminf(red, sacc[i]);
    const float other = swap_halves(red);
    red = c_pos ? fmaxf(red, other) : fminf(red, other);
    const float m_new = fmaxf(m_run, red * c);
    const float corr = fast_exp2(m_run - m_new);
    m_run = m_new;
    float p[16];
    float lsum = -0.f;  // -0 + x = x exactly, so the first add folds away
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = fast_exp2(__builtin_fmaf(sacc[i], c, -m_new));
      lsum += p[i];
    }
    l_run = l_run * corr + lsum;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= corr;
    // O^T += V^T P^T: MFMA s takes slot s; lane group g supplies key 8*(s/4) + 4*g + s%4.
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int key = (s >> 2) * 8 + g * 4 + (s & 3);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs_[key * C::ROW + db * 32 + r], p[s],
                                                        oacc[db], 0, 0, 0);
    }
  }

  const float l_tot = l_run + swap_halves(l_run);
  const float inv = 1.f / l_tot;
  if (qrow < N) {
    if (g == 0) a.lse[(size_t)bh * N + qrow] = (m_run + fast_log2(l_tot)) * kLn2;
    float* dst = static_cast<float*>(a.o) + head_off + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int d0 = db * 32 + blk * 8 + g * 4;
        *reinterpret_cast<f32x4*>(dst + d0) =
            f32x4{oacc[db][blk * 4] * inv, oacc[db][blk * 4 + 1] * inv,
                  oacc[db][blk * 4 + 2] * inv, oacc[db][blk * 4 + 3] * inv};
      }
  }
}

// ----------------------------------------------------------------------------------------
// Host-side launchers (called by the C ABI after validation).
// ----------------------------------------------------------------------------------------
// Compute units of the current device (the runtime caches the attribute).
static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

template <int D, bool IS_BF16, bool O_F32, bool CAUSAL, int QB, bool DROP, bool SPARSE>
static hipError_t launch16(FwdArgs a, hipStream_t s) {
  using C = Fwd16<D, QB, fwd_bc<D, IS_BF16, CAUSAL, SPARSE>()>;
  a.n_tiles = (a.N + C::BR - 1) / C::BR;
  const int grid = a.n_tiles * a.bh;
  // Two workgroups per CU (two waves per SIMD): a causal grid of more than one and at most two
  // per CU is resident at once, so its long and short tiles are paired per CU.
  a.fold = (CAUSAL && fwd_min_waves<D>() == 2 && grid > cu_count() && grid <= 2 * cu_count() &&
            a.n_tiles > 1) ? 1 : 0;
  constexpr int lds = C::LDS_BYTES + (SPARSE ? kSparseListBytes : 0);
  auto kern = fwd16_kernel<D, IS_BF16, O_F32, CAUSAL, QB, DROP, SPARSE>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), lds, s, a);
  return hipGetLastError();
}

template <int D, bool IS_BF16, bool O_F32, bool CAUSAL>
static hipError_t launch16pp(FwdArgs a, hipStream_t s) {
  using C = FwdPP<D, fwd_tile_keys<D, IS_BF16, CAUSAL>()>;
  a.n_tiles = (a.N + C::BR - 1) / C::BR;
  const int grid = a.n_tiles * a.bh;
  constexpr int lds = C::LDS_BYTES;
  auto kern = fwd16pp_kernel<D, IS_BF16, O_F32, CAUSAL>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::NT), lds, s, a);
  return hipGetLastError();
}

// Plain attention at d <= 128 runs the two-group kernel; dropout, block-sparse masks and d = 256
// the single-group one.
template <int D, bool IS_BF16, bool O_F32, bool DROP, bool SPARSE>
static hipError_t launch16_m(FwdArgs a, bool causal, hipStream_t s) {
  constexpr int QB = fwd_qb<D>();
  if constexpr (!DROP && !SPARSE && D <= 128) {
    // The two-group kernel's 256-query workgroups need enough of them to fill the chip: one per
    // CU without a causal mask, two per CU with one (its workgroups differ in length). Below
    // that (short sequences, few heads) the single-group kernel's 128-query workgroups give
    // twice as many, and a causal grid's longest workgroup is half as long. Measured on MI355X:
    // B=4 H=16 N=1024 d=64 causal 22 vs 25 us, non-causal 28 vs 26 us (two-group faster);
    // B=1 H=16 N=1024 d=128 27 vs 36 us.
    const long long pp_blocks = (long long)((a.N + kPpRows - 1) / kPpRows) * a.bh;
    if (pp_blocks >= (causal ? kFwdPpMinBlocks : kFwdPpMinBlocks / 2))
      return causal ? launch16pp<D, IS_BF16, O_F32, true>(a, s)
                    : launch16pp<D, IS_BF16, O_F32, false>(a, s);
  }
  return causal ? launch16<D, IS_BF16, O_F32, true, QB, DROP, SPARSE>(a, s)
                : launch16<D, IS_BF16, O_F32, false, QB, DROP, SPARSE>(a, s);
}

template <int D, bool IS_BF16, bool O_F32>
static hipError_t launch16_c(FwdArgs a, bool causal, Mode mode, hipStream_t s) {
  switch (mode) {
    case Mode::kDropout: return launch16_m<D, IS_BF16, O_F32, true, false>(a, causal, s);
    case Mode::kSparse: return launch16_m<D, IS_BF16, O_F32, false, true>(a, causal, s);
    default: return launch16_m<D, IS_BF16, O_F32, false, false>(a, causal, s);
  }
}

template <int D>
static hipError_t launch32(FwdArgs a, bool causal, hipStream_t s) {
  constexpr int BR = Fwd32<D, false>::BR;
  constexpr int LDS = Fwd32<D, false>::LDS_BYTES;
  a.n_tiles = (a.N + BR - 1) / BR;
  const int grid = a.n_tiles * a.bh;
  auto kc = fwd32_kernel<D, true>;
  auto kn = fwd32_kernel<D, false>;
  hipLaunchKernelGGL(causal ? kc : kn, dim3(grid), dim3(256), LDS, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch16_d(const FwdArgs& a, bool bf, int o_f32, bool causal, Mode mode,
                             hipStream_t s) {
  if (bf) return o_f32 ? launch16_c<D, true, true>(a, causal, mode, s)
                       : launch16_c<D, true, false>(a, causal, mode, s);
  return o_f32 ? launch16_c<D, false, true>(a, causal, mode, s)
               : launch16_c<D, false, false>(a, causal, mode, s);
}

hipError_t launch_forward(const FwdArgs& a, int d, int in_dtype, int o_f32, bool causal,
                          Mode mode, hipStream_t s) {
  if (in_dtype == 0) {
    if (mode != Mode::kPlain) return hipErrorInvalidValue;  // rejected by the C ABI already
    switch (d) {
      case 32: return launch32<32>(a, causal, s);
      case 64: return launch32<64>(a, causal, s);
      case 96: return launch32<96>(a, causal, s);
      default: return launch32<128>(a, causal, s);
    }
  }
  const bool bf = in_dtype == 2;
  if (d == 256) {  // plain attention only (the C ABI rejects dropout and block masks here)
    if (mode != Mode::kPlain) return hipErrorInvalidValue;
    if (bf) return o_f32 ? launch16_m<256, true, true, false, false>(a, causal, s)
                         : launch16_m<256, true, false, false, false>(a, causal, s);
    return o_f32 ? launch16_m<256, false, true, false, false>(a, causal, s)
                 : launch16_m<256, false, false, false, false>(a, causal, s);
  }
  switch (d) {
    case 32: return launch16_d<32>(a, bf, o_f32, causal, mode, s);
    case 64: return launch16_d<64>(a, bf, o_f32, causal, mode, s);
    case 96: return launch16_d<96>(a, bf, o_f32, causal, mode, s);
    default: return launch16_d<128>(a, bf, o_f32, causal, mode, s);
  }
}

}  // namespace fa
