// Tile configuration table of the 16-bit kernels, per head dimension, input dtype and causality
// ("FlashAttention 为什么不需要存下注意力矩阵" §05, first difference: production kernels pick their
// block sizes per head dimension, dtype and causality among precompiled configurations, by
// measurement rather than by formula):
//   forward:          keys per K/V tile (32, 64 or 128);
//   backward dK/dV:   queries per step of the keys-outer kernel (32 or 64);
//   backward dQ:      keys per K/V tile of the queries-outer kernel (32 or 64).
// A candidate is valid when its tile is a whole number of 1 KB direct loads per wave of four
// (tile * d * 2 bytes a multiple of 4 KB); invalid entries fall back to 64.
//
// The tables below are written by exact_attention_94_amd/tune.py from timings on MI355X (gfx950)
// at B=2 H=16 N=4096 (exact_attention_94_amd/tuning/tiles_mi355x.json). Index order:
// [head dim 32, 64, 96, 128][dtype f16, bf16][causal no, yes]. Candidate builds override every
// entry at once with -DFA_FWD_BC_ALL=<keys>, -DFA_DKDV_BQ_ALL=<queries>, -DFA_DQ_BC_ALL=<keys>.
// Block-sparse instances always use 64 (half a 128 x 128 mask block) and d = 256 its own fixed
// tiles (32 keys forward, 32 queries dK/dV, 32 keys dQ).
#pragma once

#define FA_FWD_BC_TABLE {{{64, 128}, {64, 128}}, {{128, 128}, {128, 128}}, {{64, 64}, {64, 64}}, {{64, 64}, {64, 64}}}
#define FA_DKDV_BQ_TABLE {{{64, 64}, {64, 64}}, {{64, 32}, {64, 32}}, {{64, 64}, {64, 64}}, {{64, 64}, {64, 64}}}
#define FA_DQ_BC_TABLE {{{64, 64}, {64, 64}}, {{64, 32}, {64, 32}}, {{64, 64}, {64, 64}}, {{32, 32}, {32, 32}}}

// LDS operand reads kept in flight ahead of the MFMAs of the score products (forward S, and S
// with dP in both backward kernels); overridable with -DFA_FWD_PRE / -DFA_DKDV_PRE / -DFA_DQ_PRE.
#ifndef FA_FWD_PRE
#define FA_FWD_PRE 4
#endif
#ifndef FA_DKDV_PRE
#define FA_DKDV_PRE 4
#endif
// The same for 32-query steps of the dK/dV kernel, which run three waves per SIMD (fewer
// registers for fragments in flight).
#ifndef FA_DKDV_PRE_32
#define FA_DKDV_PRE_32 2
#endif
#ifndef FA_DQ_PRE
#define FA_DQ_PRE 4
#endif
// The same for 32-key tiles of the dQ kernel, which run three waves per SIMD.
#ifndef FA_DQ_PRE_32
#define FA_DQ_PRE_32 0
#endif
// Fewest workgroups for which causal plain attention runs the two-group forward kernel (256
// queries per workgroup; half as many suffice without a causal mask); smaller grids run the
// single-group kernel (128 queries per workgroup).
#ifndef FA_FWD_PP_MIN_BLOCKS
#define FA_FWD_PP_MIN_BLOCKS 512
#endif
// Waves per SIMD the dK/dV kernel's register allocation must allow at d <= 64: with 64-query
// steps, and with 32-query steps of plain attention (whose score and dP blocks take half the
// registers).
#ifndef FA_DKDV_WAVES_64
#define FA_DKDV_WAVES_64 2
#endif
#ifndef FA_DKDV_WAVES_64_BQ32
#define FA_DKDV_WAVES_64_BQ32 3
#endif
// Waves per SIMD the dQ kernel's register allocation must allow at d <= 64: with 64-key tiles,
// and with 32-key tiles of plain attention.
#ifndef FA_DQ_WAVES_64
#define FA_DQ_WAVES_64 2
#endif
#ifndef FA_DQ_WAVES_64_BC32
#define FA_DQ_WAVES_64_BC32 3
#endif

namespace fa {

// Measured at d = 64 only (dK/dV kernel 4% faster); other head dims keep the scheduler's own
// order (at d = 128 the read-ahead makes the dQ kernel spill).
template <int D>
constexpr int fwd_pre() {
  return D == 64 ? FA_FWD_PRE : 0;
}
template <int D, int BQ>
constexpr int dkdv_pre() {
  return D == 64 ? (BQ == 32 ? FA_DKDV_PRE_32 : FA_DKDV_PRE) : 0;
}
template <int D, int BC>
constexpr int dq_pre() {
  return D == 64 ? (BC == 32 ? FA_DQ_PRE_32 : FA_DQ_PRE) : 0;
}
// Waves per SIMD of the dQ kernel (launch bound): d <= 64 as above (dropout and block masks keep
// two), two at d = 96 and 128, one at d = 256.
template <int D, int BC, bool PLAIN>
constexpr int dq_waves() {
  return D > 128 ? 1 : D > 64 ? 2 : (BC == 32 && PLAIN) ? FA_DQ_WAVES_64_BC32 : FA_DQ_WAVES_64;
}
// Waves per SIMD of the dK/dV kernel (launch bound): d <= 64 as above (dropout keeps the 64-query
// budget: its keep words need the registers), one wave at larger head dims.
template <int D, int BQ, bool DROP>
constexpr int dkdv_waves() {
  return D > 64 ? 1 : (BQ == 32 && !DROP) ? FA_DKDV_WAVES_64_BQ32 : FA_DKDV_WAVES_64;
}
constexpr int kFwdPpMinBlocks = FA_FWD_PP_MIN_BLOCKS;

constexpr int kFwdBcTable[4][2][2] = FA_FWD_BC_TABLE;
constexpr int kDkdvBqTable[4][2][2] = FA_DKDV_BQ_TABLE;
constexpr int kDqBcTable[4][2][2] = FA_DQ_BC_TABLE;

// Row of the tables for a head dimension (32, 64, 96, 128).
template <int D>
constexpr int tune_row() {
  return D == 32 ? 0 : D == 64 ? 1 : D == 96 ? 2 : 3;
}

// Whole 1 KB direct loads for each of four waves: tile * D * 2 bytes a multiple of 4 KB.
template <int D>
constexpr bool whole_loads(int tile) {
  return (tile * D * 2) % 4096 == 0;
}

template <int D>
constexpr int valid_or_64(int tile) {
  return whole_loads<D>(tile) ? tile : 64;
}

template <int D, bool IS_BF16, bool CAUSAL>
constexpr int fwd_tile_keys() {
#ifdef FA_FWD_BC_ALL
  if constexpr (D <= 128) return valid_or_64<D>(FA_FWD_BC_ALL);
#endif
  if constexpr (D > 128) return 32;
  else return valid_or_64<D>(kFwdBcTable[tune_row<D>()][IS_BF16 ? 1 : 0][CAUSAL ? 1 : 0]);
}

template <int D, bool IS_BF16, bool CAUSAL>
constexpr int dkdv_step_queries() {
#ifdef FA_DKDV_BQ_ALL
  if constexpr (D <= 128) return valid_or_64<D>(FA_DKDV_BQ_ALL);
#endif
  if constexpr (D > 128) return 32;
  else return valid_or_64<D>(kDkdvBqTable[tune_row<D>()][IS_BF16 ? 1 : 0][CAUSAL ? 1 : 0]);
}

template <int D, bool IS_BF16, bool CAUSAL>
constexpr int dq_tile_keys() {
#ifdef FA_DQ_BC_ALL
  if constexpr (D <= 128) return valid_or_64<D>(FA_DQ_BC_ALL);
#endif
  if constexpr (D > 128) return 32;
  else return valid_or_64<D>(kDqBcTable[tune_row<D>()][IS_BF16 ? 1 : 0][CAUSAL ? 1 : 0]);
}

}  // namespace fa
