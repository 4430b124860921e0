// Tile configuration table of the 16-bit forward kernel: keys per K/V tile for each head
// dimension ("FlashAttention 为什么不需要存下注意力矩阵" §05, first difference: production kernels
// pick their block sizes per head dimension, dtype and causality among precompiled
// configurations, by measurement rather than by formula).
//
// Written by exact_attention_94_amd/tune.py from timings on MI355X (gfx950) of the candidate
// widths 32, 64 and 128 at B=2 H=16 N=4096 causal bf16 (per head dim); each value can be
// overridden at build time with -DFA_FWD_BC_<d>=<keys>. The block-sparse instances always use
// 64 keys (half a 128-key mask block).
#pragma once

#ifndef FA_FWD_BC_32
#define FA_FWD_BC_32 128
#endif
#ifndef FA_FWD_BC_64
#define FA_FWD_BC_64 128
#endif
#ifndef FA_FWD_BC_96
#define FA_FWD_BC_96 64
#endif
#ifndef FA_FWD_BC_128
#define FA_FWD_BC_128 64
#endif
#ifndef FA_FWD_BC_256
#define FA_FWD_BC_256 32
#endif

// LDS operand reads kept in flight ahead of the MFMAs of the score products (forward S, and S
// with dP in both backward kernels); overridable with -DFA_FWD_PRE / -DFA_DKDV_PRE / -DFA_DQ_PRE.
#ifndef FA_FWD_PRE
#define FA_FWD_PRE 4
#endif
#ifndef FA_DKDV_PRE
#define FA_DKDV_PRE 4
#endif
#ifndef FA_DQ_PRE
#define FA_DQ_PRE 4
#endif
// Fewest workgroups for which causal plain attention runs the two-group forward kernel (256
// queries per workgroup; half as many suffice without a causal mask); smaller grids run the
// single-group kernel (128 queries per workgroup).
#ifndef FA_FWD_PP_MIN_BLOCKS
#define FA_FWD_PP_MIN_BLOCKS 512
#endif
// Waves per SIMD the dQ kernel's register allocation must allow at d <= 64.
#ifndef FA_DQ_WAVES_64
#define FA_DQ_WAVES_64 2
#endif

namespace fa {

// Measured at d = 64 only (dK/dV kernel 4% faster); other head dims keep the scheduler's own
// order (at d = 128 the read-ahead makes the dQ kernel spill).
template <int D>
constexpr int fwd_pre() {
  return D == 64 ? FA_FWD_PRE : 0;
}
template <int D>
constexpr int dkdv_pre() {
  return D == 64 ? FA_DKDV_PRE : 0;
}
template <int D>
constexpr int dq_pre() {
  return D == 64 ? FA_DQ_PRE : 0;
}
constexpr int kDqWaves64 = FA_DQ_WAVES_64;
constexpr int kFwdPpMinBlocks = FA_FWD_PP_MIN_BLOCKS;

template <int D>
constexpr int fwd_tile_keys() {
  return D == 32    ? FA_FWD_BC_32
         : D == 64  ? FA_FWD_BC_64
         : D == 96  ? FA_FWD_BC_96
         : D == 128 ? FA_FWD_BC_128
                    : FA_FWD_BC_256;
}

}  // namespace fa
