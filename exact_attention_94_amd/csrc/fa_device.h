// Device-side building blocks for the gfx950 attention kernels: MFMA operand types, the
// 32x32 MFMA wrappers, 16-bit conversions and lane exchanges.
//
// MFMA layout used throughout (v_mfma_f32_32x32x16_{bf16,f16}, wave64): lane l = 32*g + r
// (g = l / 32, r = l % 32).
//   A operand (32 x 16): lane l supplies row r, 8 values along the contraction (group g).
//   B operand (16 x 32): lane l supplies column r, the same 8 contraction positions (group g).
//   C (32 x 32, fp32): lane l holds column r, rows 8*(i/4) + 4*g + (i%4) for i = 0..15.
// Only the pairing of A and B contraction slots matters for the result, so any fixed map of
// contraction index -> (g, slot) that both operands share is valid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 8 16-bit values (16 bytes) as raw bits.
struct alignas(16) Frag16 {
  u32x4 w;
};

template <bool IS_BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(const Frag16& a, const Frag16& b, f32x16 c) {
  if constexpr (IS_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.w),
                                                   __builtin_bit_cast(bf16x8, b.w), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a.w),
                                                  __builtin_bit_cast(f16x8, b.w), c, 0, 0, 0);
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even float -> 16-bit storage, two at a time (low half = a); one
// v_cvt_pk_{bf16,f16}_f32 instruction.
template <bool IS_BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 v = {a, b};
  if constexpr (IS_BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
}

template <bool IS_BF16>
__device__ __forceinline__ float to_f32(uint16_t h) {
  if constexpr (IS_BF16) {
    return __uint_as_float((uint32_t)h << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, h);
  }
}

// Value held by lane l ^ 32 (the other half of the wave), through the LDS crossbar.
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// IEEE 754-2019 maximum (NaN propagates, -inf is the identity). Chains of it become
// v_maximum3_f32, without the canonicalising moves that fmaxf's NaN rule costs.
__device__ __forceinline__ float vmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// acc + lo + hi of the two fp16 values packed in w, in fp32: one v_dot2c_f32_f16 against (1, 1).
__device__ __forceinline__ float add_pair_f16(uint32_t w, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
}

// max / sum of x over lanes l and l ^ 32, with one v_permlane32_swap (VALU, no LDS). The swap
// exchanges one half of the wave between its two operands; with both operands = x, the two
// results hold x of lane l and of lane l ^ 32 in some order, so their max / sum is symmetric.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_min(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __builtin_fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;


// Swizzled tile layout (rows of D 16-bit elements, no padding): logical 16-byte chunk c of row r
// is stored at chunk c ^ swz<D>(r). gfx950's LDS has 64 four-byte banks (a 256-byte window); a
// ds_read_b128 is served 16 lanes at a time and a ds_read_b64_tr_b16 32 lanes at a time. The two
// read patterns used on these tiles are:
//   (A) MFMA operand rows: 16 consecutive rows (aligned), one logical chunk each;
//   (B) transposed operand reads: 4 consecutive rows (aligned) x 4 consecutive chunks (aligned).
// swz makes both hit 16 distinct 16-byte bank slots:
//  * D = 64 (two rows per window): (A) needs a bijection of (r / 2) mod 8 for each row parity;
//    (B) needs rows r and r + 2 to differ in bit 2 (they share a window half). Both hold for
//    swz = 4 ((r / 2) mod 2) + (r / 4) mod 4.
//  * D = 128 or 256 (rows a multiple of the window): (A) needs a bijection of r mod 16; (B) needs
//    bits 2..3 to differ between 4 consecutive rows. swz = 4 (r mod 4) + (r / 4) mod 4.
//  * D = 32 or 96 (row starts step through the window by 64 bytes): (A) needs the four rows with
//    the same r mod 4 to differ, swz = (r / 4) mod 4, which only permutes chunks within aligned
//    groups of four; (B) is conflict-free for any such permutation.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 64) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  if constexpr (D % 128 == 0) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (row >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int swz_off(int row, int col) {
  return row * D + ((((col >> 3) ^ swz<D>(row)) << 3) | (col & 7));
}

// MFMA operand (8 x 16-bit, A or B) for lane l = 32*g + n, built from a swizzled LDS tile X of
// D-element rows with two ds_read_b64_tr_b16:
//   slots 0..3 = X[row_lo + s][col0 + n],   slots 4..7 = X[row_hi + s - 4][col0 + n],
// where row_lo / row_hi already include this lane's g. ds_read_b64_tr_b16 works on groups of 16
// lanes: output lane i of a group receives, in slot k, element i % 4 of the 8 bytes addressed
// by lane 4k + i/4 of that group. Lane 4k + j therefore addresses row base + k, columns
// col0 + 16*(n / 16) + 4j .. +3 (8 bytes inside one 16-byte chunk, so the chunk swizzle keeps
// them together), and output lane i gets column col0 + 16*(n / 16) + i = col0 + n.
template <int D>
__device__ __forceinline__ u32x4 lds_tr_frag_swz(const uint16_t* tile, int row_lo, int row_hi,
                                                 int col0) {
  const int lane = threadIdx.x & 63;
  const int col = col0 + (lane & 16) + 4 * (lane & 3);
  const int dr = (lane >> 2) & 3;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(tile + swz_off<D>(row_lo + dr, col)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(tile + swz_off<D>(row_hi + dr, col)));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return u32x4{a[0], a[1], b[0], b[1]};
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a buffer straight into LDS: lane l's data lands at lds + 16 * l
// (lds must be the same for the whole wave). Out-of-range reads deposit zeros.
__device__ __forceinline__ void buf_ld16_lds(__amdgpu_buffer_rsrc_t r, uint32_t byte_off,
                                             uint16_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, byte_off, 0, 0, 0);
}

// Buffer resource over [base, base + bytes): 16-byte loads through it are branch-free and
// return zeros when they fall outside the range (ragged tails need no predication, so the
// compiler can count outstanding loads exactly and keep prefetches in flight).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
// The same load with the non-temporal (streaming) cache policy, for data read exactly once.
__device__ __forceinline__ u32x4 buf_ld16_stream(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}
__device__ __forceinline__ float buf_ldf(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// s_waitcnt vmcnt(0) (expcnt / lgkmcnt left at their maxima): every outstanding vector memory
// load of this wave has completed. Used once before a main loop so that no wait on loads issued
// before it (e.g. register-resident operands) ends up inside the loop, where it would also wait
// for the loop's own prefetches.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier without a memory fence (a fenced __syncthreads would also wait for every
// outstanding load, including prefetches meant to stay in flight). The empty asm statements keep
// the compiler from moving LDS accesses across it, and the scheduling barriers keep every other
// instruction on its side.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// A run of NF MFMAs whose operands come from LDS, fragment f read by read(f) (returning the
// 16 bytes) and consumed by use(f, frag) in that order, with the read of fragment f + PRE
// issued before the MFMA of fragment f. The scheduling barrier after each step keeps that
// order: left alone, the scheduler sinks each read to just ahead of its use to save registers,
// so that every MFMA waits out the LDS latency. Only the order of independent instructions
// changes; the arithmetic is the same.
// PRE = 0 leaves the order to the scheduler.
template <int NF, int PRE, typename Read, typename Use>
__device__ __forceinline__ void read_ahead(Read&& read, Use&& use) {
  static_assert(PRE >= 0, "prefetch depth out of range");
  if constexpr (PRE == 0) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      Frag16 fr;
      fr.w = read(f);
      use(f, fr);
    }
    return;
  }
  constexpr int P = PRE < NF ? PRE : NF;
  Frag16 fr[NF];
#pragma unroll
  for (int f = 0; f < P; ++f) fr[f].w = read(f);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + P < NF) fr[f + P].w = read(f + P);
    use(f, fr[f]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Philox-4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
// 1, 2, 3", SC'11): each round takes the full 64-bit products M0*c0 and M1*c2 and maps
// (c0, c1, c2, c3) to (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key
// advances by the Weyl increments between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // Each 32 x 32 -> 64-bit product as one v_mad_u64_u32 (measured 20% faster per call than
    // separate low and high multiplies).
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    // Three-way XORs as one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c); the compiler
    // otherwise emits two v_xor_b32 per word.
    c0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k0, 0x96);
    c1 = lo1;
    c2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k1, 0x96);
    c3 = lo0;
  }
  return u32x4{c0, c1, c2, c3};
}

// Dropout keep bits of one query and eight consecutive keys 8*group .. 8*group + 7 of head bh:
// bit e is set iff the 16-bit value e of Philox(group, query, bh, offset; seed) is below
// keep_t. The values are the output words' low and high halves in order w0.lo, w0.hi, w1.lo, ...
struct DropParams {
  uint32_t seed_lo, seed_hi, offset, keep_t;
  float keep_scale;  // 65536 / keep_t
  float log2_scale;  // log2(65536 / keep_t)
  float inv_scale;   // keep_t / 65536 (exact)
};

__device__ __forceinline__ uint32_t keep_bits8(const DropParams& dp, uint32_t group,
                                               uint32_t query, uint32_t bh) {
  const u32x4 w = philox4x32_10(group, query, bh, dp.offset, dp.seed_lo, dp.seed_hi);
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t v = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
    bits |= (v < dp.keep_t ? 1u : 0u) << e;
  }
  return bits;
}

// Block-sparse attention: the mask has one byte per (128-query block, 128-key block); a kernel
// visits only the tiles whose block is nonzero. Sequences with more than kSparseMaxN elements are
// rejected by the C ABI, so a workgroup's list of live tiles (64 rows each) fits kSparseListMax
// entries.
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxN = 65536;
constexpr int kSparseListMax = kSparseMaxN / 64;
constexpr int kSparseListBytes = kSparseListMax * 2 + 16;  // the list, then its length

// Compacts the indices t in [0, n) for which live(t) holds into list[0 .. count), in ascending
// order, with wave 0 of the workgroup (one ballot per 64 candidates), and returns count to every
// thread after a workgroup barrier. list and count_slot point into LDS.
template <typename F>
__device__ __forceinline__ int build_live_list(uint16_t* list, int* count_slot, int n, F live) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    int cnt = 0;
    for (int base = 0; base < n; base += 64) {
      const int t = base + tid;
      const bool lv = (t < n) && live(t);
      const unsigned long long bal = __ballot(lv);
      if (lv) list[cnt + __popcll(bal & ((1ull << tid) - 1ull))] = (uint16_t)t;
      cnt += __popcll(bal);
    }
    if (tid == 0) *count_slot = cnt;
  }
  __syncthreads();
  return *count_slot;
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace fa
