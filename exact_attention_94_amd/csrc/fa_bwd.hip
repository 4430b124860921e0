// Backward attention kernels for gfx950.
//
// Method ("FlashAttention 为什么不需要存下注意力矩阵" §03 3.3; "FlashAttention V1 技术深度解析" §4.2):
// the forward kept only O and the per-row logsumexp; the backward walks the tiles again,
// recomputes each probability tile as P = exp(S - LSE), and with G = dO forms
//   dV = P^T G,   dP = G V^T,   dS = P * (dP - D)  with  D = rowsum(dO * O),
//   dK = scale * dS^T Q,   dQ = scale * dS K.
// No N x N matrix is ever written to memory.
//
// Kernels (one stream, in order):
//   1. bwd_absmax: per-head max |dO| (partial maxima, no atomics); for bf16 inputs, the fp16 copy
//                 of Q in the workspace.
//      bwd_pre:   the head's dO scale 2^s (a power of two, 1 for ordinary gradients) from those
//                 maxima; D = 2^s rowsum(dO * O) in fp32 from the forward's output and the fp16
//                 copy of 2^s dO. The gradient epilogues multiply by 2^-s, which is exact.
//   2. bwd_dkdv:  keys outer. One workgroup per tile of 128 keys (4 waves x 32 keys) keeps dK and
//                 dV in registers over all query tiles (causal: those at or below the
//                 diagonal): S, dP, then P, dS, then dV += P^T dO and dK += dS^T Q. For bf16
//                 inputs it converts its own K and V rows to fp16 on load and writes them to the
//                 workspace for the dQ kernel.
//   3. bwd_dq:    queries outer, like the forward. One workgroup per tile of 128 queries keeps
//                 dQ in registers over all key tiles: S^T, dP^T, then dS^T, then
//                 dQ^T += K^T dS^T; dQ is written once, in the output dtype.
// Splitting dQ from dK/dV recomputes S and dP once more (7 products instead of 5) but needs no
// atomics: the fused alternative adds every workgroup's dQ partial into an fp32 accumulator, and
// on this chip those fp32 atomics each reach the memory side (measured: they were 42% of the
// fused kernel's time at B=2 H=16 N=4096 d=64 causal). The result is also deterministic.
//
// All products run on v_mfma_f32_32x32x16_f16 with fp32 accumulation. bf16 Q, K and V are
// converted once to fp16 (exact while 2^-14 <= |x| <= 65504; larger values are outside the
// supported range); dO is scaled per head so that its largest magnitude, and with it dP and dS,
// sits well inside fp16's range whatever the size of the upstream gradient. P and dS are rounded
// to fp16, whose 11-bit significand keeps the gradients of long peaked rows inside the error
// budget that bf16 operands would exceed. Operands that a product needs transposed are read from row-major
// LDS tiles with ds_read_b64_tr_b16, so every tile is staged once, in one layout. Streamed tiles
// (Q / dO in the dK/dV kernel, K / V in the dQ kernel) reach LDS by direct buffer->LDS loads,
// issued one step ahead, into unpadded rows with the chunk swizzle of swz_off.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_tune.h"

namespace fa {

// ----------------------------------------------------------------------------------------
// 1. D = rowsum(dO * O); for bf16 inputs, fp16 copies of Q and dO.
// ----------------------------------------------------------------------------------------
template <bool IS_BF16>
__device__ __forceinline__ u32x4 to_f16x8(u32x4 v) {
  if constexpr (IS_BF16) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      o[w] = pack2<false>(__uint_as_float(v[w] << 16), __uint_as_float(v[w] & 0xFFFF0000u));
    return o;
  } else {
    return v;
  }
}

// Threads per row in the preprocess: one per 8 elements, rounded up to a power of two (the
// row sum is a butterfly over them; the extra threads of d = 96 contribute zero).
template <int D>
constexpr int pre_tpr() {
  return D <= 32 ? 4 : D <= 64 ? 8 : D <= 128 ? 16 : 32;
}

// Largest value of x over the workgroup (256 threads), returned to every thread.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t x, uint32_t* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return max(max(red[0], red[1]), max(red[2], red[3]));
}

// 1a. Max pass. Workgroup bh * n_parts + p covers elements [p * chunk, (p + 1) * chunk) of head
// bh (chunk a multiple of 8192) and writes the largest |dO| there, as the 16-bit magnitude
// pattern (for bf16 and fp16 alike, larger magnitudes have larger patterns), to dmax[bh][p].
// For bf16 inputs it also writes the fp16 copy of the same elements of Q.
template <int D, bool IS_BF16>
__global__ __launch_bounds__(256) void bwd_absmax_kernel(BwdArgs a, int chunk, int n_parts) {
  __shared__ uint32_t red[4];
  const int bh = blockIdx.x / n_parts;
  const int p = blockIdx.x - bh * n_parts;
  const size_t head = (size_t)bh * a.N * D;
  const int n = a.N * D;
  const int beg = p * chunk;
  const int end = min(n, beg + chunk);
  const uint16_t* dout = static_cast<const uint16_t*>(a.dout) + head;
  uint32_t mx = 0;
  // Four 2048-element strides per batch, all loads issued before any use, so that a batch waits
  // for memory once rather than once per stride. The loads are unconditional through buffer
  // resources over the head (zeros past its end); elements past this part's end but inside the
  // head belong to another part of the same head, so counting them leaves the head's maximum
  // unchanged.
  const auto drs = make_rsrc(dout, (uint32_t)n * 2);
  const auto qrs = make_rsrc(static_cast<const uint16_t*>(a.q) + head, (uint32_t)n * 2);
  constexpr int U = 4;
  for (int e0 = beg + (int)threadIdx.x * 8; e0 < end; e0 += U * 2048) {
    u32x4 w[U], qv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t off = (uint32_t)(e0 + u * 2048) * 2;
      w[u] = buf_ld16(drs, off);
      if constexpr (IS_BF16) qv[u] = buf_ld16(qrs, off);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mx = max(mx, max(w[u][i] & 0x7FFFu, (w[u][i] >> 16) & 0x7FFFu));
      if constexpr (IS_BF16)
        if (e0 + u * 2048 < end) st16(a.ws_q + head + e0 + u * 2048, to_f16x8<true>(qv[u]));
    }
  }
  mx = block_max_u32(mx, red);
  if (threadIdx.x == 0) a.dmax[(size_t)bh * kMaxParts + p] = mx;
}

// Exponent s of the dO scale of a head whose largest |dO| is amax: 0 while amax lies in
// [1/2, 16] (ordinary gradients keep their bits), otherwise the s that brings amax into [8, 16),
// clamped to [-120, 120] so that 2^s and 2^-s are normal floats. amax = 0 gives s = 0.
__device__ __forceinline__ int do_scale_exp(float amax) {
  if (!(amax > 0.f) || (amax >= 0.5f && amax <= 16.f)) return 0;
  int ex;
  frexpf(amax, &ex);  // amax = f * 2^ex, f in [1/2, 1)
  return min(120, max(-120, 4 - ex));
}

// Partial maxima per head written by the max pass (at most 64, so that one wave reduces them) and
// row blocks per workgroup of the preprocess: fewer, longer workgroups keep both passes near
// memory bandwidth instead of paying a reduction per few kilobytes.
constexpr int kPreParts = 64;
constexpr int kPreBlocks = 4;
static_assert(kPreParts <= kMaxParts, "partial maxima fit the workspace");

// 1b. Preprocess, workgroup bh * n_rb + rb (row blocks kPreBlocks * rb .. of head bh): the
// head's dO scale 2^s from the partial maxima, then for each row D = 2^s rowsum(dO * O) in fp32
// and the fp16 copy of dO * 2^s (exact scaling, one rounding). Workgroup 0 of each head stores
// 2^-s for the gradient epilogues.
template <int D, bool IS_BF16, bool O_F32>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a, int n_parts, int n_rb) {
  constexpr int TPR = pre_tpr<D>();
  constexpr int RPB = 256 / TPR;
  const int t = threadIdx.x;
  const int bh = blockIdx.x / n_rb;
  const int rb = blockIdx.x - bh * n_rb;
  uint32_t part = (t & 63) < n_parts ? a.dmax[(size_t)bh * kMaxParts + (t & 63)] : 0u;
  // All loads of the workgroup's row blocks first, then the math and the stores. The loads are
  // unconditional through buffer resources over the head: rows past N, and the idle lanes of
  // d = 96 (given an offset past the end), read zeros.
  const int cc = t % TPR;
  const size_t head = (size_t)bh * a.N * D;
  const uint32_t n_el = (uint32_t)a.N * D;
  const auto drs = make_rsrc(static_cast<const uint16_t*>(a.dout) + head, n_el * 2);
  const auto ors = O_F32 ? make_rsrc(static_cast<const float*>(a.o) + head, n_el * 4)
                         : make_rsrc(static_cast<const uint16_t*>(a.o) + head, n_el * 2);
  u32x4 dw[kPreBlocks];
  f32x4 of[kPreBlocks][2];
#pragma unroll
  for (int sub = 0; sub < kPreBlocks; ++sub) {
    const int row = (rb * kPreBlocks + sub) * RPB + t / TPR;
    const uint32_t el = cc < D / 8 ? (uint32_t)row * D + cc * 8 : n_el;
    dw[sub] = buf_ld16(drs, el * 2);
    if constexpr (O_F32) {
      of[sub][0] = __builtin_bit_cast(f32x4, buf_ld16(ors, el * 4));
      of[sub][1] = __builtin_bit_cast(f32x4, buf_ld16(ors, el * 4 + 16));
    } else {
      const u32x4 ow = buf_ld16(ors, el * 2);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        of[sub][w >> 1][2 * (w & 1)] = to_f32<IS_BF16>((uint16_t)(ow[w] & 0xFFFFu));
        of[sub][w >> 1][2 * (w & 1) + 1] = to_f32<IS_BF16>((uint16_t)(ow[w] >> 16));
      }
    }
  }
  // The head's largest |dO| from its n_parts <= 64 partial maxima (loaded above), reduced by each
  // wave on its own (no LDS, no barrier), and the dO scale 2^s it gives.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) part = max(part, (uint32_t)__shfl_xor((int)part, off));
  const float amax = to_f32<IS_BF16>((uint16_t)part);
  const int sexp = do_scale_exp(amax);
  const float up = ldexpf(1.f, sexp);
  if (rb == 0 && t == 0) a.gscale[bh] = ldexpf(1.f, -sexp);
#pragma unroll
  for (int sub = 0; sub < kPreBlocks; ++sub) {
    const int row = (rb * kPreBlocks + sub) * RPB + t / TPR;
    const size_t base = head + (size_t)row * D + cc * 8;
    float dof[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dof[2 * w] = to_f32<IS_BF16>((uint16_t)(dw[sub][w] & 0xFFFFu));
      dof[2 * w + 1] = to_f32<IS_BF16>((uint16_t)(dw[sub][w] >> 16));
    }
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += dof[e] * of[sub][0][e] + dof[4 + e] * of[sub][1][e];
    if (row < a.N && cc < D / 8) {
      u32x4 o16;
#pragma unroll
      for (int w = 0; w < 4; ++w) o16[w] = pack2<false>(dof[2 * w] * up, dof[2 * w + 1] * up);
      st16(a.ws_do + base, o16);
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < a.N && cc == 0) a.delta[(size_t)bh * a.N + row] = acc * up;
  }
}

// Debug range check (see fa_kernels.h).
__global__ __launch_bounds__(256) void clear_flag_kernel(uint32_t* flag) { *flag = 0u; }

__global__ __launch_bounds__(256) void range_check_bf16_kernel(const uint16_t* x, size_t n,
                                                               uint32_t* flag) {
  bool bad = false;
  for (size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8; e < n;
       e += (size_t)gridDim.x * 256 * 8) {
    // n is a multiple of 8 (d >= 32), so whole 16-byte vectors stay in bounds.
    const u32x4 w = ld16(x + e);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      bad |= ((w[i] & 0x7FFFu) >= 0x4780u) || (((w[i] >> 16) & 0x7FFFu) >= 0x4780u);
  }
  if (bad) *flag = 1u;
}

hipError_t launch_clear_flag(uint32_t* flag, hipStream_t s) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, s, flag);
  return hipGetLastError();
}

hipError_t launch_range_check_bf16(const void* x, size_t n, uint32_t* flag, hipStream_t s) {
  const size_t vecs = (n + 7) / 8;
  const int grid = (int)min((size_t)2048, (vecs + 255) / 256);
  hipLaunchKernelGGL(range_check_bf16_kernel, dim3(grid), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), n, flag);
  return hipGetLastError();
}

// Row placement inside a 32-row block of a staged tile: LDS row r holds element
// 16*(a/2) + 8*b + 4*(a%2) + c for r = 8a + 4b + c. An MFMA that reads rows r = 0..31 as its A
// operand then leaves accumulator slot i of lane group g on element 16*(i/8) + 8*g + i%8, i.e.
// contiguous runs of 8 that feed the next MFMA's B operand without any data movement.
__device__ __forceinline__ int perm_row(int e) {
  return 8 * (2 * (e >> 4) + ((e >> 2) & 1)) + 4 * ((e >> 3) & 1) + (e & 3);
}
// Inverse of perm_row: the element placed on LDS row R.
__device__ __forceinline__ int row_key(int R) {
  return 16 * (R >> 4) + 8 * ((R >> 2) & 1) + 4 * ((R >> 3) & 1) + (R & 3);
}

// Workgroup -> (head, tile). With B*H a multiple of 8, each XCD (blockIdx % 8) works on its own
// heads so that one head's tiles share an L2. `reverse` dispatches the highest tile first.
__device__ __forceinline__ void map_bwd_block(int bid, int bh_total, bool reverse, int n_tiles,
                                              int& bh, int& tile) {
  int t;
  if ((bh_total & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3, hp = bh_total >> 3;
    t = slot / hp;
    bh = xcd * hp + (slot - t * hp);
  } else {
    t = bid / bh_total;
    bh = bid - t * bh_total;
  }
  tile = reverse ? n_tiles - 1 - t : t;
}

template <bool G_F32, bool IS_BF16>
__device__ __forceinline__ void store_grad4(void* base, size_t off, float x0, float x1, float x2,
                                            float x3) {
  if constexpr (G_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + off) = f32x4{x0, x1, x2, x3};
  } else {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + off) =
        u32x2{pack2<IS_BF16>(x0, x1), pack2<IS_BF16>(x2, x3)};
  }
}

// ----------------------------------------------------------------------------------------
// 2. dK / dV: keys outer.
// ----------------------------------------------------------------------------------------
// Queries per step of the keys-outer kernel and keys per tile of the queries-outer kernel: from
// the tuning table for plain attention (and, for the queries-outer kernel, dropout); 64 for
// block-sparse masks (half a mask block) and for the keys-outer kernel with dropout, whose keep
// words take the registers that 32-query steps would give to a third wave per SIMD.
template <int D, bool IS_BF16, bool CAUSAL, bool SPARSE, bool DROP = false>
constexpr int dkdv_bq() {
  return (SPARSE || DROP) ? 64 : dkdv_step_queries<D, IS_BF16, CAUSAL>();
}
template <int D, bool IS_BF16, bool CAUSAL, bool SPARSE>
constexpr int dq_bc() {
  return SPARSE ? 64 : dq_tile_keys<D, IS_BF16, CAUSAL>();
}

template <int D, int BQ_>
struct Dkdv {
  static constexpr int NT = 256;       // 4 waves
  static constexpr int BKV = 128;      // keys per workgroup (32 per wave)
  // Queries per step (from the table; 32 at d = 256, where dK and dV alone fill 256 accumulator
  // registers and K and V another 128: one wave per SIMD, the whole register file).
  static constexpr int BQ = BQ_;
  static constexpr int QBS = BQ / 32;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int NW = 4;
  static constexpr int TILE = BQ * D;  // Q / dO tiles: swizzled rows, no padding
  static constexpr int STAGE = 2 * TILE + 2 * BQ * 2;  // Q, dO, then LSE*log2e and D (fp32)
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int LD_INSTR = BQ * D * 2 / 1024;  // 1 KB direct loads per tile and tensor
  // Dropout instances: one 32-bit keep word per (wave, query of the step) after the stages.
  static constexpr int MASK_BYTES = 4 * BQ * 4;
};

// Groups of four waves per workgroup of the keys-outer kernel. Block-sparse instances at d <= 64
// use two: both groups hold the tile's 128 keys and take alternate live query steps, so that a
// mask column much denser than the others (a global key block, seen by every query block) costs
// its workgroup half as long; the groups' dK and dV are added in a fixed order through LDS at
// the end.
template <int D, bool SPARSE>
constexpr int dkdv_groups() {
  return (SPARSE && D <= 64) ? 2 : 1;
}

template <int D, bool IS_BF16, bool G_F32, bool CAUSAL, bool DROP, bool SPARSE>
__global__ __launch_bounds__((256 * dkdv_groups<D, SPARSE>()),
                             (dkdv_waves<D, dkdv_bq<D, IS_BF16, CAUSAL, SPARSE, DROP>(), DROP>()))
void bwd_dkdv_kernel(BwdArgs a) {
  using C = Dkdv<D, dkdv_bq<D, IS_BF16, CAUSAL, SPARSE, DROP>()>;
  constexpr int NG = dkdv_groups<D, SPARSE>();
  static_assert(!(DROP && SPARSE), "the dropout words and the sparse list share one LDS area");
  static_assert(NG == 1 || 4 * 2 * C::DB * 16 * 64 * 4 <= NG * C::LDS_BYTES,
                "the second group's dK / dV fit the stages for the final sum");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Wave-uniform (scalar) indices: group gi, wave within the group.
  const int gi = NG == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 8);
  const int wave = __builtin_amdgcn_readfirstlane(NG == 1 ? tid >> 6 : (tid >> 6) & 3);
  uint16_t* const gsm = smem + gi * 2 * C::STAGE;  // this group's two stages
  const int g = lane >> 5;
  const int r = lane & 31;
  const int N = a.N;    // query rows
  const int Nk = a.Nk;  // keys
  const int qoff = a.qoff;

  int bh, kt;
  map_bwd_block(blockIdx.x, a.bh, false, a.n_tiles, bh, kt);
  const size_t q_off = (size_t)bh * N * D;
  const size_t kv_off = (size_t)bh * Nk * D;
  const auto qrs = make_rsrc(a.q16 + q_off, (uint32_t)N * D * 2);
  // K and V in the input dtype: this kernel is the one that converts them (bf16 inputs).
  const auto krs = make_rsrc(static_cast<const uint16_t*>(a.k) + kv_off, (uint32_t)Nk * D * 2);
  const auto vrs = make_rsrc(static_cast<const uint16_t*>(a.v) + kv_off, (uint32_t)Nk * D * 2);
  const auto dors = make_rsrc(a.do16 + q_off, (uint32_t)N * D * 2);
  const auto lrs = make_rsrc(a.lse + (size_t)bh * N, (uint32_t)N * 4);
  const auto drs = make_rsrc(a.delta + (size_t)bh * N, (uint32_t)N * 4);

  const int k0 = kt * C::BKV;
  const int kw0 = k0 + wave * 32;  // this wave's first key
  const int key = kw0 + r;         // the key this lane owns in every accumulator

  // K and V rows of this wave as B operands: key kw0 + r, d = 16*ks + 8*g .. +8. bf16 inputs are
  // converted to fp16 here (exact in range) and the fp16 rows written to the workspace, where
  // the dQ kernel, launched after this one, streams them.
  Frag16 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const uint32_t off = (uint32_t)(key * D + ks * 16 + g * 8) * 2;
    kf[ks].w = buf_ld16(krs, off);
    vf[ks].w = buf_ld16(vrs, off);
  }
  if constexpr (IS_BF16) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      kf[ks].w = to_f16x8<true>(kf[ks].w);
      vf[ks].w = to_f16x8<true>(vf[ks].w);
    }
    if (gi == 0 && key < Nk) {  // one copy per key (both groups hold the same keys)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const size_t off = kv_off + (size_t)key * D + ks * 16 + g * 8;
        st16(a.ws_k + off, kf[ks].w);
        st16(a.ws_v + off, vf[ks].w);
      }
    }
  }

  f32x16 dvacc[C::DB], dkacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dvacc[db][i] = 0.f;
      dkacc[db][i] = 0.f;
    }

  const float c = a.c;  // never 0 (the host maps scale 0 to a tiny value)
  const float masked = c > 0.f ? -INFINITY : INFINITY;  // c * masked = -inf
  // Causal: query i sees key j iff j <= i + qoff, so the first step that can see this tile holds
  // query k0 - qoff; k0 < Nk = N + qoff keeps at least one step.
  const int q_begin = CAUSAL ? (max(0, k0 - qoff) / C::BQ) * C::BQ : 0;
  const int n_steps = (N - q_begin + C::BQ - 1) / C::BQ;

  // Block-sparse: the query steps (64 rows) whose 128-query block is live in this key tile's
  // column of the block mask (the key tile is exactly one 128-key block), compacted into a list
  // in LDS after the stages; steps past the list's end map past N.
  int n_live = n_steps;
  const uint16_t* live_list = nullptr;
  if constexpr (SPARSE) {
    static_assert(C::BKV == kSparseBlock && 2 * C::BQ == kSparseBlock, "tile / block mismatch");
    uint16_t* list = smem + NG * 2 * C::STAGE;
    const uint8_t* mcol = a.sparse.mask +
        (size_t)(a.sparse.mask_heads == 1 ? 0 : bh) * a.sparse.nb * a.sparse.nb + kt;
    const int nb = a.sparse.nb;
    n_live = build_live_list(list, reinterpret_cast<int*>(list + kSparseListMax), n_steps,
                             [&](int t) {
                               return mcol[(size_t)((q_begin + t * C::BQ) >> 7) * nb] != 0;
                             });
    live_list = list;
  }
  auto step_i0 = [&](int n) -> int {
    if constexpr (SPARSE)
      return n < n_live ? q_begin + (int)live_list[n] * C::BQ : q_begin + n_steps * C::BQ;
    return q_begin + n * C::BQ;
  };

  // Q and dO tiles by direct buffer->LDS loads into swizzled rows (swz_off), rows in perm_row
  // order (LDS row R holds query row_key(R) of the step): lane l of 1 KB load t deposits 16 bytes
  // at element 512 t + 8 l of the tile. The step's LSE and D go through registers, since they
  // are transformed on the way (LSE * log2 e, +inf for rows that must give P = 0).
  constexpr int LPW = C::LD_INSTR / C::NW;  // loads per wave and tensor
  uint32_t toff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int e = (wave + i * C::NW) * 512 + lane * 8;
    const int R = e / D;
    const int cch = ((e % D) >> 3) ^ swz<D>(R);
    toff[i] = (uint32_t)(((R & ~31) + row_key(R & 31)) * D + cch * 8) * 2;
  }
  float lreg, dreg;
  auto issue_tile = [&](int stage, int i0) {
    uint16_t* qs = gsm + stage * C::STAGE;
    uint16_t* os = qs + C::TILE;
    const uint32_t base = (uint32_t)i0 * D * 2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int t = wave + i * C::NW;
      buf_ld16_lds(qrs, base + toff[i], qs + t * 512);
      buf_ld16_lds(dors, base + toff[i], os + t * 512);
    }
    lreg = buf_ldf(lrs, (uint32_t)(i0 + lane) * 4);
    dreg = buf_ldf(drs, (uint32_t)(i0 + lane) * 4);
  };
  // After the loads of issue_tile have completed: the row vectors of the step.
  auto store_vec = [&](int stage, int i0) {
    float* vec = reinterpret_cast<float*>(gsm + stage * C::STAGE + 2 * C::TILE);
    if (wave == 0) {
      // Rows beyond N, and rows that saw no key (LSE = -inf, block-sparse only), get +inf, so
      // that P = 0 there.
      if (lane < C::BQ) {
        // With dropout the row vectors hold LSE log2 e - log2(1/q) and -D q (q the keep rate),
        // so that exp2 gives P / q and the dP accumulators start at -D q (see step_math).
        const float lsh = DROP ? a.drop.log2_scale : 0.f;
        vec[lane] = (i0 + lane < N && lreg != -INFINITY) ? lreg * kLog2e - lsh : INFINITY;
        vec[C::BQ + lane] = DROP ? -dreg * a.drop.inv_scale : -dreg;
      }
    }
  };

  // Math of one query tile already staged in LDS stage `stage`.
  auto step_math = [&](int stage, int i0) {
    const bool live = (i0 < N) && (!CAUSAL || (i0 + C::BQ - 1 + qoff >= kw0));
    if (!live) return;
    const uint16_t* qs = gsm + stage * C::STAGE;
    const uint16_t* os = qs + C::TILE;
    const float* lse_s = reinterpret_cast<const float*>(qs + 2 * C::TILE);
    const float* del_s = lse_s + C::BQ;

    // S = Q K^T and dP = dO V^T (rows: queries in staged order, columns: this wave's keys).
    // The dP accumulators start at -D, with dropout -D q (slot i of block qb: the row vector
    // entry of query 32qb + 16(i/8) + 8g + i%8), so that they end as dP - D (dP - D q); the
    // first MFMA of each chain takes that block as its accumulator input.
    f32x16 sacc[C::QBS], pacc[C::QBS], pinit[C::QBS];
    const f32x16 zero16 = {};
#pragma unroll
    for (int qb = 0; qb < C::QBS; ++qb) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x4 v =
              *reinterpret_cast<const f32x4*>(del_s + qb * 32 + h * 16 + g * 8 + 4 * j);
#pragma unroll
          for (int e = 0; e < 4; ++e) pinit[qb][h * 8 + 4 * j + e] = v[e];
        }
    }
    // Fragment f = (ks, qb, tensor: Q for S, dO for dP), read dkdv_pre<D, BQ>() ahead of its MFMA.
    read_ahead<2 * C::KS * C::QBS, dkdv_pre<D, C::BQ>()>(
        [&](int f) {
          const int ks = f / (2 * C::QBS), qb = (f / 2) % C::QBS;
          const uint16_t* src = (f & 1) ? os : qs;
          return *reinterpret_cast<const u32x4*>(src + swz_off<D>(qb * 32 + r, ks * 16 + g * 8));
        },
        [&](int f, const Frag16& fr) {
          const int ks = f / (2 * C::QBS), qb = (f / 2) % C::QBS;
          if (f & 1) pacc[qb] = mfma32x32x16<false>(fr, vf[ks], ks == 0 ? pinit[qb] : pacc[qb]);
          else sacc[qb] = mfma32x32x16<false>(fr, kf[ks], ks == 0 ? zero16 : sacc[qb]);
        });
    // Mask (keys beyond Nk; causal: key after query + qoff) on the few tiles that need it, as a
    // score of -inf after scaling. Slot i holds query i0 + 32*qb + 16*(i/8) + 8*g + i%8.
    if ((k0 + C::BKV > Nk) || (CAUSAL && (i0 + qoff < kw0 + 31))) {
#pragma unroll
      for (int qb = 0; qb < C::QBS; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = i0 + qb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
          const bool dead = (key >= Nk) || (CAUSAL && key > q + qoff);
          sacc[qb][i] = dead ? masked : sacc[qb][i];
        }
    }
    // Dropout: the keep bits of (query i0 + lane, this wave's 32 keys) come from four Philox
    // blocks of 8 keys; lane (g, r) needs bit r of the words of its own queries, so the words
    // go through this wave's slice of LDS (written and read by the same wave, in order).
    uint32_t* mask_w = nullptr;
    if constexpr (DROP) {
      uint32_t word = 0;
#pragma unroll
      for (int kg = 0; kg < 4; ++kg)
        word |= keep_bits8(a.drop, (uint32_t)(kw0 >> 3) + kg, (uint32_t)(i0 + lane), (uint32_t)bh)
                << (8 * kg);
      mask_w = reinterpret_cast<uint32_t*>(smem + NG * 2 * C::STAGE) + wave * C::BQ;
      mask_w[lane] = word;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // P = exp2(c*S - LSE*log2e); dS = P * (dP - D). With dropout, dV takes the kept P scaled
    // by 1 / keep rate, and dP = (dO V^T) * keep / keep rate; the row vectors then make exp2
    // return P / q directly (q the keep rate).
    Frag16 pfr[C::QBS][2], dsf[C::QBS][2];
#pragma unroll
    for (int qb = 0; qb < C::QBS; ++qb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qloc = qb * 32 + h * 16 + g * 8;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse_s + qloc);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse_s + qloc + 4);
        f32x4 d0 = {}, d1 = {};  // -D q (dropout only)
        if constexpr (DROP) {
          d0 = *reinterpret_cast<const f32x4*>(del_s + qloc);
          d1 = *reinterpret_cast<const f32x4*>(del_s + qloc + 4);
        }
        u32x4 mw0 = u32x4{0, 0, 0, 0}, mw1 = u32x4{0, 0, 0, 0};
        if constexpr (DROP) {
          mw0 = *reinterpret_cast<const u32x4*>(mask_w + qloc);
          mw1 = *reinterpret_cast<const u32x4*>(mask_w + qloc + 4);
        }
        float p[8], ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float lv = e < 4 ? l0[e] : l1[e - 4];
          const float dv = e < 4 ? d0[e] : d1[e - 4];
          const float pv = fast_exp2(__builtin_fmaf(sacc[qb][h * 8 + e], c, -lv));
          if constexpr (DROP) {
            // pv is P / q and the accumulator dP - D q: dS = P (dP / q - D) = pv (dP - D q)
            // where kept, and -P D = pv (-D q) where dropped.
            const uint32_t w = e < 4 ? mw0[e] : mw1[e - 4];
            const bool keep = (w >> r) & 1u;
            p[e] = keep ? pv : 0.f;
            ds[e] = pv * (keep ? pacc[qb][h * 8 + e] : dv);
          } else {
            p[e] = pv;
            (void)dv;
            ds[e] = pv * pacc[qb][h * 8 + e];
          }
        }
        pfr[qb][h].w = u32x4{pack2<false>(p[0], p[1]), pack2<false>(p[2], p[3]),
                             pack2<false>(p[4], p[5]), pack2<false>(p[6], p[7])};
        dsf[qb][h].w = u32x4{pack2<false>(ds[0], ds[1]), pack2<false>(ds[2], ds[3]),
                             pack2<false>(ds[4], ds[5]), pack2<false>(ds[6], ds[7])};
      }
    }
    // dV^T += dO^T P ; dK^T += Q^T dS (rows d, columns = this wave's keys). The A operands are
    // dO / Q read transposed: slots 0..3 = staged rows 32qb + 16h + 4g + s, slots 4..7 the same
    // + 8, which hold queries 32qb + 16h + 8g + s under the row permutation.
#pragma unroll
    for (int qb = 0; qb < C::QBS; ++qb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = qb * 32 + h * 16 + g * 4;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          Frag16 ot, qt;
          ot.w = lds_tr_frag_swz<D>(os, row, row + 8, db * 32);
          qt.w = lds_tr_frag_swz<D>(qs, row, row + 8, db * 32);
          dvacc[db] = mfma32x32x16<false>(ot, pfr[qb][h], dvacc[db]);
          dkacc[db] = mfma32x32x16<false>(qt, dsf[qb][h], dkacc[db]);
        }
      }
    }
  };

  // Prologue: stage the first query tile and retire every earlier load (the K/V operands). Each
  // step then starts the loads of the next tile into the other stage (whose previous tile's math
  // ended before the last barrier), does its math, waits for the loads and publishes the tile.
  // Tiles past N read zeros; their math is skipped.
  // With two groups, group gi takes live steps gi, gi + 2, ...; both run n_it iterations with the
  // same barriers (a step past the last live one maps past N: its loads read zeros, its math is
  // skipped).
  const int n_it = (n_live + NG - 1) / NG;
  auto gstep = [&](int n) { return step_i0(n * NG + gi); };
  issue_tile(0, gstep(0));
  wait_vmem_all();
  store_vec(0, gstep(0));
  __syncthreads();
  // Nothing is loaded or waited for after the last step.
  for (int step = 0; step < n_it; step += 2) {
    const bool more1 = step + 1 < n_it;
    if (more1) issue_tile(1, gstep(step + 1));
    step_math(0, gstep(step));
    if (!more1) break;
    wait_vmem_all();
    store_vec(1, gstep(step + 1));
    __syncthreads();
    const bool more2 = step + 2 < n_it;
    if (more2) issue_tile(0, gstep(step + 2));
    step_math(1, gstep(step + 1));
    if (!more2) break;
    wait_vmem_all();
    store_vec(0, gstep(step + 2));
    __syncthreads();
  }
  if constexpr (NG == 2) {
    // Group 1 hands its dK / dV to group 0 through the (now idle) stages: element (wave, block
    // j, slot i) of lane l at float ((wave * 2 DB + j) * 16 + i) * 64 + l, j < DB for dK.
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    if (gi == 1) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          red[((wave * 2 * C::DB + db) * 16 + i) * 64 + lane] = dkacc[db][i];
          red[((wave * 2 * C::DB + C::DB + db) * 16 + i) * 64 + lane] = dvacc[db][i];
        }
    }
    __syncthreads();
    if (gi == 1) return;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dkacc[db][i] += red[((wave * 2 * C::DB + db) * 16 + i) * 64 + lane];
        dvacc[db][i] += red[((wave * 2 * C::DB + C::DB + db) * 16 + i) * 64 + lane];
      }
  }

  // Epilogue: dK = scale * 2^-s (dK^T acc), dV = 2^-s (dV^T acc), 2^-s undoing the head's dO
  // scale; accumulator rows are d, the column is this lane's key.
  const float gs = a.gscale[bh];
  const float ks_ = a.scale * gs;
  if (key < Nk) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const size_t off = kv_off + (size_t)key * D + db * 32 + blk * 8 + g * 4;
        store_grad4<G_F32, IS_BF16>(a.dk, off, dkacc[db][blk * 4] * ks_,
                                    dkacc[db][blk * 4 + 1] * ks_, dkacc[db][blk * 4 + 2] * ks_,
                                    dkacc[db][blk * 4 + 3] * ks_);
        store_grad4<G_F32, IS_BF16>(a.dv, off, dvacc[db][blk * 4] * gs,
                                    dvacc[db][blk * 4 + 1] * gs, dvacc[db][blk * 4 + 2] * gs,
                                    dvacc[db][blk * 4 + 3] * gs);
      }
    }
  }
}

// ----------------------------------------------------------------------------------------
// 3. dQ: queries outer.
// ----------------------------------------------------------------------------------------
template <int D, int BC_>
struct Dq {
  static constexpr int NT = 256;   // 4 waves x 32 queries
  static constexpr int NW = 4;
  static constexpr int BR = 128;   // queries per workgroup
  // Keys per K/V tile (from the table; 32 at d = 256: fewer score registers next to the
  // 256-wide Q, dO and dQ fragments).
  static constexpr int BC = BC_;
  static constexpr int KB = BC / 32;  // 32-key MFMA blocks per tile
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int TILE = BC * D;     // swizzled rows, no padding
  static constexpr int STAGE = 2 * TILE;  // K then V
  static constexpr int LD_INSTR = BC * D * 2 / 1024;  // 1 KB direct loads per tile and tensor
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
};

template <int D, bool IS_BF16, bool G_F32, bool CAUSAL, bool DROP, bool SPARSE>
__global__ __launch_bounds__(256,
                             (dq_waves<D, dq_bc<D, IS_BF16, CAUSAL, SPARSE>(), !DROP && !SPARSE>()))
void bwd_dq_kernel(BwdArgs a) {
  using C = Dq<D, dq_bc<D, IS_BF16, CAUSAL, SPARSE>()>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int g = lane >> 5;
  const int r = lane & 31;
  const int N = a.N;    // query rows
  const int Nk = a.Nk;  // keys
  const int qoff = a.qoff;

  int bh, tile;
  map_bwd_block(blockIdx.x, a.bh, CAUSAL, a.n_tiles, bh, tile);
  const size_t q_off = (size_t)bh * N * D;
  const size_t kv_off = (size_t)bh * Nk * D;
  const auto qrs = make_rsrc(a.q16 + q_off, (uint32_t)N * D * 2);
  const auto krs = make_rsrc(a.k16 + kv_off, (uint32_t)Nk * D * 2);
  const auto vrs = make_rsrc(a.v16 + kv_off, (uint32_t)Nk * D * 2);
  const auto dors = make_rsrc(a.do16 + q_off, (uint32_t)N * D * 2);
  const auto lrs = make_rsrc(a.lse + (size_t)bh * N, (uint32_t)N * 4);
  const auto drs = make_rsrc(a.delta + (size_t)bh * N, (uint32_t)N * 4);

  const int qt0 = tile * C::BR;
  const int qw0 = qt0 + wave * 32;
  const int qrow = qw0 + r;  // the query this lane owns in every accumulator

  // Q and dO of this lane's query as B operands of S^T = K Q^T and dP^T = V dO^T.
  Frag16 qf[C::KS], of[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const uint32_t off = (uint32_t)(qrow * D + ks * 16 + g * 8) * 2;
    qf[ks].w = buf_ld16(qrs, off);
    of[ks].w = buf_ld16(dors, off);
  }
  // Per-query statistics, lane-local under the transposed layout. Rows beyond N: P = 0.
  const float lse_raw = buf_ldf(lrs, (uint32_t)qrow * 4);
  const float dlt = buf_ldf(drs, (uint32_t)qrow * 4);
  // Initial dP^T accumulator: -D, or with dropout -D q (q the keep rate; the LSE below is then
  // shifted by log2(1/q), so that exp2 gives P / q).
  const float dneg = DROP ? -dlt * a.drop.inv_scale : -dlt;
  f32x16 pinit;
#pragma unroll
  for (int i = 0; i < 16; ++i) pinit[i] = dneg;

  f32x16 dqacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  const float c = a.c;  // never 0 (the host maps scale 0 to a tiny value)
  const float masked = c > 0.f ? -INFINITY : INFINITY;  // c * masked = -inf
  const int kv_end = CAUSAL ? min(Nk, qt0 + qoff + C::BR) : Nk;
  const int n_kt = (kv_end + C::BC - 1) / C::BC;

  // Block-sparse: live K/V tiles of this query tile's row of the block mask (as in the forward).
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

  // K and V tiles by direct buffer->LDS loads into swizzled rows (swz_off); both tensors'
  // rows are placed in perm_row order (LDS row R holds key row_key(R)), since both are A
  // operands whose accumulator rows must map to keys 16*(i/8) + 8*g + i%8. Lane l of 1 KB load
  // t deposits 16 bytes at element 512 t + 8 l of the tile.
  constexpr int LPW = C::LD_INSTR / C::NW;  // loads per wave and tensor
  uint32_t toff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int e = (wave + i * C::NW) * 512 + lane * 8;
    const int R = e / D;
    const int cch = ((e % D) >> 3) ^ swz<D>(R);
    toff[i] = (uint32_t)(((R & ~31) + row_key(R & 31)) * D + cch * 8) * 2;
  }
  auto issue_tile = [&](int stage, int j0) {
    uint16_t* ks_ = smem + stage * C::STAGE;
    uint16_t* vs_ = ks_ + C::TILE;
    const uint32_t base = (uint32_t)j0 * D * 2;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int t = wave + i * C::NW;
      buf_ld16_lds(krs, base + toff[i], ks_ + t * 512);
      buf_ld16_lds(vrs, base + toff[i], vs_ + t * 512);
    }
  };

  issue_tile(0, tile_j0(0));
  wait_vmem_all();
  // Rows beyond N, and rows that saw no key (LSE = -inf, block-sparse only): P = 0.
  const float lse2 = (qrow < N && lse_raw != -INFINITY)
                         ? lse_raw * kLog2e - (DROP ? a.drop.log2_scale : 0.f)
                         : INFINITY;
  __syncthreads();

  auto tile_math = [&](int stage, int j0) {
    const bool live = (j0 < kv_end) && (!CAUSAL || (j0 <= qw0 + qoff + 31));
    if (!live) return;
    const uint16_t* ks_ = smem + stage * C::STAGE;
    const uint16_t* vs_ = ks_ + C::TILE;
    // S^T = K Q^T and dP^T = V dO^T: rows = keys (permuted), column = this lane's query. The dP^T
    // chains start from the block -D of this lane's query (-D q with dropout; pinit), so that
    // they end as dP^T - D (dP^T - D q).
    f32x16 sacc[C::KB], pacc[C::KB];
    const f32x16 zero16 = {};
    // Fragment f = (ks, kb, tensor: K for S^T, V for dP^T), read dq_pre<D, BC>() ahead of its MFMA.
    read_ahead<2 * C::KS * C::KB, dq_pre<D, C::BC>()>(
        [&](int f) {
          const int ks = f / (2 * C::KB), kb = (f / 2) % C::KB;
          const uint16_t* src = (f & 1) ? vs_ : ks_;
          return *reinterpret_cast<const u32x4*>(src + swz_off<D>(kb * 32 + r, ks * 16 + g * 8));
        },
        [&](int f, const Frag16& fr) {
          const int ks = f / (2 * C::KB), kb = (f / 2) % C::KB;
          if (f & 1) pacc[kb] = mfma32x32x16<false>(fr, of[ks], ks == 0 ? pinit : pacc[kb]);
          else sacc[kb] = mfma32x32x16<false>(fr, qf[ks], ks == 0 ? zero16 : sacc[kb]);
        });
    // Mask on the few tiles that need it. Slot i of block kb holds key
    // j0 + 32*kb + 16*(i/8) + 8*g + i%8.
    if ((j0 + C::BC > Nk) || (CAUSAL && (j0 + C::BC - 1 > qw0 + qoff))) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = j0 + kb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
          const bool dead = (kk >= Nk) || (CAUSAL && kk > qrow + qoff);
          sacc[kb][i] = dead ? masked : sacc[kb][i];
        }
    }
    // dS^T = P^T * (dP^T - D), P = exp2(c*S - LSE*log2e); with dropout dP is (dO V^T) * keep /
    // keep rate, the keep bits of this lane's 8 keys coming from one Philox block, and exp2
    // returns P / q (the shifted LSE).
    Frag16 dsf[C::KB][2];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t bits = 0xFFu;
        if constexpr (DROP)
          bits = keep_bits8(a.drop, (uint32_t)(j0 + kb * 32 + h * 16 + g * 8) >> 3,
                            (uint32_t)qrow, (uint32_t)bh);
        float ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = fast_exp2(__builtin_fmaf(sacc[kb][h * 8 + e], c, -lse2));
          if constexpr (DROP) {
            // pv is P / q and the accumulator dP - D q: dS = pv (dP - D q) where kept and
            // pv (-D q) = -P D where dropped.
            ds[e] = pv * (((bits >> e) & 1u) ? pacc[kb][h * 8 + e] : dneg);
          } else {
            ds[e] = pv * pacc[kb][h * 8 + e];
          }
        }
        dsf[kb][h].w = u32x4{pack2<false>(ds[0], ds[1]), pack2<false>(ds[2], ds[3]),
                             pack2<false>(ds[4], ds[5]), pack2<false>(ds[6], ds[7])};
      }
    }
    // dQ^T += K^T dS^T: A = K read transposed (keys 32kb + 16h + 8g + s sit on staged rows
    // 32kb + 16h + 4g + s and + 8), B = dS^T slots.
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = kb * 32 + h * 16 + g * 4;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          Frag16 kt;
          kt.w = lds_tr_frag_swz<D>(ks_, row, row + 8, db * 32);
          dqacc[db] = mfma32x32x16<false>(kt, dsf[kb][h], dqacc[db]);
        }
      }
    }
  };

  // Nothing is loaded or waited for after the last tile.
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

  // Epilogue: dQ = scale * 2^-s (dQ^T acc), 2^-s undoing the head's dO scale; accumulator rows
  // are d = 32db + 8(i/4) + 4g + i%4, the column is this lane's query.
  const float qs_ = a.scale * a.gscale[bh];
  if (qrow < N) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const size_t off = q_off + (size_t)qrow * D + db * 32 + blk * 8 + g * 4;
        store_grad4<G_F32, IS_BF16>(a.dq, off, dqacc[db][blk * 4] * qs_,
                                    dqacc[db][blk * 4 + 1] * qs_, dqacc[db][blk * 4 + 2] * qs_,
                                    dqacc[db][blk * 4 + 3] * qs_);
      }
  }
}

// ----------------------------------------------------------------------------------------
// Launchers.
// ----------------------------------------------------------------------------------------
// Elements per workgroup of the max pass: the head split into at most kPreParts slices of a
// multiple of 8192 elements (256 threads x 8 elements x the pass's batch of 4 strides).
inline int absmax_chunk(long long head_elems) {
  const long long per = (head_elems + kPreParts - 1) / kPreParts;
  return (int)((per + 8191) / 8192 * 8192);
}

template <int D, bool IS_BF16>
static hipError_t launch_pre(const BwdArgs& a, bool o_f32, hipStream_t s) {
  const long long head_elems = (long long)a.N * D;
  const int chunk = absmax_chunk(head_elems);
  const int n_parts = (int)((head_elems + chunk - 1) / chunk);
  hipLaunchKernelGGL((bwd_absmax_kernel<D, IS_BF16>), dim3(n_parts * a.bh), dim3(256), 0, s, a,
                     chunk, n_parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RPB = 256 / pre_tpr<D>();
  const int n_rb = (a.N + RPB * kPreBlocks - 1) / (RPB * kPreBlocks);
  const dim3 grid(n_rb * a.bh);
  if (o_f32)
    hipLaunchKernelGGL((bwd_pre_kernel<D, IS_BF16, true>), grid, dim3(256), 0, s, a, n_parts,
                       n_rb);
  else
    hipLaunchKernelGGL((bwd_pre_kernel<D, IS_BF16, false>), grid, dim3(256), 0, s, a, n_parts,
                       n_rb);
  return hipGetLastError();
}

template <typename K>
static hipError_t launch_dyn(K kern, int grid, int lds, BwdArgs a, hipStream_t s,
                             int threads = 256) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, s, a);
  return hipGetLastError();
}

template <int D, bool IS_BF16, bool G_F32, bool CAUSAL, bool DROP, bool SPARSE>
static hipError_t launch_grads(BwdArgs a, hipStream_t s, hipEvent_t ev_before,
                               hipEvent_t ev_after) {
  hipError_t e;
  if (ev_before && (e = hipEventRecord(ev_before, s)) != hipSuccess) return e;
  using KV = Dkdv<D, dkdv_bq<D, IS_BF16, CAUSAL, SPARSE, DROP>()>;
  using QT = Dq<D, dq_bc<D, IS_BF16, CAUSAL, SPARSE>()>;
  a.n_tiles = (a.Nk + KV::BKV - 1) / KV::BKV;
  constexpr int NG = dkdv_groups<D, SPARSE>();
  e = launch_dyn(bwd_dkdv_kernel<D, IS_BF16, G_F32, CAUSAL, DROP, SPARSE>, a.n_tiles * a.bh,
                 NG * KV::LDS_BYTES + (DROP ? KV::MASK_BYTES : 0) + (SPARSE ? kSparseListBytes : 0),
                 a, s, 256 * NG);
  if (e != hipSuccess) return e;
  if (ev_after && (e = hipEventRecord(ev_after, s)) != hipSuccess) return e;
  a.n_tiles = (a.N + QT::BR - 1) / QT::BR;
  return launch_dyn(bwd_dq_kernel<D, IS_BF16, G_F32, CAUSAL, DROP, SPARSE>, a.n_tiles * a.bh,
                    QT::LDS_BYTES + (SPARSE ? kSparseListBytes : 0), a, s);
}

template <int D, bool IS_BF16, bool G_F32, bool DROP, bool SPARSE>
static hipError_t launch_grads_c(const BwdArgs& a, bool causal, hipStream_t s,
                                 hipEvent_t ev_before, hipEvent_t ev_after) {
  return causal ? launch_grads<D, IS_BF16, G_F32, true, DROP, SPARSE>(a, s, ev_before, ev_after)
                : launch_grads<D, IS_BF16, G_F32, false, DROP, SPARSE>(a, s, ev_before, ev_after);
}

template <int D, bool IS_BF16, bool G_F32>
static hipError_t launch_grads_m(const BwdArgs& a, bool causal, Mode mode, hipStream_t s,
                                 hipEvent_t ev_before, hipEvent_t ev_after) {
  switch (mode) {
    case Mode::kDropout:
      return launch_grads_c<D, IS_BF16, G_F32, true, false>(a, causal, s, ev_before, ev_after);
    case Mode::kSparse:
      return launch_grads_c<D, IS_BF16, G_F32, false, true>(a, causal, s, ev_before, ev_after);
    default:
      return launch_grads_c<D, IS_BF16, G_F32, false, false>(a, causal, s, ev_before, ev_after);
  }
}

template <int D, bool IS_BF16>
static hipError_t launch_all(const BwdArgs& a, bool o_f32, bool g_f32, bool causal, Mode drop,
                             hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after) {
  hipError_t e = launch_pre<D, IS_BF16>(a, o_f32, s);
  if (e != hipSuccess) return e;
  return g_f32 ? launch_grads_m<D, IS_BF16, true>(a, causal, drop, s, ev_before, ev_after)
               : launch_grads_m<D, IS_BF16, false>(a, causal, drop, s, ev_before, ev_after);
}

template <int D, bool IS_BF16>
static hipError_t launch_all_plain(const BwdArgs& a, bool o_f32, bool g_f32, bool causal,
                                   hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after) {
  hipError_t e = launch_pre<D, IS_BF16>(a, o_f32, s);
  if (e != hipSuccess) return e;
  return g_f32 ? launch_grads_c<D, IS_BF16, true, false, false>(a, causal, s, ev_before, ev_after)
               : launch_grads_c<D, IS_BF16, false, false, false>(a, causal, s, ev_before,
                                                                  ev_after);
}

hipError_t launch_backward(const BwdArgs& a, int d, int in_dtype, int o_dtype, int grad_dtype,
                           bool causal, Mode drop, hipStream_t s, hipEvent_t ev_before,
                           hipEvent_t ev_after) {
  const bool bf = in_dtype == 2;
  const bool o_f32 = o_dtype == 0;
  const bool g_f32 = grad_dtype == 0;
  switch (d) {
    case 32:
      return bf ? launch_all<32, true>(a, o_f32, g_f32, causal, drop, s, ev_before, ev_after)
                : launch_all<32, false>(a, o_f32, g_f32, causal, drop, s, ev_before, ev_after);
    case 64:
      return bf ? launch_all<64, true>(a, o_f32, g_f32, causal, drop, s, ev_before, ev_after)
                : launch_all<64, false>(a, o_f32, g_f32, causal, drop, s, ev_before, ev_after);
    case 96:
      return bf ? launch_all<96, true>(a, o_f32, g_f32, causal, drop, s, ev_before, ev_after)
                : launch_all<96, false>(a, o_f32, g_f32, causal, drop, s, ev_before, ev_after);
    case 128:
      return bf ? launch_all<128, true>(a, o_f32, g_f32, causal, drop, s, ev_before, ev_after)
                : launch_all<128, false>(a, o_f32, g_f32, causal, drop, s, ev_before, ev_after);
    default:  // d = 256: plain attention only (the C ABI rejects dropout and block masks here)
      if (drop != Mode::kPlain) return hipErrorInvalidValue;
      return bf ? launch_all_plain<256, true>(a, o_f32, g_f32, causal, s, ev_before, ev_after)
                : launch_all_plain<256, false>(a, o_f32, g_f32, causal, s, ev_before, ev_after);
  }
}

}  // namespace fa
