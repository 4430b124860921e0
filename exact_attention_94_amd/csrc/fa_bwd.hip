// Backward attention kernels for gfx950.
//
// Method ("FlashAttention 为什么不需要存下注意力矩阵" §03 3.3; "FlashAttention V1 技术深度解析" §4.2):
// the forward kept only O and the per-row logsumexp; the backward walks the same tiles again,
// recomputes each probability tile as P = exp(S - LSE), and with G = dO forms
//   dV += P^T G,   dP = G V^T,   dS = P * (dP - D)  with  D = rowsum(dO * O),
//   dK += scale * dS^T Q,   dQ += scale * dS K.
// No N x N matrix is ever written to memory.
//
// Kernels (one stream, in order):
//   1. bwd_pre:   D = rowsum(dO * O) in fp32 from the forward's output; zero the fp32 dQ
//                 accumulator; fp16 copies of bf16 Q, K, V, dO.
//   2. bwd_main:  one workgroup per tile of 128 keys (4 waves x 32 keys). dK and dV stay in
//                 registers for the whole loop over query tiles (causal: only tiles at or below
//                 the diagonal). dS goes once through LDS (stored as dS^T, read transposed) and
//                 the workgroup's dQ contribution is added to the fp32 accumulator with atomics.
//   3. dq_cast:   only for 16-bit gradients: fp32 accumulator -> output dtype.
//
// All five products run on v_mfma_f32_32x32x16_f16 with fp32 accumulation. bf16 inputs are
// converted once to fp16 by bwd_pre into the workspace (exact while 2^-14 <= |x| <= 65504);
// P and dS are rounded to fp16, whose 11-bit significand keeps the gradients of long peaked
// rows inside the error budget that bf16 operands would exceed. Operands that the products
// need transposed (Q^T, dO^T, dS, K for dQ) are read from row-major LDS tiles with
// ds_read_b64_tr_b16, so every tile is staged once, in one layout.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// ----------------------------------------------------------------------------------------
// 1. D = rowsum(dO * O); zero dq_acc; for bf16 inputs, fp16 copies of Q, K, V and dO.
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

template <int D, bool IS_BF16, bool O_F32>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a, long long rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const int t = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + t / TPR;
  const int cc = t % TPR;
  float acc = 0.f;
  if (row < rows) {
    const size_t base = (size_t)row * D + cc * 8;
    const u32x4 dw = ld16(static_cast<const uint16_t*>(a.dout) + base);
    float dof[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dof[2 * w] = to_f32<IS_BF16>((uint16_t)(dw[w] & 0xFFFFu));
      dof[2 * w + 1] = to_f32<IS_BF16>((uint16_t)(dw[w] >> 16));
    }
    if constexpr (O_F32) {
      const float* op = static_cast<const float*>(a.o) + base;
      const f32x4 o0 = *reinterpret_cast<const f32x4*>(op);
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(op + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += dof[e] * o0[e] + dof[4 + e] * o1[e];
    } else {
      const u32x4 ow = ld16(static_cast<const uint16_t*>(a.o) + base);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc += dof[2 * w] * to_f32<IS_BF16>((uint16_t)(ow[w] & 0xFFFFu));
        acc += dof[2 * w + 1] * to_f32<IS_BF16>((uint16_t)(ow[w] >> 16));
      }
    }
    float* dq = a.dq_acc + base;
    *reinterpret_cast<f32x4*>(dq) = f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(dq + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (IS_BF16) {
      st16(const_cast<uint16_t*>(a.q16) + base, to_f16x8<true>(ld16(static_cast<const uint16_t*>(a.q) + base)));
      st16(const_cast<uint16_t*>(a.k16) + base, to_f16x8<true>(ld16(static_cast<const uint16_t*>(a.k) + base)));
      st16(const_cast<uint16_t*>(a.v16) + base, to_f16x8<true>(ld16(static_cast<const uint16_t*>(a.v) + base)));
      st16(const_cast<uint16_t*>(a.do16) + base, to_f16x8<true>(dw));
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && cc == 0) a.delta[row] = acc;
}

// ----------------------------------------------------------------------------------------
// 2. Main backward kernel.
// ----------------------------------------------------------------------------------------
// Query row placement inside a 32-row block of the Q / dO LDS tiles: LDS row r holds query
// 16*(a/2) + 8*b + 4*(a%2) + c for r = 8a + 4b + c, so that accumulator slot i of lane group g
// is query 16*(i/8) + 8*g + i%8 (contiguous runs of 8 feed the next MFMA's B operand).
__device__ __forceinline__ int qrow_of_query(int qq) {
  return 8 * (2 * (qq >> 4) + ((qq >> 2) & 1)) + 4 * ((qq >> 3) & 1) + (qq & 3);
}

template <int D>
struct Bwd {
  static constexpr int NW = 4;
  static constexpr int NT = 256;
  static constexpr int BKV = NW * 32;  // keys per workgroup
  static constexpr int BQ = 64;        // queries per inner step
  static constexpr int QBS = BQ / 32;  // 32-query blocks per step
  static constexpr int KS = D / 16;    // contraction steps over d
  static constexpr int DB = D / 32;    // 32-row blocks over d
  static constexpr int QROW = D + 8;   // Q / dO / K tile row stride (elements)
  static constexpr int SROW = BQ + 8;  // dS^T row stride (elements)
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = OFF_Q + BQ * QROW;
  static constexpr int OFF_K = OFF_DO + BQ * QROW;
  static constexpr int OFF_DS = OFF_K + BKV * QROW;
  static constexpr int OFF_VEC = OFF_DS + BKV * SROW;  // 16-bit element offset of the fp32 vectors
  static constexpr int LDS_BYTES = OFF_VEC * 2 + 2 * BQ * 4;
  static constexpr int CHUNKS = BQ * D / 8 / NT;  // 16-byte chunks per thread per tile
  static constexpr int DQ_BLOCKS = QBS * DB / NW; // dQ 32x32 blocks per wave
  static constexpr int MIN_WG = (D == 64) ? 2 : 1;
};

template <int D, bool IS_BF16, bool G_F32, bool CAUSAL>
__global__ __launch_bounds__(256, Bwd<D>::MIN_WG) void bwd_main_kernel(BwdArgs a) {
  using C = Bwd<D>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* Qs = smem + C::OFF_Q;    // [BQ][QROW], rows in qrow_of_query order per 32 block
  uint16_t* dOs = smem + C::OFF_DO;  // same layout as Qs
  uint16_t* Ks = smem + C::OFF_K;    // [BKV][QROW], keys in order
  uint16_t* dSt = smem + C::OFF_DS;  // dS^T: [BKV][SROW], queries in order
  float* lse_s = reinterpret_cast<float*>(smem + C::OFF_VEC);
  float* del_s = lse_s + C::BQ;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int r = lane & 31;
  const int N = a.N;

  // Workgroup -> (head, key tile); causal: the longest (first) key tiles are dispatched first;
  // with B*H a multiple of 8 each XCD works on its own heads.
  int bh, kt;
  if ((a.bh & 7) == 0) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, hp = a.bh >> 3;
    const int t = slot / hp;
    bh = xcd * hp + (slot - t * hp);
    kt = t;
  } else {
    kt = blockIdx.x / a.bh;
    bh = blockIdx.x - kt * a.bh;
  }
  const size_t head_off = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto qrs = make_rsrc(a.q16 + head_off, head_bytes);
  const auto krs = make_rsrc(a.k16 + head_off, head_bytes);
  const auto vrs = make_rsrc(a.v16 + head_off, head_bytes);
  const auto dors = make_rsrc(a.do16 + head_off, head_bytes);
  const auto lrs = make_rsrc(a.lse + (size_t)bh * N, (uint32_t)N * 4);
  const auto drs = make_rsrc(a.delta + (size_t)bh * N, (uint32_t)N * 4);
  const auto dqrs = make_rsrc(a.dq_acc + head_off, (uint32_t)N * D * 4);

  const int k0 = kt * C::BKV;
  const int kw0 = k0 + wave * 32;  // this wave's first key
  const int key = kw0 + r;         // the key this lane owns in every accumulator

  // K and V of this wave as B operands: key kw0 + r, d = 16*ks + 8*g .. +8 (zeros beyond N).
  Frag16 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const uint32_t off = (uint32_t)(key * D + ks * 16 + g * 8) * 2;
    kf[ks].w = buf_ld16(krs, off);
    vf[ks].w = buf_ld16(vrs, off);
  }
  // K of the whole workgroup in LDS (B operand of dQ = dS K, read transposed).
#pragma unroll
  for (int i = 0; i < C::BKV * D / 8 / C::NT; ++i) {
    const int chunk = tid + i * C::NT;
    const int kk = chunk / (D / 8), cc = chunk % (D / 8);
    st16(Ks + kk * C::QROW + cc * 8, buf_ld16(krs, (uint32_t)(k0 * D + chunk * 8) * 2));
  }

  f32x16 dvacc[C::DB], dkacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dvacc[db][i] = 0.f;
      dkacc[db][i] = 0.f;
    }

  const float c = a.c;
  const int q_begin = CAUSAL ? (k0 / C::BQ) * C::BQ : 0;
  const int n_steps = (N - q_begin + C::BQ - 1) / C::BQ;  // >= 1: k0 < N

  // Prefetch registers for one Q / dO tile and its LSE / D values (rows beyond N read as 0;
  // their LSE is set to +inf when staged so that P = 0 there).
  u32x4 qreg[C::CHUNKS], oreg[C::CHUNKS];
  float lreg = 0.f, dreg = 0.f;
  auto load_tile = [&](int i0) {
#pragma unroll
    for (int u = 0; u < C::CHUNKS; ++u) {
      const uint32_t off = (uint32_t)(i0 * D + (tid + u * C::NT) * 8) * 2;
      qreg[u] = buf_ld16(qrs, off);
      oreg[u] = buf_ld16(dors, off);
    }
    lreg = buf_ldf(lrs, (uint32_t)(i0 + lane) * 4);
    dreg = buf_ldf(drs, (uint32_t)(i0 + lane) * 4);
  };
  auto store_tile = [&](int i0) {
#pragma unroll
    for (int u = 0; u < C::CHUNKS; ++u) {
      const int chunk = tid + u * C::NT;
      const int qq = chunk / (D / 8), cc = chunk % (D / 8);
      const int row = (qq & ~31) + qrow_of_query(qq & 31);
      st16(Qs + row * C::QROW + cc * 8, qreg[u]);
      st16(dOs + row * C::QROW + cc * 8, oreg[u]);
    }
    if (wave == 0) {
      lse_s[lane] = (i0 + lane < N) ? lreg * kLog2e : INFINITY;
      del_s[lane] = dreg;
    }
  };

  load_tile(q_begin);
  store_tile(q_begin);
  wait_vmem_all();
  __syncthreads();

  for (int step = 0; step < n_steps; ++step) {
    const int i0 = q_begin + step * C::BQ;
    if (step + 1 < n_steps) load_tile(i0 + C::BQ);

    // ---- phase A: S, P, dP, dS, dV, dK for this wave's 32 keys ----------------------------
    const bool live = !CAUSAL || (i0 + C::BQ - 1 >= kw0);
    if (live) {
      f32x16 sacc[C::QBS], pacc[C::QBS];
#pragma unroll
      for (int qb = 0; qb < C::QBS; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[qb][i] = 0.f;
          pacc[qb][i] = 0.f;
        }
      // S = Q K^T and dP = dO V^T (rows: queries, columns: this wave's keys).
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int qb = 0; qb < C::QBS; ++qb) {
          Frag16 qa, da;
          qa.w = *reinterpret_cast<const u32x4*>(Qs + (qb * 32 + r) * C::QROW + ks * 16 + g * 8);
          da.w = *reinterpret_cast<const u32x4*>(dOs + (qb * 32 + r) * C::QROW + ks * 16 + g * 8);
          sacc[qb] = mfma32x32x16<false>(qa, kf[ks], sacc[qb]);
          pacc[qb] = mfma32x32x16<false>(da, vf[ks], pacc[qb]);
        }
      }
      // P = exp2(c*S - LSE*log2e); dS = P * (dP - D).
      // Slot i: query i0 + 32*qb + 16*(i/8) + 8*g + i%8.
      const bool need_mask = (k0 + C::BKV > N) || (CAUSAL && (i0 < kw0 + 31));
      Frag16 pfr[C::QBS][2], dsf[C::QBS][2];
#pragma unroll
      for (int qb = 0; qb < C::QBS; ++qb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int qloc = qb * 32 + h * 16 + g * 8;
          const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse_s + qloc);
          const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse_s + qloc + 4);
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(del_s + qloc);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(del_s + qloc + 4);
          float p[8], ds[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float lv = e < 4 ? l0[e] : l1[e - 4];
            const float dv = e < 4 ? d0[e] : d1[e - 4];
            float pv = fast_exp2(__builtin_fmaf(sacc[qb][h * 8 + e], c, -lv));
            if (need_mask) {
              const int q = i0 + qloc + e;
              const bool dead = (key >= N) || (CAUSAL && key > q);
              pv = dead ? 0.f : pv;
            }
            p[e] = pv;
            ds[e] = pv * (pacc[qb][h * 8 + e] - dv);
          }
          pfr[qb][h].w = u32x4{pack2<false>(p[0], p[1]), pack2<false>(p[2], p[3]),
                               pack2<false>(p[4], p[5]), pack2<false>(p[6], p[7])};
          dsf[qb][h].w = u32x4{pack2<false>(ds[0], ds[1]), pack2<false>(ds[2], ds[3]),
                               pack2<false>(ds[4], ds[5]), pack2<false>(ds[6], ds[7])};
          // dS^T[key][queries qloc .. qloc + 7] for the dQ product.
          st16(dSt + (wave * 32 + r) * C::SROW + qloc, dsf[qb][h].w);
        }
      }
      // dV^T += dO^T P ; dK^T += Q^T dS   (rows d, columns = this wave's keys). The A operands
      // are Q / dO read transposed: slots 0..3 = LDS rows 32qb + 16h + 4g + s, slots 4..7 the
      // same + 8 (queries 16h + 8g + s under the row permutation).
#pragma unroll
      for (int qb = 0; qb < C::QBS; ++qb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = qb * 32 + h * 16 + g * 4;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            Frag16 ot, qt;
            ot.w = lds_tr_frag(dOs, C::QROW, row, row + 8, db * 32);
            qt.w = lds_tr_frag(Qs, C::QROW, row, row + 8, db * 32);
            dvacc[db] = mfma32x32x16<false>(ot, pfr[qb][h], dvacc[db]);
            dkacc[db] = mfma32x32x16<false>(qt, dsf[qb][h], dkacc[db]);
          }
        }
      }
    } else {
      // Keys entirely after every query of this tile: dS is 0 for them.
#pragma unroll
      for (int qq = 0; qq < C::BQ; qq += 8) st16(dSt + (wave * 32 + r) * C::SROW + qq, u32x4{0, 0, 0, 0});
    }
    __syncthreads();

    // ---- phase B: next tile into LDS; dQ(tile) += scale * dS K over the 128 keys ------------
    if (step + 1 < n_steps) store_tile(i0 + C::BQ);
#pragma unroll
    for (int bi = 0; bi < C::DQ_BLOCKS; ++bi) {
      const int blk = wave * C::DQ_BLOCKS + bi;
      const int qb = blk / C::DB, db = blk % C::DB;
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int t = 0; t < C::BKV / 16; ++t) {
        // A = dS[q = 32qb + r][keys 16t + 8g + s], B = K[keys 16t + 8g + s][d = 32db + r].
        Frag16 sa, kb;
        sa.w = lds_tr_frag(dSt, C::SROW, t * 16 + g * 8, t * 16 + g * 8 + 4, qb * 32);
        kb.w = lds_tr_frag(Ks, C::QROW, t * 16 + g * 8, t * 16 + g * 8 + 4, db * 32);
        acc = mfma32x32x16<false>(sa, kb, acc);
      }
      // acc: column d = 32*db + r, rows = queries 8*(i/4) + 4*g + i%4 of block qb.
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = i0 + qb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        buf_atomic_add(dqrs, (uint32_t)(q * D + db * 32 + r) * 4, acc[i] * a.scale);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: dK = scale * dK^T acc, dV = dV^T acc, rows = this lane's key ---------------
  if (key < N) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int d0 = db * 32 + blk * 8 + g * 4;
        const size_t off = head_off + (size_t)key * D + d0;
        const float k0v = dkacc[db][blk * 4] * a.scale, k1v = dkacc[db][blk * 4 + 1] * a.scale;
        const float k2v = dkacc[db][blk * 4 + 2] * a.scale, k3v = dkacc[db][blk * 4 + 3] * a.scale;
        const float v0 = dvacc[db][blk * 4], v1 = dvacc[db][blk * 4 + 1];
        const float v2 = dvacc[db][blk * 4 + 2], v3 = dvacc[db][blk * 4 + 3];
        if constexpr (G_F32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.dk) + off) = f32x4{k0v, k1v, k2v, k3v};
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.dv) + off) = f32x4{v0, v1, v2, v3};
        } else {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.dk) + off) =
              u32x2{pack2<IS_BF16>(k0v, k1v), pack2<IS_BF16>(k2v, k3v)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.dv) + off) =
              u32x2{pack2<IS_BF16>(v0, v1), pack2<IS_BF16>(v2, v3)};
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------------------
// 3. fp32 dQ accumulator -> 16-bit dQ.
// ----------------------------------------------------------------------------------------
template <bool IS_BF16>
__global__ __launch_bounds__(256) void dq_cast_kernel(const float* __restrict__ src,
                                                      uint16_t* __restrict__ dst, long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(src + i * 8);
  const f32x4 b = *reinterpret_cast<const f32x4*>(src + i * 8 + 4);
  st16(dst + i * 8, u32x4{pack2<IS_BF16>(a[0], a[1]), pack2<IS_BF16>(a[2], a[3]),
                          pack2<IS_BF16>(b[0], b[1]), pack2<IS_BF16>(b[2], b[3])});
}

// ----------------------------------------------------------------------------------------
// Launchers.
// ----------------------------------------------------------------------------------------
template <int D, bool IS_BF16>
static hipError_t launch_pre(const BwdArgs& a, bool o_f32, hipStream_t s) {
  const long long rows = (long long)a.bh * a.N;
  constexpr int RPB = 256 / (D / 8);
  const int grid = (int)((rows + RPB - 1) / RPB);
  if (o_f32)
    hipLaunchKernelGGL((bwd_pre_kernel<D, IS_BF16, true>), dim3(grid), dim3(256), 0, s, a, rows);
  else
    hipLaunchKernelGGL((bwd_pre_kernel<D, IS_BF16, false>), dim3(grid), dim3(256), 0, s, a, rows);
  return hipGetLastError();
}

template <int D, bool IS_BF16, bool G_F32, bool CAUSAL>
static hipError_t launch_main(BwdArgs a, hipStream_t s) {
  using C = Bwd<D>;
  a.n_tiles = (a.N + C::BKV - 1) / C::BKV;
  auto kern = bwd_main_kernel<D, IS_BF16, G_F32, CAUSAL>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.n_tiles * a.bh), dim3(C::NT), C::LDS_BYTES, s, a);
  return hipGetLastError();
}

template <int D, bool IS_BF16>
static hipError_t launch_all(const BwdArgs& a, bool o_f32, bool g_f32, bool causal,
                             hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after) {
  hipError_t e = launch_pre<D, IS_BF16>(a, o_f32, s);
  if (e != hipSuccess) return e;
  if (ev_before && (e = hipEventRecord(ev_before, s)) != hipSuccess) return e;
  if (g_f32)
    e = causal ? launch_main<D, IS_BF16, true, true>(a, s) : launch_main<D, IS_BF16, true, false>(a, s);
  else
    e = causal ? launch_main<D, IS_BF16, false, true>(a, s) : launch_main<D, IS_BF16, false, false>(a, s);
  if (e != hipSuccess) return e;
  if (ev_after && (e = hipEventRecord(ev_after, s)) != hipSuccess) return e;
  if (!g_f32) {
    const long long n8 = (long long)a.bh * a.N * D / 8;
    hipLaunchKernelGGL((dq_cast_kernel<IS_BF16>), dim3((unsigned)((n8 + 255) / 256)), dim3(256),
                       0, s, a.dq_acc, static_cast<uint16_t*>(a.dq), n8);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_backward(const BwdArgs& a, int d, int in_dtype, int o_dtype, int grad_dtype,
                           bool causal, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after) {
  const bool bf = in_dtype == 2;
  const bool o_f32 = o_dtype == 0;
  const bool g_f32 = grad_dtype == 0;
  if (d == 64) return bf ? launch_all<64, true>(a, o_f32, g_f32, causal, s, ev_before, ev_after)
                         : launch_all<64, false>(a, o_f32, g_f32, causal, s, ev_before, ev_after);
  return bf ? launch_all<128, true>(a, o_f32, g_f32, causal, s, ev_before, ev_after)
            : launch_all<128, false>(a, o_f32, g_f32, causal, s, ev_before, ev_after);
}

}  // namespace fa
