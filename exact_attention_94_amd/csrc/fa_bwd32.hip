// Backward attention for fp32 inputs on gfx950's true-fp32 MFMA (v_mfma_f32_32x32x2_f32).
//
// Same method as the 16-bit backward ("FlashAttention 为什么不需要存下注意力矩阵" §03 3.3;
// "FlashAttention V1 技术深度解析" §4.2): P is recomputed from the forward's logsumexp,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D)  with  D = rowsum(dO * O),
//   dK = scale * dS^T Q,  dQ = scale * dS K,
// here with every operand and product in fp32, so that the results meet an fp32 tolerance.
// Three kernels run in order: the row sums D, a keys-outer kernel that keeps dK and dV in
// registers, and a queries-outer kernel that keeps dQ in registers (no atomics, deterministic).
//
// MFMA layout (wave64, lane l = 32 g + r): the A operand (32 x 2) takes A[r][g] from lane l, the
// B operand (2 x 32) takes B[g][r], and accumulator slot e of lane l holds C[8(e/4) + 4g + e%4][r].
// A product accumulated over the rows of a previous accumulator therefore walks its contraction
// in 16 steps e, lane group g supplying row 8(e/4) + 4g + e%4 at step e: the accumulator slots
// feed the next MFMA's B operand directly. Tiles are staged in LDS in natural [row][d] order with
// one float of padding per row.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// Row of a 32-row accumulator block held by slot e of lane group g.
__device__ __forceinline__ int acc_row(int e, int g) { return 8 * (e >> 2) + 4 * g + (e & 3); }

// D[row] = rowsum(dO * O) over all B*H*N rows (one thread per row, 16-byte loads).
template <int D>
__global__ __launch_bounds__(256) void bwd32_pre_kernel(BwdArgs a, long long rows) {
  const long long row = (long long)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const float* o = static_cast<const float*>(a.o) + row * D;
  const float* g = static_cast<const float*>(a.dout) + row * D;
  float acc = 0.f;
#pragma unroll 8
  for (int k = 0; k < D; k += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(o + k);
    const f32x4 y = *reinterpret_cast<const f32x4*>(g + k);
    acc += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
  }
  a.delta[row] = acc;
}

template <int D>
struct Bwd32 {
  static constexpr int ROW = D + 1;     // padded LDS row (floats)
  static constexpr int DB = D / 32;     // 32-row blocks of d
  // dK/dV kernel: 2 waves x 32 keys, 32 queries per step.
  static constexpr int KV_NT = 128;
  static constexpr int BKV = 64;
  static constexpr int BQ = 32;
  static constexpr int KV_LDS = (2 * BKV * ROW + 2 * BQ * ROW + 2 * BQ) * 4;
  // dQ kernel: 4 waves x 32 queries, 32 keys per step.
  static constexpr int Q_NT = 256;
  static constexpr int BR = 128;
  static constexpr int BC = 32;
  static constexpr int Q_LDS = 2 * BC * ROW * 4;
};

// Keys outer: workgroup = 64 keys (wave w owns keys k0 + 32 w + r as accumulator columns).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(128) void bwd32_dkdv_kernel(BwdArgs a) {
  using C = Bwd32<D>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem16[];
  float* ks = reinterpret_cast<float*>(smem16);
  float* vs = ks + C::BKV * C::ROW;
  float* qs = vs + C::BKV * C::ROW;
  float* gs = qs + C::BQ * C::ROW;   // dO tile
  float* ls = gs + C::BQ * C::ROW;   // LSE * log2(e) of the step's queries
  float* ds = ls + C::BQ;            // D of the step's queries

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int r = lane & 31;
  const int N = a.N, Nk = a.Nk, qoff = a.qoff;
  const int bh = blockIdx.x % a.bh;
  const int kt = blockIdx.x / a.bh;
  const size_t q_off = (size_t)bh * N * D;
  const size_t kv_off = (size_t)bh * Nk * D;
  const float* qh = static_cast<const float*>(a.q) + q_off;
  const float* gh = static_cast<const float*>(a.dout) + q_off;
  const float* kh = static_cast<const float*>(a.k) + kv_off;
  const float* vh = static_cast<const float*>(a.v) + kv_off;
  const float* lse = a.lse + (size_t)bh * N;
  const float* del = a.delta + (size_t)bh * N;

  const int k0 = kt * C::BKV;
  const int key = k0 + wave * 32 + r;
  for (int e = tid; e < C::BKV * D; e += C::KV_NT) {
    const int j = e / D, c = e % D;
    const bool in = k0 + j < Nk;
    ks[j * C::ROW + c] = in ? kh[(size_t)(k0 + j) * D + c] : 0.f;
    vs[j * C::ROW + c] = in ? vh[(size_t)(k0 + j) * D + c] : 0.f;
  }

  f32x16 dk[C::DB], dv[C::DB];
#pragma unroll
  for (int b = 0; b < C::DB; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[b][e] = 0.f;
      dv[b][e] = 0.f;
    }
  const float c = a.c;
  const float masked = c > 0.f ? -INFINITY : INFINITY;  // c * masked = -inf
  const int q_begin = CAUSAL ? (max(0, k0 - qoff) / C::BQ) * C::BQ : 0;
  const float* kw = ks + (wave * 32 + r) * C::ROW;
  const float* vw = vs + (wave * 32 + r) * C::ROW;

  for (int i0 = q_begin; i0 < N; i0 += C::BQ) {
    __syncthreads();  // the previous step's reads of the Q / dO tiles are done
    for (int e = tid; e < C::BQ * D; e += C::KV_NT) {
      const int i = e / D, cc = e % D;
      const bool in = i0 + i < N;
      qs[i * C::ROW + cc] = in ? qh[(size_t)(i0 + i) * D + cc] : 0.f;
      gs[i * C::ROW + cc] = in ? gh[(size_t)(i0 + i) * D + cc] : 0.f;
    }
    if (tid < C::BQ) {
      const bool in = i0 + tid < N;
      ls[tid] = in ? lse[i0 + tid] * kLog2e : INFINITY;  // rows past N: P = 0
      ds[tid] = in ? del[i0 + tid] : 0.f;
    }
    __syncthreads();
    if (CAUSAL && i0 + C::BQ - 1 + qoff < k0 + wave * 32) continue;  // no query sees these keys

    // S[i][j] and dP[i][j]: rows = the step's queries (A = Q, dO), column = this lane's key.
    f32x16 s, p;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s[e] = 0.f;
      p[e] = 0.f;
    }
#pragma unroll 8
    for (int k = 0; k < D / 2; ++k) {
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[r * C::ROW + 2 * k + g], kw[2 * k + g], s, 0, 0,
                                               0);
      p = __builtin_amdgcn_mfma_f32_32x32x2f32(gs[r * C::ROW + 2 * k + g], vw[2 * k + g], p, 0, 0,
                                               0);
    }
    // P = exp2(c S - LSE log2 e) (masked keys: P = 0); dS = P (dP - D).
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = acc_row(e, g);
      const bool dead = key >= Nk || (CAUSAL && key > i0 + i + qoff);
      const float pv = fast_exp2(__builtin_fmaf(dead ? masked : s[e], c, -ls[i]));
      s[e] = pv;
      p[e] = pv * (p[e] - ds[i]);
    }
    // dV^T[dd][j] += sum_i dO[i][dd] P[i][j]; dK^T[dd][j] += sum_i Q[i][dd] dS[i][j].
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = acc_row(e, g);
#pragma unroll
      for (int b = 0; b < C::DB; ++b) {
        dv[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(gs[i * C::ROW + 32 * b + r], s[e], dv[b], 0,
                                                     0, 0);
        dk[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[i * C::ROW + 32 * b + r], p[e], dk[b], 0,
                                                     0, 0);
      }
    }
  }

  if (key < Nk) {
    float* dkp = static_cast<float*>(a.dk) + kv_off + (size_t)key * D;
    float* dvp = static_cast<float*>(a.dv) + kv_off + (size_t)key * D;
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int d0 = 32 * b + 8 * blk + 4 * g;
        *reinterpret_cast<f32x4*>(dkp + d0) =
            f32x4{dk[b][4 * blk] * a.scale, dk[b][4 * blk + 1] * a.scale,
                  dk[b][4 * blk + 2] * a.scale, dk[b][4 * blk + 3] * a.scale};
        *reinterpret_cast<f32x4*>(dvp + d0) =
            f32x4{dv[b][4 * blk], dv[b][4 * blk + 1], dv[b][4 * blk + 2], dv[b][4 * blk + 3]};
      }
  }
}

// Queries outer: workgroup = 128 queries (wave w owns queries qt0 + 32 w + r as columns).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd32_dq_kernel(BwdArgs a) {
  using C = Bwd32<D>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem16[];
  float* ks = reinterpret_cast<float*>(smem16);
  float* vs = ks + C::BC * C::ROW;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int r = lane & 31;
  const int N = a.N, Nk = a.Nk, qoff = a.qoff;
  const int bh = blockIdx.x % a.bh;
  const int tile = blockIdx.x / a.bh;
  const size_t q_off = (size_t)bh * N * D;
  const size_t kv_off = (size_t)bh * Nk * D;
  const float* kh = static_cast<const float*>(a.k) + kv_off;
  const float* vh = static_cast<const float*>(a.v) + kv_off;

  const int qt0 = tile * C::BR;
  const int qw0 = qt0 + wave * 32;
  const int qrow = qw0 + r;
  const bool qin = qrow < N;
  // Q and dO of this lane's query as B operands: slot k holds element 2k + g.
  float qf[D / 2], gf[D / 2];
  {
    const float* qp = static_cast<const float*>(a.q) + q_off + (size_t)qrow * D;
    const float* gp = static_cast<const float*>(a.dout) + q_off + (size_t)qrow * D;
#pragma unroll
    for (int k = 0; k < D / 2; ++k) {
      qf[k] = qin ? qp[2 * k + g] : 0.f;
      gf[k] = qin ? gp[2 * k + g] : 0.f;
    }
  }
  const float lse2 = qin ? a.lse[(size_t)bh * N + qrow] * kLog2e : INFINITY;
  const float dlt = qin ? a.delta[(size_t)bh * N + qrow] : 0.f;

  f32x16 dq[C::DB];
#pragma unroll
  for (int b = 0; b < C::DB; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[b][e] = 0.f;
  const float c = a.c;
  const float masked = c > 0.f ? -INFINITY : INFINITY;
  const int kv_end = CAUSAL ? min(Nk, qt0 + qoff + C::BR) : Nk;

  for (int j0 = 0; j0 < kv_end; j0 += C::BC) {
    __syncthreads();
    for (int e = tid; e < C::BC * D; e += C::Q_NT) {
      const int j = e / D, cc = e % D;
      const bool in = j0 + j < Nk;
      ks[j * C::ROW + cc] = in ? kh[(size_t)(j0 + j) * D + cc] : 0.f;
      vs[j * C::ROW + cc] = in ? vh[(size_t)(j0 + j) * D + cc] : 0.f;
    }
    __syncthreads();
    if (CAUSAL && j0 > qw0 + 31 + qoff) continue;  // every key after every query of this wave

    // S^T[j][i] and dP^T[j][i]: rows = the tile's keys (A = K, V), column = this lane's query.
    f32x16 s, p;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s[e] = 0.f;
      p[e] = 0.f;
    }
    // Fully unrolled: qf and gf must stay registers (a loop index into them would not).
#pragma unroll
    for (int k = 0; k < D / 2; ++k) {
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[r * C::ROW + 2 * k + g], qf[k], s, 0, 0, 0);
      p = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[r * C::ROW + 2 * k + g], gf[k], p, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int j = j0 + acc_row(e, g);
      const bool dead = j >= Nk || (CAUSAL && j > qrow + qoff);
      const float pv = fast_exp2(__builtin_fmaf(dead ? masked : s[e], c, -lse2));
      p[e] = pv * (p[e] - dlt);  // dS^T
    }
    // dQ^T[dd][i] += sum_j K[j][dd] dS^T[j][i].
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int j = acc_row(e, g);
#pragma unroll
      for (int b = 0; b < C::DB; ++b)
        dq[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[j * C::ROW + 32 * b + r], p[e], dq[b], 0,
                                                     0, 0);
    }
  }

  if (qin) {
    float* dqp = static_cast<float*>(a.dq) + q_off + (size_t)qrow * D;
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int d0 = 32 * b + 8 * blk + 4 * g;
        *reinterpret_cast<f32x4*>(dqp + d0) =
            f32x4{dq[b][4 * blk] * a.scale, dq[b][4 * blk + 1] * a.scale,
                  dq[b][4 * blk + 2] * a.scale, dq[b][4 * blk + 3] * a.scale};
      }
  }
}

template <int D>
static hipError_t launch_bwd32_d(BwdArgs a, bool causal, hipStream_t s) {
  using C = Bwd32<D>;
  const long long rows = (long long)a.bh * a.N;
  hipLaunchKernelGGL(bwd32_pre_kernel<D>, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s,
                     a, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto kv = causal ? bwd32_dkdv_kernel<D, true> : bwd32_dkdv_kernel<D, false>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kv),
                          hipFuncAttributeMaxDynamicSharedMemorySize, C::KV_LDS);
  if (e != hipSuccess) return e;
  const int kv_grid = ((a.Nk + C::BKV - 1) / C::BKV) * a.bh;
  hipLaunchKernelGGL(kv, dim3(kv_grid), dim3(C::KV_NT), C::KV_LDS, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto qk = causal ? bwd32_dq_kernel<D, true> : bwd32_dq_kernel<D, false>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(qk),
                          hipFuncAttributeMaxDynamicSharedMemorySize, C::Q_LDS);
  if (e != hipSuccess) return e;
  const int q_grid = ((a.N + C::BR - 1) / C::BR) * a.bh;
  hipLaunchKernelGGL(qk, dim3(q_grid), dim3(C::Q_NT), C::Q_LDS, s, a);
  return hipGetLastError();
}

hipError_t launch_backward_f32(const BwdArgs& a, int d, bool causal, hipStream_t s) {
  switch (d) {
    case 32: return launch_bwd32_d<32>(a, causal, s);
    case 64: return launch_bwd32_d<64>(a, causal, s);
    case 96: return launch_bwd32_d<96>(a, causal, s);
    default: return launch_bwd32_d<128>(a, causal, s);
  }
}

}  // namespace fa
