// Split-KV decoding kernels for gfx950: a few query rows (Nq <= 4, the last positions of the
// sequence) against a long K/V cache (Nk keys).
//
// Method: the online-softmax recurrence ("FlashAttention 为什么不需要存下注意力矩阵" §03 3.2) gives
// the same result for any blocking of the keys, so the keys are cut into chunks processed by
// different workgroups, each producing an unnormalised partial (O_c, m_c, l_c); a second kernel
// merges the chunks with the same rescale, O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
// Flash-Decoding is named (without details) in "FlashAttention V1 技术深度解析" (conclusion) and
// "Flash Attention：一个数学技巧把内存省 5 倍" §七.
//
// With one query row per head there is no matrix product worth a matrix core (an MFMA would use
// 1 of its 32 columns): every K and V byte is read once and used once, so the split kernel is
// HBM-bound and is built for bandwidth. A key row (d = 128 bf16: 256 bytes) is loaded by 16
// lanes with 16-byte buffer loads, up to eight loads per lane and tensor in flight; the partial dot
// products are summed across those lanes, and each lane keeps the running (m, l) and 8 output
// elements of its stream of keys. Streams are merged inside the wave by lane exchanges, then
// across the workgroup's waves through LDS. K and V are read with the non-temporal (streaming)
// cache policy: each byte is used once, so keeping it in the caches only evicts other data
// (measured: 5.7 -> 6.5 TB/s on a 1 GB bf16 cache).
#include <mutex>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <int D, int NQ>
struct Dec {
  static constexpr int LPK = D / 8;        // lanes per key row (8 elements = 16 bytes each)
  static constexpr int KPW = 64 / LPK;     // key rows per wave and load instruction
  // Loads in flight per lane and tensor: 8 for one query row; 4 for four rows, whose
  // accumulators leave fewer registers.
  static constexpr int U = NQ == 1 ? 8 : 4;
  static constexpr int NW = 4;             // waves per workgroup
  static constexpr int KPI = KPW * U * NW; // keys per workgroup iteration
};

// Workgroup = (head, chunk). Writes the chunk's unnormalised O (fp32, per query and d), its
// running maximum m (log2 domain, sentinel -3e38 when nothing was visible) and its sum l.
template <int D, int NQ, bool IS_BF16, bool CAUSAL>
__global__ __launch_bounds__(256) void decode_split_kernel(DecArgs a) {
  using C = Dec<D, NQ>;
  __shared__ float red[C::NW][NQ][C::LPK][10];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane / C::LPK;  // key row within a load
  const int dc = lane % C::LPK;   // 8-element slice of d
  const int split = blockIdx.x % a.n_split;
  const int bh = blockIdx.x / a.n_split;
  const int Nk = a.Nk, Nq = a.Nq;
  const int j_begin = split * a.chunk;
  const int j_end = min(Nk, j_begin + a.chunk);

  // Query slices in fp32, pre-multiplied by scale * log2(e) (rows beyond Nq are zero and
  // never written back).
  float qv[NQ][8];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    u32x4 w = u32x4{0, 0, 0, 0};
    if (qi < Nq) w = ld16(static_cast<const uint16_t*>(a.q) + ((size_t)bh * Nq + qi) * D + dc * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t h = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu));
      qv[qi][e] = to_f32<IS_BF16>(h) * a.c;
    }
  }
  float m[NQ], l[NQ], o[NQ][8];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    m[qi] = -3.0e38f;
    l[qi] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[qi][e] = 0.f;
  }

  const size_t head = (size_t)bh * Nk * D;
  const uint32_t head_bytes = (uint32_t)Nk * D * 2;
  const auto krs = make_rsrc(static_cast<const uint16_t*>(a.k) + head, head_bytes);
  const auto vrs = make_rsrc(static_cast<const uint16_t*>(a.v) + head, head_bytes);

  for (int j0 = j_begin; j0 < j_end; j0 += C::KPI) {
    u32x4 kr[C::U], vr[C::U];
    int key[C::U];
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      key[u] = j0 + (u * C::NW + wave) * C::KPW + sub;
      const uint32_t off = (uint32_t)(key[u] * D + dc * 8) * 2;  // past Nk: zeros
      kr[u] = buf_ld16_stream(krs, off);
      vr[u] = buf_ld16_stream(vrs, off);
    }
    float kf[C::U][8], vf[C::U][8];
#pragma unroll
    for (int u = 0; u < C::U; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) ? 16 : 0;
        kf[u][e] = to_f32<IS_BF16>((uint16_t)((kr[u][e >> 1] >> sh) & 0xFFFFu));
        vf[u][e] = to_f32<IS_BF16>((uint16_t)((vr[u][e >> 1] >> sh) & 0xFFFFu));
      }
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      float s[C::U];
#pragma unroll
      for (int u = 0; u < C::U; ++u) {
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x = __builtin_fmaf(qv[qi][e], kf[u][e], x);
#pragma unroll
        for (int off = 1; off < C::LPK; off <<= 1) x += __shfl_xor(x, off);
        // Keys outside this chunk (or past Nk), and with CAUSAL keys after the query's position
        // Nk - Nq + qi, are invisible.
        const bool dead = key[u] >= j_end || (CAUSAL && key[u] > Nk - Nq + qi);
        s[u] = dead ? -INFINITY : x;
      }
      float mb = s[0];
#pragma unroll
      for (int u = 1; u < C::U; ++u) mb = __builtin_fmaxf(mb, s[u]);
      const float m_new = __builtin_fmaxf(m[qi], mb);
      const float corr = fast_exp2(m[qi] - m_new);
      m[qi] = m_new;
      float p[C::U];
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < C::U; ++u) {
        p[u] = fast_exp2(s[u] - m_new);
        ps += p[u];
      }
      l[qi] = l[qi] * corr + ps;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = o[qi][e] * corr;
#pragma unroll
        for (int u = 0; u < C::U; ++u) acc = __builtin_fmaf(p[u], vf[u][e], acc);
        o[qi][e] = acc;
      }
    }
  }

  // Merge the KPW key streams of the wave (lanes with the same d slice), then the waves.
  auto merge = [](float& m0, float& l0, float (&o0)[8], float m1, float l1, const float (&o1)[8]) {
    const float mm = __builtin_fmaxf(m0, m1);
    const float a0 = fast_exp2(m0 - mm), a1 = fast_exp2(m1 - mm);
    m0 = mm;
    l0 = l0 * a0 + l1 * a1;
#pragma unroll
    for (int e = 0; e < 8; ++e) o0[e] = o0[e] * a0 + o1[e] * a1;
  };
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
#pragma unroll
    for (int off = C::LPK; off < 64; off <<= 1) {
      float o1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o1[e] = __shfl_xor(o[qi][e], off);
      const float m1 = __shfl_xor(m[qi], off), l1 = __shfl_xor(l[qi], off);
      merge(m[qi], l[qi], o[qi], m1, l1, o1);
    }
    if (sub == 0) {
      float* r = red[wave][qi][dc];
      r[0] = m[qi];
      r[1] = l[qi];
#pragma unroll
      for (int e = 0; e < 8; ++e) r[2 + e] = o[qi][e];
    }
  }
  __syncthreads();
  if (wave == 0 && sub == 0) {
    const size_t part = (size_t)bh * a.n_split + split;
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      if (qi >= Nq) break;
#pragma unroll
      for (int w = 1; w < C::NW; ++w) {
        const float* r = red[w][qi][dc];
        float o1[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o1[e] = r[2 + e];
        merge(m[qi], l[qi], o[qi], r[0], r[1], o1);
      }
      float* po = a.part_o + (part * NQ + qi) * D + dc * 8;
      *reinterpret_cast<f32x4*>(po) = f32x4{o[qi][0], o[qi][1], o[qi][2], o[qi][3]};
      *reinterpret_cast<f32x4*>(po + 4) = f32x4{o[qi][4], o[qi][5], o[qi][6], o[qi][7]};
      if (dc == 0) {
        a.part_ml[(part * NQ + qi) * 2] = m[qi];
        a.part_ml[(part * NQ + qi) * 2 + 1] = l[qi];
      }
    }
  }
}

// Block-wide reduction of one float per thread (256 threads) through LDS.
template <bool MAX>
__device__ __forceinline__ float block_reduce(float x, float* scratch) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float y = __shfl_xor(x, off);
    x = MAX ? __builtin_fmaxf(x, y) : x + y;
  }
  const int t = threadIdx.x;
  if ((t & 63) == 0) scratch[t >> 6] = x;
  __syncthreads();
  x = scratch[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) x = MAX ? __builtin_fmaxf(x, scratch[w]) : x + scratch[w];
  __syncthreads();
  return x;
}

// One workgroup of 256 threads per (head, query). The chunks' maxima and weights
// w_c = 2^(m_c - M) are computed once per chunk (threads over chunks); then thread t accumulates
// element t % D of O over the chunks c = t / D (mod 256 / D), with several loads in flight, and
// the 256 / D partial sums are added through LDS. The number of chunks never exceeds
// kDecodeMaxSplit, so their weights fit in LDS.
template <int D, int NQ, bool IS_BF16, bool O_F32>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecArgs a) {
  __shared__ float wts[kDecodeMaxSplit];
  __shared__ float scratch[4];
  __shared__ float osum[256];
  constexpr int G = 256 / D;  // chunk groups
  const int t = threadIdx.x;
  const int qi = blockIdx.x % a.Nq;
  const int bh = blockIdx.x / a.Nq;
  const int ns = a.n_split;
  const size_t base = (size_t)bh * ns;
  float mx = -3.0e38f;
  for (int c = t; c < ns; c += 256) mx = __builtin_fmaxf(mx, a.part_ml[((base + c) * NQ + qi) * 2]);
  mx = block_reduce<true>(mx, scratch);
  float ls = 0.f;
  for (int c = t; c < ns; c += 256) {
    const size_t p = (base + c) * NQ + qi;
    const float w = fast_exp2(a.part_ml[p * 2] - mx);
    wts[c] = w;
    ls = __builtin_fmaf(a.part_ml[p * 2 + 1], w, ls);
  }
  const float lsum = block_reduce<false>(ls, scratch);  // its barrier also publishes wts
  const int dd = t % D, grp = t / D;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int c = grp;
  for (; c + 3 * G < ns; c += 4 * G) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc[u] = __builtin_fmaf(a.part_o[((base + c + u * G) * NQ + qi) * D + dd], wts[c + u * G],
                              acc[u]);
  }
  for (; c < ns; c += G) acc[0] = __builtin_fmaf(a.part_o[((base + c) * NQ + qi) * D + dd], wts[c], acc[0]);
  osum[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (t >= D) return;
  float tot = osum[t];
#pragma unroll
  for (int g2 = 1; g2 < G; ++g2) tot += osum[t + g2 * D];
  const float out = tot / lsum;
  const size_t oi = ((size_t)bh * a.Nq + qi) * D + t;
  if constexpr (O_F32) {
    static_cast<float*>(a.o)[oi] = out;
  } else if constexpr (IS_BF16) {
    static_cast<__bf16*>(a.o)[oi] = (__bf16)out;
  } else {
    static_cast<_Float16*>(a.o)[oi] = (_Float16)out;
  }
  if (t == 0) a.lse[(size_t)bh * a.Nq + qi] = (mx + fast_log2(lsum)) * kLn2;
}

// ----------------------------------------------------------------------------------------
// Host side.
// ----------------------------------------------------------------------------------------
void decode_plan(int bh, int nk, int d, int& n_split, int& chunk) {
  (void)d;
  // Enough workgroups to keep every CU streaming (about 8 per CU), chunks of at least 256 keys
  // and a multiple of 256 (a whole number of workgroup iterations for every instance).
  const int target = kDecodeMaxSplit;
  int want = (target + bh - 1) / bh;
  const int max_split = (nk + 255) / 256;
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  chunk = (nk + want - 1) / want;
  chunk = (chunk + 255) / 256 * 256;
  n_split = (nk + chunk - 1) / chunk;
}

template <int D, int NQ, bool IS_BF16>
static hipError_t launch_dec(const DecArgs& a, bool causal, bool o_f32, hipStream_t s) {
  const int grid = a.bh * a.n_split;
  if (causal)
    hipLaunchKernelGGL((decode_split_kernel<D, NQ, IS_BF16, true>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, NQ, IS_BF16, false>), dim3(grid), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int mgrid = a.bh * a.Nq;
  if (o_f32)
    hipLaunchKernelGGL((decode_merge_kernel<D, NQ, IS_BF16, true>), dim3(mgrid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_merge_kernel<D, NQ, IS_BF16, false>), dim3(mgrid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dec_d(const DecArgs& a, bool bf, bool causal, bool o_f32,
                               hipStream_t s) {
  if (a.Nq == 1)
    return bf ? launch_dec<D, 1, true>(a, causal, o_f32, s) : launch_dec<D, 1, false>(a, causal, o_f32, s);
  return bf ? launch_dec<D, 4, true>(a, causal, o_f32, s) : launch_dec<D, 4, false>(a, causal, o_f32, s);
}

hipError_t launch_decode(const DecArgs& a, int d, int in_dtype, bool o_f32, bool causal,
                         hipStream_t s) {
  const bool bf = in_dtype == 2;
  return d == 64 ? launch_dec_d<64>(a, bf, causal, o_f32, s)
                 : launch_dec_d<128>(a, bf, causal, o_f32, s);
}

// ----------------------------------------------------------------------------------------
// Scratch for the allocation-free decoding entry point: the per-chunk partials live in this
// file-scope device array instead of a caller workspace. Each GPU the library runs on holds its
// own copy until the process ends. In host code `scratch` names a host-side stand-in, not a
// device address, so the kernels only ever receive the address hipGetSymbolAddress reports for
// the current device, fetched once per device and kept below.
// ----------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
