// C ABI of the attention library: argument validation, workspace layout and dispatch to the
// kernel launchers. Every check runs before the first HIP call, so an invalid call launches
// nothing and touches no device state.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/fa.h"
#include "fa_kernels.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
static_assert(FA_DECODE_SCRATCH_BYTES == fa::kDecodeScratchBytes, "scratch size mismatch");

bool valid_dtype(int t) { return t == FA_F32 || t == FA_F16 || t == FA_BF16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared shape checks. Returns FA_OK or the status to report. d = 256 passes here; only the
// plain 16-bit forward provides it (the other entry points reject it themselves).
fa_status check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  const long long elems = (long long)B * H * N * d;
  if (elems > 0x7FFFFFFFLL) return FA_ERR_INVALID_ARG;
  // Per-head byte offsets (and the prefetches a few tiles past N) must fit the 32-bit offsets
  // of buffer loads.
  if ((long long)N * d >= (1LL << 30)) return FA_ERR_INVALID_ARG;
  if (d != 32 && d != 64 && d != 96 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// scale * log2(e) as used by the kernels. scale == 0 (uniform attention) maps to a tiny
// positive factor: every exponent then rounds to exactly 2^0 in fp32, which is the same result.
float log2_scale(float scale) {
  const float c = scale * kLog2e;
  return c == 0.f ? 1e-30f : c;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Dropout parameters: keep threshold T = floor((1 - p) * 65536 + 1/2) over 16-bit random values
// and the multiplier 65536 / T of kept probabilities. p must be finite and in [0, 1).
bool make_drop(float p, uint64_t seed, uint32_t offset, fa::DropParams& dp) {
  if (!(p >= 0.f && p < 1.f)) return false;
  const double t = floor((1.0 - (double)p) * 65536.0 + 0.5);
  if (t < 1.0) return false;  // p so close to 1 that nothing would be kept
  dp.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  dp.seed_hi = (uint32_t)(seed >> 32);
  dp.offset = offset;
  dp.keep_t = (uint32_t)t;
  dp.keep_scale = (float)(65536.0 / t);
  dp.log2_scale = (float)log2(65536.0 / t);
  dp.inv_scale = (float)(t / 65536.0);
  return true;
}

// Workspace, each section 256-byte aligned: D (fp32 [B,H,Nq]) | the per-head dO scale 2^-s
// (fp32 [B,H]) | partial maxima of |dO| (kMaxParts words per head) | a debug flag word |
// fp16 copies (16-bit inputs only): dO ([B,H,Nq,d]); for bf16 inputs also Q ([B,H,Nq,d]), K and
// V ([B,H,Nk,d] each).
struct WsLayout {
  size_t gscale_off, dmax_off, flag_off, f16_off, q_elems, k_elems, total;
};

WsLayout workspace_layout(int B, int H, int Nq, int Nk, int d, fa_dtype in_dtype) {
  const size_t bh = (size_t)B * H;
  const size_t rows = bh * Nq;
  WsLayout w;
  w.q_elems = rows * (size_t)d;
  w.k_elems = bh * Nk * (size_t)d;
  w.gscale_off = round_up(rows * sizeof(float), 256);
  w.dmax_off = w.gscale_off + round_up(bh * sizeof(float), 256);
  w.flag_off = w.dmax_off + round_up(bh * fa::kMaxParts * sizeof(uint32_t), 256);
  w.f16_off = w.flag_off + 256;
  // fp32 inputs use their own tensors as operands: no copies.
  const size_t f16_elems = in_dtype == FA_F32 ? 0
                           : w.q_elems + ((in_dtype == FA_BF16) ? (w.q_elems + 2 * w.k_elems) : 0);
  w.total = w.f16_off + f16_elems * 2;
  return w;
}

// Argument checks shared by the backward entry points and their workspace-size queries
// (shapes, dtypes and the mode restrictions). FA_OK if fa_backward* would accept them.
fa_status backward_dtypes_ok(int B, int H, int N, int Nk, int d, fa_dtype in_dtype,
                             fa_dtype o_dtype, fa_dtype grad_dtype, bool extra_mode) {
  if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype) || !valid_dtype(grad_dtype))
    return FA_ERR_INVALID_ARG;
  const fa_status st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (Nk != 0) {
    const fa_status sk = check_shape(B, H, Nk, d);
    if (sk != FA_OK) return sk;
  }
  // d = 256: plain 16-bit attention only (as the forward).
  if (d == 256 && (in_dtype == FA_F32 || extra_mode)) return FA_ERR_UNSUPPORTED;
  if (o_dtype != in_dtype && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (grad_dtype != in_dtype && grad_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  // fp32 inputs: plain attention over N = Nk only (as the fp32 forward).
  if (in_dtype == FA_F32 && (Nk != 0 || extra_mode)) return FA_ERR_UNSUPPORTED;
  if (Nk != 0 && extra_mode) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// FA_DEBUG_CHECKS=1 in the environment turns on the input range check of the backward.
bool debug_checks() {
  const char* e = getenv("FA_DEBUG_CHECKS");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument (null or misaligned pointer, bad size, non-finite scale, bad flag)";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim, dtype combination or mode not provided by this library";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP runtime call or kernel launch failed";
    case FA_ERR_RANGE: return "FA_ERR_RANGE: an input value lies outside the range the backward's fp16 operands hold (|x| >= 65536 or not finite; found by the FA_DEBUG_CHECKS=1 range check)";
  }
  return "unknown fa_status";
}

}  // extern "C"

namespace {

// Block-sparse arguments: a device mask of mask_heads x nb x nb bytes, nb = ceil(N / 128),
// mask_heads 1 or B*H; sequences up to 65536.
fa_status check_sparse(const uint8_t* mask, int mask_heads, int B, int H, int N,
                       fa::SparseParams& sp) {
  if (!mask) return FA_ERR_INVALID_ARG;
  if (mask_heads != 1 && (long long)mask_heads != (long long)B * H) return FA_ERR_INVALID_ARG;
  if (N > fa::kSparseMaxN) return FA_ERR_UNSUPPORTED;
  sp.mask = mask;
  sp.mask_heads = mask_heads;
  sp.nb = (N + fa::kSparseBlock - 1) / fa::kSparseBlock;
  return FA_OK;
}

// Nk = 0: self-attention (Nk = N). Otherwise N query rows attend to Nk >= 1 keys, the queries
// being the last N positions of the key sequence when causal (N <= Nk then).
fa_status forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int N, int d, float scale, int causal, fa_dtype in_dtype,
                       fa_dtype o_dtype, const fa::DropParams* drop,
                       const fa::SparseParams* sparse, void* stream, int Nk = 0) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  const fa_status st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (o_dtype != in_dtype && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if ((drop || sparse) && in_dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (d == 256 && (drop || sparse || in_dtype == FA_F32)) return FA_ERR_UNSUPPORTED;
  if (Nk != 0) {
    const fa_status sk = check_shape(B, H, Nk, d);
    if (sk != FA_OK) return sk;
    if (causal && N > Nk) return FA_ERR_INVALID_ARG;
    if (in_dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  }

  fa::FwdArgs a{};
  fa::Mode mode = fa::Mode::kPlain;
  if (drop) {
    a.drop = *drop;
    mode = fa::Mode::kDropout;
  }
  if (sparse) {
    a.sparse = *sparse;
    mode = fa::Mode::kSparse;
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.N = N;
  a.Nk = Nk != 0 ? Nk : N;
  a.qoff = (Nk != 0 && causal) ? Nk - N : 0;
  a.bh = B * H;
  a.c = log2_scale(scale);
  const hipError_t e = fa::launch_forward(a, d, (int)in_dtype, o_dtype == FA_F32 ? 1 : 0,
                                          causal != 0, mode, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Nk = 0: self-attention (Nk = N); otherwise as in forward_impl (plain mode only).
fa_status backward_impl(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                        int H, int N, int d, float scale, int causal, fa_dtype in_dtype,
                        fa_dtype o_dtype, fa_dtype grad_dtype, const fa::DropParams* drop,
                        const fa::SparseParams* sparse, void* workspace, size_t workspace_bytes,
                        void* stream, int Nk = 0, hipEvent_t ev_before = nullptr,
                        hipEvent_t ev_after = nullptr) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  const fa_status st = backward_dtypes_ok(B, H, N, Nk, d, in_dtype, o_dtype, grad_dtype,
                                          drop != nullptr || sparse != nullptr);
  if (st != FA_OK) return st;
  if (Nk != 0 && causal && N > Nk) return FA_ERR_INVALID_ARG;
  const int nk = Nk != 0 ? Nk : N;
  const WsLayout ws = workspace_layout(B, H, N, nk, d, in_dtype);
  if (!workspace || !aligned16(workspace) || workspace_bytes < ws.total) return FA_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(workspace);

  const hipStream_t hs = static_cast<hipStream_t>(stream);

  // Debug range check (FA_DEBUG_CHECKS=1): bf16 Q, K and V become fp16 operands, which hold
  // |x| < 65520 only; a value beyond that would turn into an infinity and silently spoil the
  // gradients. The check runs before any backward kernel and waits for its answer. (dO needs no
  // check: it is scaled per head into fp16's range.)
  if (in_dtype == FA_BF16 && debug_checks()) {
    uint32_t* flag = reinterpret_cast<uint32_t*>(wsb + ws.flag_off);
    uint32_t host_flag = 0;
    if (fa::launch_clear_flag(flag, hs) != hipSuccess ||
        fa::launch_range_check_bf16(q, ws.q_elems, flag, hs) != hipSuccess ||
        fa::launch_range_check_bf16(k, ws.k_elems, flag, hs) != hipSuccess ||
        fa::launch_range_check_bf16(v, ws.k_elems, flag, hs) != hipSuccess ||
        hipMemcpyAsync(&host_flag, flag, sizeof(host_flag), hipMemcpyDeviceToHost, hs) !=
            hipSuccess ||
        hipStreamSynchronize(hs) != hipSuccess)
      return FA_ERR_HIP;
    if (host_flag != 0) return FA_ERR_RANGE;
  }

  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.delta = static_cast<float*>(workspace);
  a.gscale = reinterpret_cast<float*>(wsb + ws.gscale_off);
  a.dmax = reinterpret_cast<uint32_t*>(wsb + ws.dmax_off);
  uint16_t* f16 = reinterpret_cast<uint16_t*>(wsb + ws.f16_off);
  a.ws_do = f16;
  a.do16 = a.ws_do;
  if (in_dtype == FA_BF16) {
    a.ws_q = a.ws_do + ws.q_elems;
    a.ws_k = a.ws_q + ws.q_elems;
    a.ws_v = a.ws_k + ws.k_elems;
    a.q16 = a.ws_q;
    a.k16 = a.ws_k;
    a.v16 = a.ws_v;
  } else {
    a.q16 = static_cast<const uint16_t*>(q);
    a.k16 = static_cast<const uint16_t*>(k);
    a.v16 = static_cast<const uint16_t*>(v);
  }
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.N = N;
  a.Nk = nk;
  a.qoff = (Nk != 0 && causal) ? Nk - N : 0;
  a.bh = B * H;
  a.scale = scale;
  a.c = log2_scale(scale);
  fa::Mode mode = fa::Mode::kPlain;
  if (drop) {
    a.drop = *drop;
    mode = fa::Mode::kDropout;
  }
  if (sparse) {
    a.sparse = *sparse;
    mode = fa::Mode::kSparse;
  }
  const hipError_t e =
      in_dtype == FA_F32
          ? fa::launch_backward_f32(a, d, causal != 0, hs)
          : fa::launch_backward(a, d, (int)in_dtype, (int)o_dtype, (int)grad_dtype, causal != 0,
                                mode, hs, ev_before, ev_after);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int N, int d, float scale, int causal, fa_dtype in_dtype,
                     fa_dtype o_dtype, void* stream) {
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, in_dtype, o_dtype, nullptr,
                      nullptr, stream);
}

fa_status fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int N, int d, float scale, int causal,
                             fa_dtype in_dtype, fa_dtype o_dtype, float dropout_p, uint64_t seed,
                             uint32_t offset, void* stream) {
  fa::DropParams dp{};
  if (!make_drop(dropout_p, seed, offset, dp)) return FA_ERR_INVALID_ARG;
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, in_dtype, o_dtype, &dp,
                      nullptr, stream);
}

fa_status fa_forward_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int Nq, int Nk, int d, float scale, int causal, fa_dtype in_dtype,
                        fa_dtype o_dtype, void* stream) {
  if (Nk < 1) return FA_ERR_INVALID_ARG;
  return forward_impl(q, k, v, o, lse, B, H, Nq, d, scale, causal, in_dtype, o_dtype, nullptr,
                      nullptr, stream, Nk);
}

fa_status fa_forward_blocksparse(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int B, int H, int N, int d, float scale, int causal,
                                 fa_dtype in_dtype, fa_dtype o_dtype, const uint8_t* block_mask,
                                 int mask_heads, void* stream) {
  fa::SparseParams sp{};
  if (B >= 1 && H >= 1 && N >= 1) {
    const fa_status st = check_sparse(block_mask, mask_heads, B, H, N, sp);
    if (st != FA_OK) return st;
  }
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, in_dtype, o_dtype, nullptr,
                      &sp, stream);
}

size_t fa_backward_workspace_bytes(int B, int H, int N, int d, fa_dtype in_dtype,
                                   fa_dtype grad_dtype) {
  // o_dtype = in_dtype is always accepted, so it does not narrow the check.
  if (backward_dtypes_ok(B, H, N, 0, d, in_dtype, in_dtype, grad_dtype, false) != FA_OK) return 0;
  return workspace_layout(B, H, N, N, d, in_dtype).total;
}

size_t fa_backward_kv_workspace_bytes(int B, int H, int Nq, int Nk, int d, fa_dtype in_dtype,
                                      fa_dtype grad_dtype) {
  if (Nk < 1 || backward_dtypes_ok(B, H, Nq, Nk, d, in_dtype, in_dtype, grad_dtype, false) != FA_OK)
    return 0;
  return workspace_layout(B, H, Nq, Nk, d, in_dtype).total;
}

fa_status fa_backward(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                      int H, int N, int d, float scale, int causal, fa_dtype in_dtype,
                      fa_dtype o_dtype, fa_dtype grad_dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, in_dtype,
                       o_dtype, grad_dtype, nullptr, nullptr, workspace, workspace_bytes, stream);
}

fa_status fa_backward_kv(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int H, int Nq, int Nk, int d, float scale, int causal,
                         fa_dtype in_dtype, fa_dtype o_dtype, fa_dtype grad_dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (Nk < 1) return FA_ERR_INVALID_ARG;
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, d, scale, causal, in_dtype,
                       o_dtype, grad_dtype, nullptr, nullptr, workspace, workspace_bytes, stream,
                       Nk);
}

fa_status fa_backward_dropout(const void* q, const void* k, const void* v, const void* o,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              int B, int H, int N, int d, float scale, int causal,
                              fa_dtype in_dtype, fa_dtype o_dtype, fa_dtype grad_dtype,
                              float dropout_p, uint64_t seed, uint32_t offset, void* workspace,
                              size_t workspace_bytes, void* stream) {
  fa::DropParams dp{};
  if (!make_drop(dropout_p, seed, offset, dp)) return FA_ERR_INVALID_ARG;
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, in_dtype,
                       o_dtype, grad_dtype, &dp, nullptr, workspace, workspace_bytes, stream);
}

fa_status fa_backward_blocksparse(const void* q, const void* k, const void* v, const void* o,
                                  const void* dout, const float* lse, void* dq, void* dk,
                                  void* dv, int B, int H, int N, int d, float scale, int causal,
                                  fa_dtype in_dtype, fa_dtype o_dtype, fa_dtype grad_dtype,
                                  const uint8_t* block_mask, int mask_heads, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  fa::SparseParams sp{};
  if (B >= 1 && H >= 1 && N >= 1) {
    const fa_status st = check_sparse(block_mask, mask_heads, B, H, N, sp);
    if (st != FA_OK) return st;
  }
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, in_dtype,
                       o_dtype, grad_dtype, nullptr, &sp, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Decoding workspace: per (head, chunk, query slot) the unnormalised O (d floats), then the
// (m, l) pairs, each section 256-byte aligned.
struct DecLayout {
  int n_split, chunk, slots;
  size_t ml_off, total;
};

fa_status decode_layout(int B, int H, int Nq, int Nk, int d, DecLayout& L) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if ((long long)B * H * Nk * d > 0x7FFFFFFFLL) return FA_ERR_INVALID_ARG;
  if ((long long)Nk * d >= (1LL << 30)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (Nq > 4) return FA_ERR_UNSUPPORTED;
  if (Nq > Nk) return FA_ERR_INVALID_ARG;
  const int bh = B * H;
  fa::decode_plan(bh, Nk, d, L.n_split, L.chunk);
  L.slots = Nq == 1 ? 1 : 4;
  const size_t parts = (size_t)bh * L.n_split * L.slots;
  L.ml_off = round_up(parts * d * sizeof(float), 256);
  L.total = L.ml_off + round_up(parts * 2 * sizeof(float), 256);
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  DecLayout L;
  return decode_layout(B, H, Nq, Nk, d, L) == FA_OK ? L.total : 0;
}

fa_status fa_decode_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Nq, int Nk, int d, float scale, int causal,
                            fa_dtype in_dtype, fa_dtype o_dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  DecLayout L;
  const fa_status st = decode_layout(B, H, Nq, Nk, d, L);
  if (st != FA_OK) return st;
  if (in_dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (o_dtype != in_dtype && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (!workspace || !aligned16(workspace) || workspace_bytes < L.total) return FA_ERR_WORKSPACE;

  fa::DecArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.ml_off);
  a.Nq = Nq;
  a.Nk = Nk;
  a.bh = B * H;
  a.n_split = L.n_split;
  a.chunk = L.chunk;
  a.c = log2_scale(scale);
  const hipError_t e = fa::launch_decode(a, d, (int)in_dtype, o_dtype == FA_F32, causal != 0,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_decode_forward_noalloc(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                                    int causal, fa_dtype in_dtype, fa_dtype o_dtype,
                                    void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if (!valid_dtype(in_dtype) || !valid_dtype(o_dtype)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  DecLayout L;
  const fa_status st = decode_layout(B, H, Nq, Nk, d, L);
  if (st != FA_OK) return st;
  if (in_dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (o_dtype != in_dtype && o_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (L.total > fa::kDecodeScratchBytes) return FA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (fa::decode_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
  return fa_decode_forward(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, in_dtype, o_dtype,
                           ws, L.total, stream);
}

fa_status fa_backward_timed(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            int B, int H, int N, int d, float scale, int causal,
                            fa_dtype in_dtype, fa_dtype o_dtype, fa_dtype grad_dtype,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* ev_before, void* ev_after) {
  if (!ev_before || !ev_after) return FA_ERR_INVALID_ARG;
  if (in_dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, in_dtype,
                       o_dtype, grad_dtype, nullptr, nullptr, workspace, workspace_bytes, stream,
                       0, static_cast<hipEvent_t>(ev_before), static_cast<hipEvent_t>(ev_after));
}

}  // extern "C"
