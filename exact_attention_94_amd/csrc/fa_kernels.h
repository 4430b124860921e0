// Kernel argument blocks and launcher entry points shared by the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fa_device.h"

namespace fa {

// Block mask [mask_heads][nb][nb] (device memory, one byte per 128 x 128 block, nonzero = live),
// nb = ceil(N / 128); mask_heads is 1 (shared by all heads) or B*H.
struct SparseParams {
  const uint8_t* mask;
  int mask_heads;
  int nb;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int N;        // query rows per head (the sequence length unless Nk says otherwise)
  int Nk;       // keys per head (= N for self-attention)
  int qoff;     // position of query row 0 in the key sequence (causal alignment), usually 0
  int bh;       // B * H
  int n_tiles;  // query tiles per head (set by the launcher)
  // Causal grids resident in one round at two workgroups per CU (set by the launcher): the
  // second half of the tile order runs shortest-first, so that each CU pairs a long query tile
  // with a short one.
  int fold;
  float c;      // scale * log2(e), never 0
  DropParams drop;  // used only by the dropout instances
  SparseParams sparse;  // used only by the block-sparse instances
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // float32 [B,H,N]: rowsum(dO * O) * 2^s_bh (the head's dO scale, below)
  // Per-head power-of-two scaling of dO: the fp16 operand copy of dO holds dO * 2^s_bh, chosen
  // from the head's max |dO| so that small or large upstream gradients keep fp16's precision;
  // gscale[bh] = 2^-s_bh undoes it in the gradient epilogues. dmax holds kMaxParts partial
  // maxima of |dO| per head (16-bit magnitude patterns) for the preprocess to reduce.
  float* gscale;
  uint32_t* dmax;
  // fp16 operands of the gradient kernels: Q, K and V are the inputs themselves for fp16 inputs
  // and fp16 copies in the workspace for bf16 inputs (ws_q written by the max pass, ws_k and
  // ws_v by the dK/dV kernel for the dQ kernel after it; null for fp16 inputs); dO is always the
  // scaled fp16 copy ws_do written by the preprocess.
  const uint16_t* q16;
  const uint16_t* k16;
  const uint16_t* v16;
  const uint16_t* do16;
  uint16_t* ws_q;
  uint16_t* ws_k;
  uint16_t* ws_v;
  uint16_t* ws_do;
  int N;     // query rows per head
  int Nk;    // keys per head (= N for self-attention)
  int qoff;  // position of query row 0 in the key sequence (causal alignment), usually 0
  int bh;
  int n_tiles;
  float scale;
  float c;  // scale * log2(e)
  DropParams drop;  // used only by the dropout instances
  SparseParams sparse;  // used only by the block-sparse instances
};

// Partial maxima of |dO| per head (one per workgroup of the max pass).
constexpr int kMaxParts = 256;

// Split-KV decoding: Nq (<= 4) query rows per head against Nk keys; partials per (head, chunk).
struct DecArgs {
  const void* q;  // [B,H,Nq,d]
  const void* k;  // [B,H,Nk,d]
  const void* v;
  void* o;        // [B,H,Nq,d]
  float* lse;     // [B,H,Nq]
  float* part_o;  // [bh][n_split][nq_slots][d], nq_slots = 1 if Nq == 1 else 4
  float* part_ml; // [bh][n_split][nq_slots][2]: running max (log2 domain) and sum
  int Nq, Nk, bh, n_split, chunk;
  float c;        // scale * log2(e)
};

// Upper bound of the number of key chunks per head (the merge kernel keeps their weights in LDS).
constexpr int kDecodeMaxSplit = 2048;

// Bytes of the device-resident scratch array of the allocation-free decoding entry point
// (FA_DECODE_SCRATCH_BYTES in fa.h), and its address on the current device (looked up once per
// device with hipGetSymbolAddress; never the host-side name of the array).
constexpr size_t kDecodeScratchBytes = (size_t)8 << 20;
hipError_t decode_scratch(void** out);

// Chunking of Nk keys for bh heads (shared by the workspace size query and the launch).
void decode_plan(int bh, int nk, int d, int& n_split, int& chunk);
hipError_t launch_decode(const DecArgs& a, int d, int in_dtype, bool o_f32, bool causal,
                         hipStream_t s);

// in_dtype / o_dtype / grad_dtype codes follow fa_dtype: 0 = f32, 1 = f16, 2 = bf16.
// Variant of the kernels to run (16-bit inputs only for the last two).
enum class Mode { kPlain = 0, kDropout = 1, kSparse = 2 };

hipError_t launch_forward(const FwdArgs& a, int d, int in_dtype, int o_f32, bool causal,
                          Mode mode, hipStream_t s);
// ev_before / ev_after (may be null): recorded on `s` around the dK/dV kernel.
hipError_t launch_backward(const BwdArgs& a, int d, int in_dtype, int o_dtype, int grad_dtype,
                           bool causal, Mode mode, hipStream_t s, hipEvent_t ev_before,
                           hipEvent_t ev_after);

// Backward of fp32 attention (in_dtype, o_dtype and grad_dtype all fp32; N = Nk): D, then the
// keys-outer dK/dV and queries-outer dQ kernels on true-fp32 MFMA. Uses a.delta only.
hipError_t launch_backward_f32(const BwdArgs& a, int d, bool causal, hipStream_t s);

// Debug range check of 16-bit inputs bound for fp16 operands: sets *flag to 1 if any of the n
// 16-bit bf16 values at x has a magnitude fp16 cannot hold (|x| >= 65536 after rounding, or not
// finite). *flag must be zero beforehand (clear_flag).
hipError_t launch_clear_flag(uint32_t* flag, hipStream_t s);
hipError_t launch_range_check_bf16(const void* x, size_t n, uint32_t* flag, hipStream_t s);

}  // namespace fa
