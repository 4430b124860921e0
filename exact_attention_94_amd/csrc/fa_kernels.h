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
  float* delta;  // float32 [B,H,N]: rowsum(dO * O)
  // fp16 operands of the gradient kernels: the inputs themselves for fp16 inputs; for bf16
  // inputs, fp16 copies in the workspace (ws_q .. ws_do, null for fp16 inputs): Q and dO written
  // by the preprocess kernel, K and V by the dK/dV kernel (read by the dQ kernel after it).
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

}  // namespace fa
