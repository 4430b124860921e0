// Kernel argument blocks and launcher entry points shared by the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fa_device.h"

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int N;        // sequence length
  int bh;       // B * H
  int n_tiles;  // query tiles per head (set by the launcher)
  float c;      // scale * log2(e), never 0
  DropParams drop;  // used only by the dropout instances
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
  // inputs, the copies the preprocess kernel writes to ws16 (Q, K, V, dO, `elems` apart).
  const uint16_t* q16;
  const uint16_t* k16;
  const uint16_t* v16;
  const uint16_t* do16;
  uint16_t* ws16;
  size_t elems;  // B*H*N*d
  int N;
  int bh;
  int n_tiles;
  float scale;
  float c;  // scale * log2(e)
  DropParams drop;  // used only by the dropout instances
};

// in_dtype / o_dtype / grad_dtype codes follow fa_dtype: 0 = f32, 1 = f16, 2 = bf16.
// dropout: run the instances that apply the keep mask of a.drop (16-bit inputs only).
hipError_t launch_forward(const FwdArgs& a, int d, int in_dtype, int o_f32, bool causal,
                          bool dropout, hipStream_t s);
// ev_before / ev_after (may be null): recorded on `s` around the dK/dV kernel.
hipError_t launch_backward(const BwdArgs& a, int d, int in_dtype, int o_dtype, int grad_dtype,
                           bool causal, bool dropout, hipStream_t s, hipEvent_t ev_before,
                           hipEvent_t ev_after);

}  // namespace fa
