// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t B, H, N, D;
  float scale;
  int causal;
  int dtype;
  hipStream_t stream;
  // Dense: B batches of N tokens each and H_kv = H. Packed variable-length
  // batch: B sequences given by cu_seqlens (device memory), N = the longest
  // sequence, total = tokens in the batch; H_kv divides H.
  int64_t H_kv;
  const int32_t* cu_seqlens;
  int64_t total;
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
  void* workspace;
  int64_t B, H, N, D;
  float scale;
  int causal;
  int dtype;
  hipStream_t stream;
};

// Byte offsets of the backward workspace's parts (each 256-byte aligned).
struct BwdWorkspace {
  size_t delta_off, delta_bytes;    // fp32 [B, H, N]: sum_d dO * O
  size_t lse2_off, lse2_bytes;      // fp32 [B, H, N]: LSE * log2(e)
  size_t total;
};
bool backward_workspace_layout(int64_t B, int64_t H, int64_t N, int64_t D, BwdWorkspace* ws);

hipError_t launch_forward(const FwdArgs& a);
hipError_t launch_forward_f32(const FwdArgs& a);
hipError_t launch_backward(const BwdArgs& a, const BwdWorkspace& ws);

}  // namespace fa
