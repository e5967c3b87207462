// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"
#include "fa_sched.h"

namespace fa {

// Attention dropout constants of one call: element (i, j) of head bh is
// dropped when byte j % 4 of word i % 4 of Philox4x32-10 with counter
// (j / 4, i / 4, bh, offset) and key (k0, k1) is below thr.
struct DropParams {
  uint32_t thr;       // floor(256 p + 0.5); 0 = no dropout
  uint32_t k0, k1;    // seed, low and high 32 bits
  uint32_t offset;
  float inv_keep;     // 1 / (1 - thr / 256)
  uint32_t thr4;      // thr in each of the four bytes
  uint32_t bias4;     // 0x80808080 - (thr4 & 0x7f7f7f7f): see keep_flags4
};

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
  DropParams drop;   // thr = 0: none
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
  DropParams drop;   // thr = 0: none
  // Packed variable-length batch, as in FwdArgs: B sequences given by
  // cu_seqlens, N = the longest, total = tokens; H_kv divides H (0: H).
  int64_t H_kv;
  const int32_t* cu_seqlens;
  int64_t total;
};

// Byte offsets of the backward workspace's parts (each 256-byte aligned).
struct BwdWorkspace {
  size_t delta_off, delta_bytes;    // fp32 [B, H, N]: sum_d dO * O
  size_t lse2_off, lse2_bytes;      // fp32 [B, H, N]: LSE * log2(e)
  size_t total;
};
bool backward_workspace_layout(int64_t B, int64_t H, int64_t N, int64_t D, BwdWorkspace* ws);

// Decode: s_q new tokens per sequence against a K/V cache of capacity cap.
struct DecodeArgs {
  const void* q;             // [B, s_q, H, D]
  const void* k_cache;       // [B, cap, H_kv, D]
  const void* v_cache;       // [B, cap, H_kv, D]
  const int32_t* cache_seqlens;  // [B], device
  void* o;                   // [B, s_q, H, D]
  float* lse;                // [B, H, s_q]
  void* workspace;
  int64_t B, s_q, cap, max_len, H, H_kv, D;
  float scale;
  int dtype;
  hipStream_t stream;
};

// The chunk plan of a decode call (DecodePlan, decode_plan) is in fa_sched.h.

hipError_t launch_forward(const FwdArgs& a);
hipError_t launch_forward_f32(const FwdArgs& a);
hipError_t launch_backward(const BwdArgs& a, const BwdWorkspace& ws);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan);
hipError_t launch_clock_probe(uint64_t* out, int iters, hipStream_t stream);

}  // namespace fa
