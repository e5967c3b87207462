// Fused attention forward for gfx950.
//
// One workgroup owns BM = 128 query rows of one (batch, head) and streams
// the key/value rows through LDS in tiles of BN keys, keeping per query row
// a running maximum, a running sum of exponentials and an unnormalised
// output accumulator (online softmax: "From Self-Attention to
// FlashAttention", section 2; "FlashAttention in ops-transformer", "Core
// idea" and "Online softmax"). Scores and probabilities live only in
// registers; O and the row logsumexp are the only results written back.
//
// Wave layout (4 waves, 32 query rows each). Scores are computed transposed,
// S^T = K Q^T, so that the MFMA result puts one query in each lane pair
// (lane j and j+32) and 16 keys per 32-key block in each lane's registers:
// row maxima and sums are in-register reductions plus one exchange between
// the two wave halves. The output is accumulated transposed as well,
// O^T = V^T P^T, whose B operand is the probability tile exactly as the
// score MFMA left it in registers; V is staged transposed in LDS so that its
// A operand is two 8-byte LDS reads per lane.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;  // query rows per workgroup
// Rescale the accumulator only when a row maximum grows by more than this
// many powers of two; until then probabilities are taken against the older,
// smaller reference, so each is at most 2^kTau. The final O = acc / sum and
// LSE = ref + log2(sum) do not depend on which reference was used.
constexpr float kTau = 8.0f;

// ---------------------------------------------------------------- bf16/fp16

template <typename TT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_half_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, float c, uint32_t qsign) {
  constexpr int BN = 64;             // keys per tile: two 32-key MFMA blocks
  constexpr int KSTR = D + 8;        // K row stride in LDS (elements)
  constexpr int VSTR = BN + 4;       // V^T row stride in LDS (elements)
  constexpr int DB = D / 32;         // 32-row blocks of the head dim
  constexpr int KK = D / 16;         // k-steps of the score MFMA
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vts[D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lq = lane & 31, hi = lane >> 5;

  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int bh = logical / n_qtiles;
  const int qt = n_qtiles - 1 - (logical % n_qtiles);  // heavier causal tiles first
  const int q0 = qt * kBM;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  // This lane's query row and its operand fragment: the B operand of
  // S^T = K Q^T for k-step kk is Q[row][16*kk + 8*hi + 0..7].
  const int qw0 = q0 + 32 * w;
  const int qi = qw0 + lq;
  u32x4 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < N) x = *(const u32x4*)(Qh + (size_t)qi * D + 16 * kk + 8 * hi);
    qf[kk] = x ^ qsign;  // sign flip for negative scale (exact)
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mref = -INFINITY;  // reference maximum, log2 units (score * c)
  float lsum = 0.f;        // this lane's share of the row sum

  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BN;
    __syncthreads();
    // Stage K rows [k0, k0+BN) row-major; rows past N read as zero.
#pragma unroll
    for (int c8 = tid; c8 < BN * D / 8; c8 += kThreads) {
      const int row = c8 / (D / 8), col = (c8 % (D / 8)) * 8;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (k0 + row < N) x = *(const u32x4*)(Kh + (size_t)(k0 + row) * D + col);
      *(u32x4*)(Ks + row * KSTR + col) = x;
    }
    // Stage V transposed: each thread takes 4 keys x 8 head-dim values and
    // writes 8 rows of V^T with 4 keys each.
#pragma unroll
    for (int c8 = tid; c8 < (BN / 4) * (D / 8); c8 += kThreads) {
      const int col = (c8 % (D / 8)) * 8, g = c8 / (D / 8);
      u32x4 r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + 4 * g + j;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < N) x = *(const u32x4*)(Vh + (size_t)key * D + col);
        r[j] = x;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        u32x2 out;
        if ((e & 1) == 0) {
          out[0] = (r[0][wi] & 0xffffu) | (r[1][wi] << 16);
          out[1] = (r[2][wi] & 0xffffu) | (r[3][wi] << 16);
        } else {
          out[0] = (r[0][wi] >> 16) | (r[1][wi] & 0xffff0000u);
          out[1] = (r[2][wi] >> 16) | (r[3][wi] & 0xffff0000u);
        }
        *(u32x2*)(Vts + (col + e) * VSTR + 4 * g) = out;
      }
    }
    __syncthreads();

    // Which 32-key blocks hold any key this wave may see.
    bool active[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kbase = k0 + 32 * kb;
      active[kb] = kbase < N && (!CAUSAL || kbase <= qw0 + 31);
    }
    const bool need_mask = (k0 + BN > N) || (CAUSAL && k0 + BN - 1 > qw0);

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      if (active[kb]) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4 a = *(const u32x4*)(Ks + (32 * kb + lq) * KSTR + 16 * kk + 8 * hi);
          s[kb] = TT::mma(a, qf[kk], s[kb]);
        }
      }
    }

    // Mask keys past N, keys after this lane's query (causal) and whole
    // inactive blocks; then the row maximum over the tile.
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = active[kb] && key < N && (!CAUSAL || key <= qi);
          s[kb][r] = ok ? s[kb][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = half_swap_max(mx);
    const float tmx = (mx == -INFINITY) ? -INFINITY : mx * c;

    if (wave_any(tmx > mref + kTau)) {
      const float mnew = fmaxf(mref, tmx);
      const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(mref - mnew);
      mref = mnew;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }

    // Probabilities against the reference, their sum, and the packed
    // B operands of O^T += V^T P^T (slot e of lane half hi in step (kb, h)
    // is key 32*kb + 16*h + 4*hi + (e < 4 ? e : e + 4)).
    u32x4 pf[2][2];
    const float nm = -mref;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = fast_exp2(fmaf(s[kb][r], c, nm));
        if (need_mask) x = (s[kb][r] == -INFINITY) ? 0.f : x;
        p[r] = x;
        lsum += x;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) pf[kb][h][e] = TT::pack2(p[8 * h + 2 * e], p[8 * h + 2 * e + 1]);
    }

#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint16_t* vrow = Vts + (32 * db + lq) * VSTR + 4 * hi;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!active[kb]) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x2 lo = *(const u32x2*)(vrow + 32 * kb + 16 * h);
          const u32x2 up = *(const u32x2*)(vrow + 32 * kb + 16 * h + 8);
          const u32x4 a = {lo[0], lo[1], up[0], up[1]};
          oacc[db] = TT::mma(a, pf[kb][h], oacc[db]);
        }
      }
    }
  }

  // Epilogue: O = acc / sum rounded to the dtype; LSE = ln 2 * (ref + log2 sum).
  const float ltot = half_swap_sum(lsum);
  const float inv = 1.f / ltot;
  if (qi < N) {
    uint16_t* orow = O + head + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 out;
        out[0] = TT::pack2(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv);
        out[1] = TT::pack2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
        *(u32x2*)(orow + 32 * db + 8 * g4 + 4 * hi) = out;
      }
    if (hi == 0) LSE[(size_t)bh * N + qi] = kLn2 * (mref + __log2f(ltot));
  }
}

// ---------------------------------------------------------------- fp32

// fp32 inputs: v_mfma_f32_32x32x2_f32 throughout, so nothing is rounded
// below fp32 (probabilities included). Same transposed formulation as the
// half-precision kernel with 32-key tiles.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, float c, float qsgn) {
  constexpr int BN = 32;
  constexpr int KSTR = D + 1;  // odd stride: the 32 rows read by a k-step hit 32 banks
  constexpr int VSTR = D;
  constexpr int DB = D / 32;
  constexpr int KK = D / 2;
  __shared__ float Ks[BN * KSTR];
  __shared__ float Vs[BN * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lq = lane & 31, hi = lane >> 5;
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int bh = logical / n_qtiles;
  const int qt = n_qtiles - 1 - (logical % n_qtiles);
  const int q0 = qt * kBM;
  const size_t head = (size_t)bh * (size_t)N * D;
  const float* Qh = Q + head;
  const float* Kh = K + head;
  const float* Vh = V + head;

  const int qw0 = q0 + 32 * w;
  const int qi = qw0 + lq;
  float qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = (qi < N) ? qsgn * Qh[(size_t)qi * D + 2 * kk + hi] : 0.f;

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mref = -INFINITY, lsum = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BN;
    __syncthreads();
    for (int c4 = tid; c4 < BN * D / 4; c4 += kThreads) {
      const int row = c4 / (D / 4), col = (c4 % (D / 4)) * 4;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (k0 + row < N) {
        kx = *(const f32x4*)(Kh + (size_t)(k0 + row) * D + col);
        vx = *(const f32x4*)(Vh + (size_t)(k0 + row) * D + col);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) Ks[row * KSTR + col + e] = kx[e];
      *(f32x4*)(Vs + row * VSTR + col) = vx;
    }
    __syncthreads();

    const bool active = k0 < N && (!CAUSAL || k0 <= qw0 + 31);
    if (!active) continue;  // wave-uniform; barriers above are shared by all waves
    const bool need_mask = (k0 + BN > N) || (CAUSAL && k0 + BN - 1 > qw0);

    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[lq * KSTR + 2 * kk + hi], qf[kk], s, 0, 0, 0);

    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const bool ok = key < N && (!CAUSAL || key <= qi);
        s[r] = ok ? s[r] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = half_swap_max(mx);
    const float tmx = (mx == -INFINITY) ? -INFINITY : mx * c;
    if (wave_any(tmx > mref + kTau)) {
      const float mnew = fmaxf(mref, tmx);
      const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(mref - mnew);
      mref = mnew;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = fast_exp2(fmaf(s[r], c, -mref));
      if (need_mask) x = (s[r] == -INFINITY) ? 0.f : x;
      p[r] = x;
      lsum += x;
    }
    // O^T += V^T P^T, one key pair per MFMA: lane half hi carries key
    // 8*(r/4) + 4*hi + (r%4) of register r in both operands.
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * hi + (r & 3);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * VSTR + 32 * db + lq], p[r],
                                                        oacc[db], 0, 0, 0);
      }
  }

  const float ltot = half_swap_sum(lsum);
  const float inv = 1.f / ltot;
  if (qi < N) {
    float* orow = O + head + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = oacc[db][4 * g4 + e] * inv;
        *(f32x4*)(orow + 32 * db + 8 * g4 + 4 * hi) = out;
      }
    if (hi == 0) LSE[(size_t)bh * N + qi] = kLn2 * (mref + __log2f(ltot));
  }
}

template <typename TT, int D>
hipError_t launch_half(const FwdArgs& a, bool causal) {
  const int n_qtiles = (int)((a.N + kBM - 1) / kBM);
  const int64_t grid = (int64_t)n_qtiles * a.B * a.H;
  const float c = fabsf(a.scale) * kLog2e;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  if (causal)
    hipLaunchKernelGGL((fwd_half_kernel<TT, D, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, (int)a.N, n_qtiles, c, qsign);
  else
    hipLaunchKernelGGL((fwd_half_kernel<TT, D, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, (int)a.N, n_qtiles, c, qsign);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const FwdArgs& a, bool causal) {
  const int n_qtiles = (int)((a.N + kBM - 1) / kBM);
  const int64_t grid = (int64_t)n_qtiles * a.B * a.H;
  const float c = fabsf(a.scale) * kLog2e;
  const float qsgn = a.scale < 0.f ? -1.f : 1.f;
  if (causal)
    hipLaunchKernelGGL((fwd_f32_kernel<D, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                       a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (float*)a.o, a.lse, (int)a.N, n_qtiles, c, qsgn);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                       a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (float*)a.o, a.lse, (int)a.N, n_qtiles, c, qsgn);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a) {
  const bool causal = a.causal != 0;
  switch (a.dtype) {
    case FA_BF16:
      return a.D == 64 ? launch_half<Bf16, 64>(a, causal) : launch_half<Bf16, 128>(a, causal);
    case FA_FP16:
      return a.D == 64 ? launch_half<F16, 64>(a, causal) : launch_half<F16, 128>(a, causal);
    default:
      return a.D == 64 ? launch_f32<64>(a, causal) : launch_f32<128>(a, causal);
  }
}

}  // namespace fa
