// Attention backward for gfx950, by recomputation from the forward's row
// logsumexp ("Flash Attention algorithm design and I/O optimisation",
// "Core mechanism": keep a few row statistics, recompute local blocks;
// "FlashAttention in ops-transformer", "A surprise": the backward needs the
// forward's state). The gradient formulas are the chain rule through the
// softmax of the forward definition:
//   P = exp(scale*QK^T - LSE), dV = P^T dO, dP = dO V^T,
//   delta_i = sum_d dO[i,d] O[i,d], dS = P*(dP - delta),
//   dQ = scale dS K, dK = scale dS^T Q.
//
// Three launches on the caller's stream:
//   1. bwd_pre_kernel   delta for every row; zero the fp32 dQ accumulator.
//   2. bwd_main_kernel  one workgroup per 128-key tile of one (batch, head):
//                       K and V stay in registers, dK and dV accumulate in
//                       registers over the query blocks that can see the
//                       tile, and each block's dQ contribution is added to
//                       the fp32 accumulator with atomics.
//   3. bwd_dq_kernel    dQ accumulator -> dtype.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- delta

template <typename TT, int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                           const uint16_t* __restrict__ dO,
                                                           float* __restrict__ delta,
                                                           float* __restrict__ dq_acc,
                                                           int64_t rows) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = gid / TPR;
  const int part = (int)(gid % TPR);
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = *(const u32x4*)(O + row * D + part * 8);
    const u32x4 g = *(const u32x4*)(dO + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(TT::lo(o[i]), TT::lo(g[i]), acc);
      acc = fmaf(TT::hi(o[i]), TT::hi(g[i]), acc);
    }
    float* z = dq_acc + row * D + part * 8;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    *(f32x4*)z = zero;
    *(f32x4*)(z + 4) = zero;
  }
  // Reduce over the TPR consecutive lanes of the row (TPR divides 64).
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) delta[row] = acc;
}

// ---------------------------------------------------------------- main

template <typename TT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ delta, float* __restrict__ dq_acc,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int n_ktiles, float c,
    float dk_scale, float dq_scale, uint32_t qsign) {
  constexpr int BK = 128;         // keys per workgroup: 32 per wave
  constexpr int BM = 64;          // query rows per iteration: two 32-row blocks
  constexpr int RSTR = D + 8;     // row-major Q / dO stride (elements)
  constexpr int TSTR = BM + 4;    // transposed Q^T / dO^T stride
  constexpr int KTSTR = BK + 8;   // K^T stride
  constexpr int SSTR = BK + 8;    // dS stride
  constexpr int DB = D / 32;
  constexpr int KK = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[BM * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[BM * RSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Qts[D * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dOts[D * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Kts[D * KTSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dSs[BM * SSTR];
  __shared__ float lse2s[BM];
  __shared__ float dels[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lq = lane & 31, hi = lane >> 5;
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int bh = logical / n_ktiles;
  const int kt = logical % n_ktiles;  // low key tiles see the most queries: first
  const int k0 = kt * BK;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const uint16_t* dOh = dO + head;
  const float* lseh = LSE + (size_t)bh * N;
  const float* delh = delta + (size_t)bh * N;
  float* dqh = dq_acc + head;

  // This wave's 32 keys as B operands (K for S = Q K^T, V for dP = dO V^T):
  // lane (key lq, half hi), k-step kk -> row[16*kk + 8*hi + 0..7].
  const int kw0 = k0 + 32 * w;
  const int kidx = kw0 + lq;
  u32x4 kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (kidx < N) {
      a = *(const u32x4*)(Kh + (size_t)kidx * D + 16 * kk + 8 * hi);
      b = *(const u32x4*)(Vh + (size_t)kidx * D + 16 * kk + 8 * hi);
    }
    kf[kk] = a;
    vf[kk] = b;
  }
  // K^T of the whole tile in LDS for dQ = dS K (4 keys x 8 dims per item).
  for (int it = tid; it < (BK / 4) * (D / 8); it += kThreads) {
    const int col = (it % (D / 8)) * 8, g = it / (D / 8);
    u32x4 r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + 4 * g + j;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < N) x = *(const u32x4*)(Kh + (size_t)key * D + col);
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
      *(u32x2*)(Kts + (col + e) * KTSTR + 4 * g) = out;
    }
  }

  f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk_acc[i][r] = 0.f;
      dv_acc[i][r] = 0.f;
    }

  const int nq = (N + BM - 1) / BM;
  const int qb_begin = CAUSAL ? (k0 / BM) : 0;
  for (int qbk = qb_begin; qbk < nq; ++qbk) {
    const int i0 = qbk * BM;
    __syncthreads();
    // Stage Q (sign-flipped for negative scale) and dO, both row-major and
    // transposed, plus the rows' LSE (log2 units) and delta.
    for (int it = tid; it < (BM / 4) * (D / 8); it += kThreads) {
      const int col = (it % (D / 8)) * 8, g = it / (D / 8);
      u32x4 rq[4], rg[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = i0 + 4 * g + j;
        u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
        if (row < N) {
          x = *(const u32x4*)(Qh + (size_t)row * D + col) ^ qsign;
          y = *(const u32x4*)(dOh + (size_t)row * D + col);
        }
        rq[j] = x;
        rg[j] = y;
        *(u32x4*)(Qs + (4 * g + j) * RSTR + col) = x;
        *(u32x4*)(dOs + (4 * g + j) * RSTR + col) = y;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        u32x2 oq, og;
        if ((e & 1) == 0) {
          oq[0] = (rq[0][wi] & 0xffffu) | (rq[1][wi] << 16);
          oq[1] = (rq[2][wi] & 0xffffu) | (rq[3][wi] << 16);
          og[0] = (rg[0][wi] & 0xffffu) | (rg[1][wi] << 16);
          og[1] = (rg[2][wi] & 0xffffu) | (rg[3][wi] << 16);
        } else {
          oq[0] = (rq[0][wi] >> 16) | (rq[1][wi] & 0xffff0000u);
          oq[1] = (rq[2][wi] >> 16) | (rq[3][wi] & 0xffff0000u);
          og[0] = (rg[0][wi] >> 16) | (rg[1][wi] & 0xffff0000u);
          og[1] = (rg[2][wi] >> 16) | (rg[3][wi] & 0xffff0000u);
        }
        *(u32x2*)(Qts + (col + e) * TSTR + 4 * g) = oq;
        *(u32x2*)(dOts + (col + e) * TSTR + 4 * g) = og;
      }
    }
    if (tid < BM) {
      const int row = i0 + tid;
      lse2s[tid] = row < N ? lseh[row] * kLog2e : 0.f;
      dels[tid] = row < N ? delh[row] : 0.f;
    }
    __syncthreads();

#pragma unroll
    for (int qb = 0; qb < BM / 32; ++qb) {
      const int qbase = i0 + 32 * qb;
      const bool active = kw0 < N && qbase < N && (!CAUSAL || qbase + 31 >= kw0);
      if (!active) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dSs[(32 * qb + 8 * (r >> 2) + 4 * hi + (r & 3)) * SSTR + 32 * w + lq] = 0;
        continue;
      }
      // S and dP for 32 queries x this wave's 32 keys: lane = key,
      // register r = query 8*(r/4) + 4*hi + r%4 of the block.
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 aq = *(const u32x4*)(Qs + (32 * qb + lq) * RSTR + 16 * kk + 8 * hi);
        const u32x4 ag = *(const u32x4*)(dOs + (32 * qb + lq) * RSTR + 16 * kk + 8 * hi);
        s = TT::mma(aq, kf[kk], s);
        dp = TT::mma(ag, vf[kk], dp);
      }
      float p[16], ds[16];
      const bool need_mask = (kw0 + 31 >= N) || (qbase + 31 >= N) || (CAUSAL && kw0 + 31 > qbase);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 32 * qb + 8 * (r >> 2) + 4 * hi + (r & 3);
        float x = fast_exp2(fmaf(s[r], c, -lse2s[ql]));
        if (need_mask) {
          const int qidx = i0 + ql;
          const bool ok = kidx < N && qidx < N && (!CAUSAL || kidx <= qidx);
          x = ok ? x : 0.f;
        }
        p[r] = x;
        ds[r] = x * (dp[r] - dels[ql]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over this block's 32 queries:
      // slot e of lane half hi in step h is query 16*h + 4*hi + (e<4 ? e : e+4).
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 pf, sf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pf[e] = TT::pack2(p[8 * h + 2 * e], p[8 * h + 2 * e + 1]);
          sf[e] = TT::pack2(ds[8 * h + 2 * e], ds[8 * h + 2 * e + 1]);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int toff = (32 * db + lq) * TSTR + 32 * qb + 16 * h + 4 * hi;
          const u32x2 g0 = *(const u32x2*)(dOts + toff);
          const u32x2 g1 = *(const u32x2*)(dOts + toff + 8);
          const u32x2 q0 = *(const u32x2*)(Qts + toff);
          const u32x2 q1 = *(const u32x2*)(Qts + toff + 8);
          const u32x4 ag = {g0[0], g0[1], g1[0], g1[1]};
          const u32x4 aq = {q0[0], q0[1], q1[0], q1[1]};
          dv_acc[db] = TT::mma(ag, pf, dv_acc[db]);
          dk_acc[db] = TT::mma(aq, sf, dk_acc[db]);
        }
      }
      // dS (rounded to the dtype) into LDS, row = query, column = key.
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const uint32_t pk = TT::pack2(ds[r], ds[r + 1]);
        const int ql = 32 * qb + 8 * (r >> 2) + 4 * hi + (r & 3);
        dSs[ql * SSTR + 32 * w + lq] = (uint16_t)(pk & 0xffffu);
        dSs[(ql + 1) * SSTR + 32 * w + lq] = (uint16_t)(pk >> 16);
      }
    }
    __syncthreads();

    // dQ[i0 .. i0+BM) += scale * dS K over the tile's 128 keys. Output
    // blocks (32 queries x 32 dims) are spread over the 4 waves.
    constexpr int NBLK = (BM / 32) * DB;
#pragma unroll
    for (int blk = w; blk < NBLK; blk += 4) {
      const int qb = blk / DB, db = blk % DB;
      if (i0 + 32 * qb >= N) continue;
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const u32x4 a = *(const u32x4*)(dSs + (32 * qb + lq) * SSTR + 16 * kk + 8 * hi);
        const u32x4 b = *(const u32x4*)(Kts + (32 * db + lq) * KTSTR + 16 * kk + 8 * hi);
        acc = TT::mma(a, b, acc);
      }
      // A = dS (rows = queries), B = K (columns = this block's dims): acc[r]
      // is dQ[query 8*(r/4)+4*hi+r%4][dim lq] of the block.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qidx = i0 + 32 * qb + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (qidx < N) atomicAdd(dqh + (size_t)qidx * D + 32 * db + lq, acc[r] * dq_scale);
      }
    }
  }

  // dK = scale * acc, dV = acc, rounded to the dtype. Lane lq holds key
  // kidx; register r holds dim 32*db + 8*(r/4) + 4*hi + r%4.
  if (kidx < N) {
    uint16_t* dkr = dK + head + (size_t)kidx * D;
    uint16_t* dvr = dV + head + (size_t)kidx * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 ok, ov;
        ok[0] = TT::pack2(dk_acc[db][4 * g4] * dk_scale, dk_acc[db][4 * g4 + 1] * dk_scale);
        ok[1] = TT::pack2(dk_acc[db][4 * g4 + 2] * dk_scale, dk_acc[db][4 * g4 + 3] * dk_scale);
        ov[0] = TT::pack2(dv_acc[db][4 * g4], dv_acc[db][4 * g4 + 1]);
        ov[1] = TT::pack2(dv_acc[db][4 * g4 + 2], dv_acc[db][4 * g4 + 3]);
        *(u32x2*)(dkr + 32 * db + 8 * g4 + 4 * hi) = ok;
        *(u32x2*)(dvr + 32 * db + 8 * g4 + 4 * hi) = ov;
      }
  }
}

// ---------------------------------------------------------------- dQ cast

template <typename TT>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(const float* __restrict__ acc,
                                                          uint16_t* __restrict__ dq,
                                                          int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *(const f32x4*)(acc + 8 * i);
  const f32x4 b = *(const f32x4*)(acc + 8 * i + 4);
  u32x4 out;
  out[0] = TT::pack2(a[0], a[1]);
  out[1] = TT::pack2(a[2], a[3]);
  out[2] = TT::pack2(b[0], b[1]);
  out[3] = TT::pack2(b[2], b[3]);
  *(u32x4*)(dq + 8 * i) = out;
}

template <typename TT, int D>
hipError_t launch_typed(const BwdArgs& a, const BwdWorkspace& ws) {
  char* wsb = (char*)a.workspace;
  float* dq_acc = (float*)(wsb + ws.dq_acc_off);
  float* delta = (float*)(wsb + ws.delta_off);
  const int64_t rows = a.B * a.H * a.N;

  const int64_t pre_threads = rows * (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<TT, D>),
                     dim3((unsigned)((pre_threads + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     a.stream, (const uint16_t*)a.o, (const uint16_t*)a.dout, delta, dq_acc, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int n_ktiles = (int)((a.N + 127) / 128);
  const int64_t grid = (int64_t)n_ktiles * a.B * a.H;
  const float c = fabsf(a.scale) * kLog2e;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  // Q is staged sign-flipped when scale < 0, so dK = |scale| dS^T (-Q) ...
  // = scale dS^T Q; dQ = scale dS K does not involve Q.
  const float dk_scale = fabsf(a.scale);
  const float dq_scale = a.scale;
  if (a.causal)
    hipLaunchKernelGGL((bwd_main_kernel<TT, D, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, delta, dq_acc, (uint16_t*)a.dk,
                       (uint16_t*)a.dv, (int)a.N, n_ktiles, c, dk_scale, dq_scale, qsign);
  else
    hipLaunchKernelGGL((bwd_main_kernel<TT, D, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, delta, dq_acc, (uint16_t*)a.dk,
                       (uint16_t*)a.dv, (int)a.N, n_ktiles, c, dk_scale, dq_scale, qsign);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int64_t n8 = rows * D / 8;
  hipLaunchKernelGGL((bwd_dq_kernel<TT>), dim3((unsigned)((n8 + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, a.stream, dq_acc, (uint16_t*)a.dq, n8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, const BwdWorkspace& ws) {
  if (a.dtype == FA_BF16)
    return a.D == 64 ? launch_typed<Bf16, 64>(a, ws) : launch_typed<Bf16, 128>(a, ws);
  return a.D == 64 ? launch_typed<F16, 64>(a, ws) : launch_typed<F16, 128>(a, ws);
}

}  // namespace fa
