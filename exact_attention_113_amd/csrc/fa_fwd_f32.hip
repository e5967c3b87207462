// Fused attention forward for fp32 inputs on gfx950.
//
// Same online-softmax algorithm as the half-precision kernel ("From
// Self-Attention to FlashAttention", section 2), computed with
// v_mfma_f32_32x32x2_f32 so that nothing, probabilities included, is
// rounded below fp32. Scores are computed transposed (S^T = K Q^T) so each
// lane pair holds one query, and O^T = V^T P^T takes the probabilities
// straight from registers.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr float kTau = 8.0f;

// fp32 inputs: v_mfma_f32_32x32x2_f32 throughout, so nothing is rounded
// below fp32 (probabilities included). Same transposed formulation as the
// half-precision kernel. The waves form NRG row groups of 32 query rows,
// and KS waves of a row group split the keys: a K/V tile holds KS blocks of
// 32 keys, and wave kh of the group computes block kh of every tile with
// its own online-softmax state. At the end the KS states of a row group are
// merged (the rescale-and-add of the online softmax over disjoint key
// sets). Every workgroup has four waves: KS = 1 is the plain kernel (four
// row groups over whole key ranges); small grids use KS waves per row group
// (4 / KS row groups) and a KS times shorter key loop per wave.
template <int D, bool CAUSAL, int KS>
__global__ __launch_bounds__(64 * f32_row_groups(KS) * KS, 1) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int n_qtiles, float c, float qsgn,
    int heads, int group) {
  constexpr int NRG = f32_row_groups(KS);  // row groups
  constexpr int kThreads = 64 * NRG * KS;
  constexpr int BM = 32 * NRG;              // query rows per workgroup
  constexpr int BN = 32 * KS;               // keys per tile
  constexpr int KSTR = D + 1;  // odd stride: the 32 rows read by a k-step hit 32 banks
  constexpr int VSTR = D;
  constexpr int DB = D / 32;
  constexpr int KK = D / 2;
  // Two K and two V tiles: tile t + 1 is fetched into registers while tile
  // t is used, then written to the other buffer (one barrier per tile).
  __shared__ float Ks[2][BN * KSTR];
  __shared__ float Vs[2][BN * VSTR];
  constexpr int NX = KS > 1 ? NRG * (KS - 1) : 1;  // merge slots of the key splits
  __shared__ float xm[NX][64], xl[NX][64];
  constexpr int PER = BN * D / 4 / kThreads;  // 16-byte pieces per thread and tensor
  static_assert(PER * kThreads * 4 == BN * D, "tile not divisible among the threads");
  static_assert(NX * 32 * D <= 2 * BN * KSTR, "merge slots exceed the K buffers");

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lq = lane & 31, hi = lane >> 5;
  const int rg = w % NRG, kh = w / NRG;  // row group, key split
  int qt, bh;
  f32_tile_of(blockIdx.x, gridDim.x, n_qtiles, qt, bh);
  const int q0 = qt * BM;
  // (batch, query head) pair bh; query head h reads K/V head h / group.
  const size_t head = (size_t)bh * (size_t)N * D;
  const int b = bh / heads, h = bh - b * heads;
  const size_t kv_head = ((size_t)b * (heads / group) + h / group) * (size_t)N * D;
  const float* Qh = Q + head;
  const float* Kh = K + kv_head;
  const float* Vh = V + kv_head;

  const int qw0 = q0 + 32 * rg;
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

  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int ntiles = (kv_end + BN - 1) / BN;
  f32x4 kx[PER], vx[PER];
  auto fetch = [&](int t) __attribute__((always_inline)) {
    const int k0 = t * BN;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c4 = tid + i * kThreads;
      const int row = c4 / (D / 4), col = (c4 % (D / 4)) * 4;
      // Rows past N read row N - 1 and are zeroed when stored.
      const int grow = min(k0 + row, N - 1);
      kx[i] = *(const f32x4*)(Kh + (size_t)grow * D + col);
      vx[i] = *(const f32x4*)(Vh + (size_t)grow * D + col);
    }
  };
  auto stash = [&](int t, int buf) __attribute__((always_inline)) {
    const int k0 = t * BN;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c4 = tid + i * kThreads;
      const int row = c4 / (D / 4), col = (c4 % (D / 4)) * 4;
      const bool ok = k0 + row < N;
#pragma unroll
      for (int e = 0; e < 4; ++e) Ks[buf][row * KSTR + col + e] = ok ? kx[i][e] : 0.f;
      *(f32x4*)(&Vs[buf][row * VSTR + col]) = ok ? vx[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  if (ntiles > 0) {
    fetch(0);
    stash(0, 0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BN + 32 * kh;  // this wave's 32 keys of the tile
    const int buf = t & 1;
    if (t + 1 < ntiles) fetch(t + 1);
    const float* Kt = Ks[buf] + 32 * kh * KSTR;
    const float* Vt = Vs[buf] + 32 * kh * VSTR;
    const bool active = k0 < N && (!CAUSAL || k0 <= qw0 + 31);  // wave-uniform
    if (active) {
    const bool need_mask = (k0 + 32 > N) || (CAUSAL && k0 + 31 > qw0);

    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(Kt[lq * KSTR + 2 * kk + hi], qf[kk], s, 0, 0, 0);

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
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vt[key * VSTR + 32 * db + lq], p[r],
                                                        oacc[db], 0, 0, 0);
      }
    }
    // Tile t + 1 into the other buffer (its last readers passed the barrier
    // that ended iteration t - 1), then one barrier for both buffers.
    if (t + 1 < ntiles) stash(t + 1, buf ^ 1);
    __syncthreads();
  }

  if constexpr (KS > 1) {
    // Merge of the key splits (every wave is past the loop's last barrier,
    // so the K buffers are free): waves kh > 0 leave their reference, sum
    // share and accumulator in a slot of their own; wave kh = 0 of the row
    // group rescales all of them to the largest reference and adds.
    float* xo = &Ks[0][0];
    constexpr int SLOT = DB * 16 * 64;  // floats of one wave's accumulator
    if (kh > 0) {
      const int slot = rg * (KS - 1) + kh - 1;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[slot * SLOT + (db * 16 + r) * 64 + lane] = oacc[db][r];
      xm[slot][lane] = mref;
      xl[slot][lane] = lsum;
    }
    __syncthreads();
    if (kh > 0) return;
    float mm = mref;
#pragma unroll
    for (int x = 0; x < KS - 1; ++x) mm = fmaxf(mm, xm[rg * (KS - 1) + x][lane]);
    const float a0 = mref == -INFINITY ? 0.f : fast_exp2(mref - mm);
    lsum *= a0;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= a0;
#pragma unroll
    for (int x = 0; x < KS - 1; ++x) {
      const int slot = rg * (KS - 1) + x;
      const float mx = xm[slot][lane];
      const float ax = mx == -INFINITY ? 0.f : fast_exp2(mx - mm);
      lsum = fmaf(xl[slot][lane], ax, lsum);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          oacc[db][r] = fmaf(xo[slot * SLOT + (db * 16 + r) * 64 + lane], ax, oacc[db][r]);
    }
    mref = mm;
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


template <int D, bool CAUSAL, int KS>
hipError_t launch_f32(const FwdArgs& a, const F32Shape& sh) {
  const float c = fabsf(a.scale) * kLog2e;
  const float qsgn = a.scale < 0.f ? -1.f : 1.f;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, KS>), dim3((unsigned)sh.grid),
                     dim3(64 * f32_row_groups(KS) * KS), 0, a.stream, (const float*)a.q,
                     (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, (int)a.N,
                     sh.n_qtiles, c, qsgn, (int)a.H, (int)(a.H / (a.H_kv > 0 ? a.H_kv : a.H)));
  return hipGetLastError();
}

template <int D, int KS_SPLIT>
hipError_t launch_f32_d(const FwdArgs& a, bool causal) {
  const F32Shape sh = f32_shape(a.B * a.H, a.N, D);
  if (sh.ks == 1)
    return causal ? launch_f32<D, true, 1>(a, sh) : launch_f32<D, false, 1>(a, sh);
  return causal ? launch_f32<D, true, KS_SPLIT>(a, sh) : launch_f32<D, false, KS_SPLIT>(a, sh);
}

}  // namespace

hipError_t launch_forward_f32(const FwdArgs& a) {
  const bool causal = a.causal != 0;
  return a.D == 64 ? launch_f32_d<64, f32_split(64)>(a, causal)
                   : launch_f32_d<128, f32_split(128)>(a, causal);
}

}  // namespace fa
