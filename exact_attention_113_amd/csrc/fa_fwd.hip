// Fused attention forward for bf16/fp16 inputs on gfx950.
//
// One workgroup owns BM = 256 query rows of one (batch, head) and streams
// the key/value rows through LDS in tiles of BN = 64 keys, keeping per
// query row a running maximum, a running sum of exponentials and an
// unnormalised fp32 output accumulator (online softmax: "From
// Self-Attention to FlashAttention", section 2; "FlashAttention in
// ops-transformer", "Core idea" and "Online softmax"). Scores and
// probabilities live only in registers; O and the row logsumexp are the
// only results written back ("only O is written to HBM", flowchart of
// section 1 of the first page).
//
// Waves. Four waves of 64 query rows each: wave w owns the 32-row blocks
// w and w + 4 of the workgroup's rows, so the four waves reach the causal
// diagonal within a tile of each other. Scores are computed transposed,
// S^T = K Q^T (32x32x16 MFMA, fp32 accumulate): lane j and j + 32 share one
// query and each holds 16 of a 32-key block's scores, so row maxima and
// sums are in-register reductions plus one exchange of the wave halves.
// The output is accumulated transposed as well, O^T = V^T P^T, whose B
// operand is the probability tile as the score MFMA left it in registers.
//
// Memory path. K and V tiles (32 keys) go from global memory straight into LDS with
// global_load_lds_dwordx4 (no staging registers), double-buffered: while a
// tile is consumed the next one is in flight. Each 16-byte chunk of a row
// is stored at an XOR-swizzled position so that the MFMA operand reads hit
// distinct LDS banks. V stays row-major in LDS; its transposed A operand is
// read with ds_read_b64_tr_b16, which hands lane i of each 16-lane group
// element i%4 of the chunks addressed by lanes 4j + i/4 (j = 0..3).
//
// Pipeline. K runs one tile ahead of V: iteration t computes the scores of
// tile t + 1 while it turns the scores of tile t into probabilities and
// accumulates P V for tile t, so the score MFMAs and the softmax VALU work
// are independent within an iteration. One barrier per tile.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 512;  // 8 waves: two per SIMD
constexpr int kWaves = kThreads / 64;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup: 32 per wave
constexpr int kBN = 64;           // keys per tile: two 32-key MFMA blocks
// Rescale the accumulator only when a row maximum grows by more than this
// many powers of two; until then probabilities are taken against the older,
// smaller reference, so each is at most 2^kTau. The final O = acc / sum and
// LSE = ref + log2(sum) do not depend on which reference was used.
constexpr float kTau = 8.0f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Work-item order: heavier causal query tiles first (longest job first
// over the CUs); when the heads divide evenly over the 8 XCDs each XCD
// keeps the same BH/8 heads, so their K and V stay in that XCD's L2.
__device__ __forceinline__ void tile_of(int lin, int n_qtiles, int bh_count, int& qt, int& bh) {
  if ((bh_count & 7) == 0) {
    const int hpx = bh_count >> 3;
    const int xcd = lin & 7, slot = lin >> 3;
    qt = n_qtiles - 1 - slot / hpx;
    bh = xcd * hpx + slot % hpx;
  } else {
    qt = n_qtiles - 1 - lin / bh_count;
    bh = lin % bh_count;
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <typename TT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE, int N,
    int n_qtiles, int bh_count, float c, uint32_t qsign) {
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int ROWB = 2 * D;                 // bytes per row
  constexpr int TILEB = kBN * ROWB;           // bytes per K or V tile
  constexpr int RPI = 64 / CH;                // rows per wave-wide direct load (1 KiB)
  constexpr int LPW = kBN / (kWaves * RPI);   // direct loads per wave, tile and tensor
  constexpr int DB = D / 32;                  // 32-row blocks of the head dim
  constexpr int KK = D / 16;                  // k-steps of the score MFMA
  static_assert(LPW >= 1, "tile too small for one direct load per wave");
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lq = lane & 31, hi = lane >> 5;

  int qt, bh;
  tile_of(blockIdx.x, n_qtiles, bh_count, qt, bh);
  const int q0 = qt * kBM;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  // This wave's 32 query rows and their B operands of S^T = K Q^T:
  // lane (query lq, half hi), k-step kk -> Q[row][16*kk + 8*hi + 0..7].
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
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float mref = -INFINITY;  // reference maximum, log2 units
  float lsum = 0.f;        // this lane's share of the row sum

  const int kv_end = CAUSAL ? min(N, q0 + kBM) : N;
  const int ntiles = (kv_end + kBN - 1) / kBN;
  // First tile where this wave needs masks or block skipping: the causal
  // diagonal of its rows, or the tile holding key N-1.
  int first_edge = (N - 1) / kBN;
  if (CAUSAL) first_edge = min(first_edge, (qw0 + 1) / kBN);

  char* const kbuf0 = smem;
  char* const vbuf0 = smem + 2 * TILEB;

  // Direct global->LDS load of rows [t*BN, t*BN + BN) of X. Lane l of load
  // i writes row R0 + l/CH at chunk position l%CH, fetching the chunk that
  // the swizzle puts there; rows past N repeat row N-1 (masked later).
  auto load_tile = [&](const uint16_t* Xh, int t, char* dst, bool is_v) {
    const int k0 = t * kBN;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int R0 = (w * LPW + i) * RPI;
      const int r = R0 + lane / CH, p = lane % CH;
      const int cg = is_v ? (p ^ (2 * (r & 3))) : (p ^ (r % CH));
      const int grow = min(k0 + r, N - 1);
      __builtin_amdgcn_global_load_lds(Xh + (size_t)grow * D + cg * 8,
                                       (lds_void*)(dst + R0 * ROWB), 16, 0, 0);
    }
  };

  // Per-lane parts of the LDS operand addresses.
  const int kxor = lq % CH;
  const int tj = (lane & 15) >> 2, tm = lane & 3, dsub = (lane >> 4) & 1;
  const int vlane = (4 * hi + tj) * ROWB + 8 * (tm & 1);
  const int vx = (2 * dsub + (tm >> 1)) ^ (2 * tj);

  // One tile: S^T = K Q^T, online-softmax update, O^T += V^T P^T.
  auto tile = [&](auto edge, int t) {
    constexpr bool EDGE = decltype(edge)::value;
    const char* kt = kbuf0 + (t & 1) * TILEB;
    const char* vt = vbuf0 + (t & 1) * TILEB;
    const int k0 = t * kBN;
    bool act[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kbase = k0 + 32 * kb;
      act[kb] = !EDGE || (kbase < N && (!CAUSAL || kbase <= qw0 + 31));
    }

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!act[kb]) continue;
        const u32x4 a =
            *(const u32x4*)(kt + (32 * kb + lq) * ROWB + 16 * ((2 * kk + hi) ^ kxor));
        s[kb] = TT::mma(a, qf[kk], s[kb]);
      }

    if (EDGE) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = act[kb] && key < N && (!CAUSAL || key <= qi);
          s[kb][r] = ok ? s[kb][r] : -INFINITY;
        }
    }
    float mx = s[0][0];
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
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }

    // Probabilities and the packed B operands of O^T += V^T P^T: slot e of
    // lane half hi in step (kb, h) is key 32*kb + 16*h + 4*hi + (e<4 ? e : e+4).
    const float nm = -mref;
    u32x4 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = fast_exp2(fmaf(s[kb][r], c, nm));
        if (EDGE) x = (s[kb][r] == -INFINITY) ? 0.f : x;
        p[r] = x;
        lsum += x;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) pf[kb][h][e] = TT::pack2(p[8 * h + 2 * e], p[8 * h + 2 * e + 1]);
    }

    // The A operand (32 dims x 16 keys) is two transposing LDS reads.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!act[kb]) continue;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const char* base = vt + (32 * kb + 16 * h) * ROWB + vlane + 16 * ((4 * db) ^ vx);
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)base);
          const s16x4 up =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * ROWB));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
          const u32x2 u2 = __builtin_bit_cast(u32x2, up);
          const u32x4 a = {l2[0], l2[1], u2[0], u2[1]};
          oacc[db] = TT::mma(a, pf[kb][h], oacc[db]);
        }
    }
  };

  // Pipeline: tile t+1 is in flight into the other buffers while tile t is
  // consumed; one barrier per tile makes the landed tile visible and frees
  // the consumed buffers.
  load_tile(Kh, 0, kbuf0, false);
  load_tile(Vh, 0, vbuf0, true);
  wait_vmem();
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) {
      load_tile(Kh, t + 1, kbuf0 + ((t + 1) & 1) * TILEB, false);
      load_tile(Vh, t + 1, vbuf0 + ((t + 1) & 1) * TILEB, true);
    }
    if (t < first_edge)
      tile(std::false_type{}, t);
    else
      tile(std::true_type{}, t);
    wait_vmem();
    __syncthreads();
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

template <typename TT, int D>
hipError_t launch_half(const FwdArgs& a) {
  const int n_qtiles = (int)((a.N + kBM - 1) / kBM);
  const int bh_count = (int)(a.B * a.H);
  const int64_t grid = (int64_t)n_qtiles * bh_count;
  const float c = fabsf(a.scale) * kLog2e;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  if (a.causal)
    hipLaunchKernelGGL((fwd_kernel<TT, D, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, (int)a.N, n_qtiles, bh_count,
                       c, qsign);
  else
    hipLaunchKernelGGL((fwd_kernel<TT, D, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, (int)a.N, n_qtiles, bh_count,
                       c, qsign);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a) {
  switch (a.dtype) {
    case FA_BF16: return a.D == 64 ? launch_half<Bf16, 64>(a) : launch_half<Bf16, 128>(a);
    case FA_FP16: return a.D == 64 ? launch_half<F16, 64>(a) : launch_half<F16, 128>(a);
    default: return launch_forward_f32(a);
  }
}

}  // namespace fa
