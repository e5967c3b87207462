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
// Three launches on the caller's stream, none with atomics, so the result
// is bitwise reproducible (the "deterministic" option of "FlashAttention in
// ops-transformer", "Complete operator", holds always):
//   1. bwd_pre_kernel   delta and LSE*log2(e) for every row.
//   2. bwd_dkdv_kernel  one workgroup per 128-key tile of one (sequence,
//                       K/V head), iterating over the 64-row query tiles
//                       that can see it, of every query head that shares
//                       the K/V head (so dK and dV sum over the group).
//                       Waves are paired on a SIMD: the first of a pair
//                       computes S = Q K^T and P for its 32 keys and
//                       accumulates dV^T += dO^T P; the second computes
//                       dP = dO V^T, takes P from the first through LDS,
//                       forms dS and accumulates dK^T += Q^T dS. Each wave
//                       keeps one 32 x D accumulator and one operand tile in
//                       registers.
//   3. bwd_dq_kernel    one workgroup per 256-row query tile of one
//                       (sequence, query head), streaming the
//                       K and V tiles like the forward: S^T = K Q^T and
//                       dP^T = V dO^T, dS, then dQ^T += K^T dS^T.
//
// Operand layouts (32x32x16 MFMA, see fa_device.h): a tile read row-wise
// gives lane i + 32g the 8 values [row i][16k + 8g ..] of k-step k; a tile
// read with ds_read_b64_tr_b16 gives lane j + 32g the values of column j at
// rows {16h + 4g + 0..3, 16h + 8 + 4g + 0..3} of step h, which is the row
// order in which a C-layout register block packs into an MFMA operand.
// Tiles that are read both ways store their 16-byte chunks at the position
// logical ^ swz(row), which keeps both kinds of read free of LDS bank
// conflicts.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 512;  // 8 waves, two per SIMD
constexpr int kWaves = kThreads / 64;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Chunk swizzle of a tile with CH 16-byte chunks per row. Row-wise reads
// touch 16 consecutive rows at one logical chunk (a bijection over them);
// transposed reads of a half-wave touch four consecutive rows and four
// consecutive chunks (distinct chunk groups, or bank halves, per row).
template <int CH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CH == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Direct global->LDS load of 64 rows [row0, row0 + 64) of an N-row matrix
// with `stride` elements between rows into dst (rows past N repeat row N-1),
// each row swizzled by swz. All waves of the workgroup take part.
template <int D>
__device__ __forceinline__ void load_rows64(const uint16_t* Xh, size_t stride, int row0, int N,
                                            char* dst, int w, int lane) {
  constexpr int CH = D / 8, ROWB = 2 * D, RPI = 64 / CH, LPW = 64 / (kWaves * RPI);
  static_assert(LPW >= 1, "tile too small");
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int R0 = (w * LPW + i) * RPI;
    const int r = R0 + lane / CH, p = lane % CH;
    const int grow = min(row0 + r, N - 1);
    const int cg = p ^ swz<CH>(r);  // logical chunk stored at position p
    __builtin_amdgcn_global_load_lds((const void*)(Xh + (size_t)grow * stride + cg * 8),
                                     (lds_void*)(dst + R0 * ROWB), 16, 0, 0);
  }
}

// Per-lane byte offsets of the operand reads inside a tile, for row bases
// that are multiples of 16 (the swizzle repeats every 16 rows). They are
// computed once per kernel and made opaque to the compiler, so that every
// read is this register plus its tile's and rows' base as the instruction's
// constant offset (without that, the compiler re-added tile bases per block
// and spilled the partial sums).
//   row[kk]   row-wise operand: lane (i + 32 hi), k-step kk -> row i,
//             dims 16 kk + 8 hi ..
//   tlo/tup   transposed operand: lane (j + 32 hi) -> column 32 db + j at
//             rows {4hi + 0..3} (tlo) and {8 + 4hi + 0..3} (tup)
template <int D>
struct LdsOffsets {
  static constexpr int CH = D / 8, ROWB = 2 * D;
  int row[D / 16];
  int tlo[D / 32], tup[D / 32];
  __device__ __forceinline__ void init(int lane) {
    const int lq = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      row[kk] = lq * ROWB + 16 * ((2 * kk + hi) ^ swz<CH>(lq));
      asm volatile("" : "+v"(row[kk]));
    }
    const int tj = (lane & 15) >> 2, tm = lane & 3, dsub = (lane >> 4) & 1;
    const int rlo = 4 * hi + tj, rup = rlo + 8;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int c = 4 * db + 2 * dsub + (tm >> 1);
      tlo[db] = rlo * ROWB + 16 * (c ^ swz<CH>(rlo)) + 8 * (tm & 1);
      tup[db] = rup * ROWB + 16 * (c ^ swz<CH>(rup)) + 8 * (tm & 1);
      asm volatile("" : "+v"(tlo[db]), "+v"(tup[db]));
    }
  }
};

// Row-wise operand of k-step kk from rows r0 .. r0 + 31 of a tile.
template <int D>
__device__ __forceinline__ u32x4 rd_row(const char* tile, int r0, const LdsOffsets<D>& lo, int kk) {
  return *(const u32x4*)(tile + r0 * (2 * D) + lo.row[kk]);
}

// Transposed operand of column block db from rows r0 .. r0 + 15 of a tile.
template <int D>
__device__ __forceinline__ u32x4 rd_tr(const char* tile, int r0, const LdsOffsets<D>& lo, int db) {
  const char* base = tile + r0 * (2 * D);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + lo.tlo[db]));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + lo.tup[db]));
  const u32x2 a2 = __builtin_bit_cast(u32x2, a);
  const u32x2 b2 = __builtin_bit_cast(u32x2, b);
  return u32x4{a2[0], a2[1], b2[0], b2[1]};
}

// ---------------------------------------------------------------- delta, LSE

template <typename TT, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                      const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ LSE,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ lse2, int64_t rows,
                                                      int64_t total, int heads) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / TPR;
  const int part = (int)(gid % TPR);
  float acc = 0.f;
  if (row < rows) {
    // Row of the statistics: (b, h, i) of [B, H, N], or (h, t) of a packed
    // batch's [H, total], whose O and dO rows are [total, H, D].
    const int64_t off = total > 0 ? ((row % total) * heads + row / total) * D : row * D;
    const u32x4 o = *(const u32x4*)(O + off + part * 8);
    const u32x4 g = *(const u32x4*)(dO + off + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(TT::lo(o[i]), TT::lo(g[i]), acc);
      acc = fmaf(TT::hi(o[i]), TT::hi(g[i]), acc);
    }
  }
  // Reduce over the TPR consecutive lanes of the row (TPR divides 64).
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) {
    delta[row] = acc;
    lse2[row] = LSE[row] * kLog2e;
  }
}

// ---------------------------------------------------------------- shared

// Arguments of the two main kernels. Dense: Q, O-side tensors [B, H, N, D],
// K, V [B, H / group, N, D], statistics [B, H, N]. Packed variable-length
// batch (cu != null): Q [total, H, D], K, V [total, H / group, D],
// statistics [H, total]; sequence b is tokens [cu[b], cu[b+1]). Query head
// h reads K/V head h / group in both.
struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse2;
  const float* delta;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const int32_t* cu;
  int seqlen;        // dense N, or the longest packed sequence
  int total;         // packed: tokens in the batch
  int batch;         // sequences
  int heads, group;  // query heads; query heads per K/V head
  int n_tiles;       // per sequence: key tiles (dK/dV) or query tiles (dQ)
  float c;           // |scale| * log2(e)
  float grad_scale;  // scale, for dK (dK/dV kernel) or dQ (dQ kernel)
  uint32_t qsign;
  DropParams drop;   // dense batches only
  int diag;          // query i sees keys 0 .. i + diag (0: causal; >= N: all)
  int round_major;   // work order of small grids (see each kernel)
};

// Where sequence b's rows are: its length, the element offsets of row 0 of
// query head h and of K/V head hk, their row strides, and the offset of
// head h's statistics.
struct SeqRows {
  int N;
  size_t qbase, qstride, kvbase, kvstride, sbase;
};
template <int D>
__device__ __forceinline__ SeqRows seq_rows(const BwdParams& p, int b, int h, int hk) {
  SeqRows r;
  const int hkv = p.heads / p.group;
  if (p.cu) {
    int s0;
    seq_span(p.cu, b, p.total, p.seqlen, s0, r.N);
    r.qbase = ((size_t)s0 * p.heads + h) * D;
    r.qstride = (size_t)p.heads * D;
    r.kvbase = ((size_t)s0 * hkv + hk) * D;
    r.kvstride = (size_t)hkv * D;
    r.sbase = (size_t)h * p.total + s0;
  } else {
    r.N = p.seqlen;
    r.qbase = ((size_t)b * p.heads + h) * (size_t)p.seqlen * D;
    r.qstride = D;
    r.kvbase = ((size_t)b * hkv + hk) * (size_t)p.seqlen * D;
    r.kvstride = D;
    r.sbase = ((size_t)b * p.heads + h) * (size_t)p.seqlen;
  }
  return r;
}

// ---------------------------------------------------------------- dK, dV

template <typename TT, int D, bool DROP, bool COMPACT>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(const BwdParams prm) {
  constexpr int BK = kBwdKeyTile;        // keys per workgroup: 32 per wave pair
  constexpr int BM = 64;                 // query rows per iteration
  constexpr int ROWB = 2 * D;
  constexpr int TILEB = BM * ROWB;
  constexpr int DB = D / 32;
  constexpr int KK = D / 16;
  __shared__ __attribute__((aligned(1024))) char qt0[TILEB];
  __shared__ __attribute__((aligned(1024))) char qt1[TILEB];
  __shared__ __attribute__((aligned(1024))) char gt0[TILEB];
  __shared__ __attribute__((aligned(1024))) char gt1[TILEB];
  __shared__ __attribute__((aligned(16))) float st0[2 * BM];  // lse2 then delta
  __shared__ __attribute__((aligned(16))) float st1[2 * BM];
  // P of each pair: [pair][q-block][4 x u32x4 per lane][64 lanes], fp32.
  __shared__ __attribute__((aligned(16))) f32x4 pex[4 * 2 * 4 * 64];
  // With dropout, the keep flags of each pair's scores (role B computes
  // them, role A masks its dV operand with them): [pair][q-block][64 lanes].
  __shared__ __attribute__((aligned(16))) u32x4 kex[DROP ? 4 * 2 * 64 : 1];
  // With dropout: each role-B wave's area for the keep bytes' quad transpose.
  __shared__ __attribute__((aligned(16))) uint32_t dxa[DROP ? 4 * kQuadXWords : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lq = lane & 31, hi = lane >> 5;
  const int pair = w & 3;
  const bool role_a = w < 4;  // S, P, dV; the other wave of the pair: dP, dS, dK

  const float c = prm.c;
  const uint32_t qsign = prm.qsign;
  const DropParams& drop = prm.drop;
  // One (sequence b, K/V head hk, key tile): key tiles with the most query
  // tiles first, heads pinned to XCDs. Units run head-major, so that each
  // XCD's share holds every sequence of a few heads (sequences of unequal
  // length would otherwise load the XCDs unevenly). Unit-major (the
  // default): each XCD runs one unit's key tiles after another, sharing its
  // Q and dO in L2. Round-major (small grids): round r takes key tile r of
  // every unit, which spreads heavy and light tiles evenly over the CUs. The
  // group's query heads all contribute to this tile's dK and dV.
  // COMPACT (packed batches within bwd_packed_compact_ok's limits): a grid
  // of only real key tiles, in the unit-major order below.
  int unit, kt;
  if constexpr (COMPACT) {
    const int g8 = (prm.heads / prm.group) >> 3;
    int j, b;
    if (!bwd_packed_compact_wave(prm.cu, prm.batch, prm.total, prm.seqlen, BK, g8,
                                 (int)(blockIdx.x >> 3), lane, j, b, kt))
      return;  // past the batch's last key tile
    unit = ((int)(blockIdx.x & 7) * g8 + j) * prm.batch + b;
  } else {
    bwd_unit_slot(blockIdx.x, gridDim.x, prm.round_major != 0, prm.batch * (prm.heads / prm.group),
                  prm.n_tiles, unit, kt);
  }
  const int hk = unit / prm.batch, bidx = unit - hk * prm.batch;
  const SeqRows sr0 = seq_rows<D>(prm, bidx, hk * prm.group, hk);
  const int N = sr0.N;
  // Element and statistics offsets from one query head to the next (the
  // group's heads are consecutive), so the loop below never re-reads the
  // sequence offsets.
  const size_t q_head = prm.cu ? (size_t)D : (size_t)N * D;
  const size_t s_head = prm.cu ? (size_t)prm.total : (size_t)N;
  const int k0 = kt * BK;
  if (k0 >= N) return;  // a key tile past the end of a shorter sequence
  LdsOffsets<D> ldo;
  ldo.init(lane);

  // This pair's 32 keys as the B operand of S = Q K^T (role A) or of
  // dP = dO V^T (role B): lane (key lq, half hi), k-step kk -> row[16kk + 8hi ..].
  const int kw0 = k0 + 32 * pair;
  const int key = kw0 + lq;
  // All loads go out together: keys past N read key N - 1 and are zeroed
  // afterwards (a load under a per-key branch made the compiler wait for the
  // first ones before issuing the rest).
  u32x4 bf[KK];
  {
    const uint16_t* Xh = (role_a ? prm.k : prm.v) + sr0.kvbase +
                         (size_t)min(key, N - 1) * sr0.kvstride + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) bf[kk] = *(const u32x4*)(Xh + 16 * kk);
    const uint32_t kmask = key < N ? 0xffffffffu : 0u;
    // K sign-flipped for negative scale: S = Q (-K)^T (exact).
    const uint32_t ksign = role_a ? qsign : 0u;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) bf[kk] = (bf[kk] ^ ksign) & kmask;
  }
  f32x16 acc[DB];  // dV^T (role A) or dK^T (role B): lane = key, register = dim
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  const int nq = (N + BM - 1) / BM;
  // The first query tile with a row that sees key k0.
  const int i_begin = max(0, k0 - prm.diag) / BM;
  // Work items u = g * nqg + (i - i_begin): query head hk * group + g, query
  // tile i, so that one loop covers every query row of the group.
  const int nqg = nq - i_begin;
  const int n_items = prm.group * nqg;
  auto item_head = [&] __device__ (int u) __attribute__((always_inline)) {
    return hk * prm.group + u / nqg;
  };
  auto item_tile = [&] __device__ (int u) __attribute__((always_inline)) {
    return i_begin + u % nqg;
  };

  // Item u: Q and dO rows go straight to LDS; threads 0..127 fetch the
  // tile's lse2 (0..63) and delta (64..127) values into a register, stored
  // to LDS by store_stats once this iteration's reads are done.
  auto load_qtile = [&] __device__ (int u, char* qd, char* gd) __attribute__((always_inline)) {
    const int g = u / nqg, i = i_begin + (u - g * nqg);
    const size_t qbase = sr0.qbase + (size_t)g * q_head, sbase = sr0.sbase + (size_t)g * s_head;
    load_rows64<D>(prm.q + qbase, sr0.qstride, i * BM, N, qd, w, lane);
    load_rows64<D>(prm.dout + qbase, sr0.qstride, i * BM, N, gd, w, lane);
    float v = 0.f;
    if (tid < 2 * BM) {
      const int row = min(i * BM + (tid & (BM - 1)), N - 1);
      v = tid < BM ? prm.lse2[sbase + row] : prm.delta[sbase + row];
    }
    return v;
  };
  auto store_stats = [&] __device__ (float* sd, float v) __attribute__((always_inline)) {
    if (tid < 2 * BM) sd[tid] = v;
  };

  // Role A, phase 1: S = Q K^T for one 32-row query block, P (masked),
  // P to LDS for the pair, P packed as the B operand of dV^T += dO^T P.
  auto phase_a1 = [&] __device__ (auto masked, int i, int h, const char* qt, const float* st,
                                  int qb, u32x4 (&pp)[2]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(masked)::value;
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) s = TT::mma(rd_row<D>(qt, 32 * qb, ldo, kk), bf[kk], s);
    float p[16];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4 l4 = *(const f32x4*)(st + 32 * qb + 8 * m + 4 * hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * m + e;
        float x = fast_exp2(fmaf(s[r], c, -l4[e]));
        if (MASK) {
          const int q = i * BM + 32 * qb + 8 * m + 4 * hi + e;
          const bool ok = q < N && key < N && key <= q + prm.diag;
          x = ok ? x : 0.f;
        }
        p[r] = x;
      }
    }
    // P goes to the partner unmasked; with dropout the dV operand is masked
    // after the barrier, with the keep flags the partner computed meanwhile.
    f32x4* dst = pex + ((pair * 2 + qb) * 4) * 64 + lane;
#pragma unroll
    for (int m = 0; m < 4; ++m) dst[64 * m] = f32x4{p[4 * m], p[4 * m + 1], p[4 * m + 2], p[4 * m + 3]};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) pp[h][e] = TT::pack2(p[8 * h + 2 * e], p[8 * h + 2 * e + 1]);
  };

  // Role B, phase 1: dP = dO V^T for one query block.
  // With dropout, also the keep flags of the block (lane = key, register =
  // row, the layout of S and dP), kept for phase 2 and shared with role A:
  // Philox work that overlaps this role's products instead of lengthening
  // role A's phase 1, which the barrier waits for.
  auto phase_b1 = [&] __device__ (const char* gt, int qb, f32x16& dp, int i, int h, u32x4& kf)
      __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) dp = TT::mma(rd_row<D>(gt, 32 * qb, ldo, kk), bf[kk], dp);
    if constexpr (DROP) {
      kf = keep_flags_keys(drop, bidx * prm.heads + h, key, i * BM + 32 * qb, hi, lane,
                           dxa + pair * kQuadXWords);
      kex[(pair * 2 + qb) * 64 + lane] = kf;
    }
  };

  // Role A, phase 2: dV^T += dO^T P.
  auto phase_a2 = [&] __device__ (const char* gt, int qb, const u32x4 (&pp0)[2]) __attribute__((always_inline)) {
    u32x4 pp[2] = {pp0[0], pp0[1]};
    if constexpr (DROP) {
      // Elements 8 h + 2 e and 8 h + 2 e + 1: bytes 2 (e % 2) and
      // 2 (e % 2) + 1 of flag word 2 h + e / 2.
      const u32x4 kf = kex[(pair * 2 + qb) * 64 + lane];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) pp[h][e] &= keep_mask_pair(kf[2 * h + (e >> 1)], e & 1);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc[db] = TT::mma(rd_tr<D>(gt, 32 * qb + 16 * h, ldo, db), pp[h], acc[db]);
  };

  // Role B, phase 2: dS = P (dP - delta), dK^T += Q^T dS.
  auto phase_b2 = [&] __device__ (const char* qt, const float* st, int qb, const f32x16& dp,
                                  const u32x4& kf) __attribute__((always_inline)) {
    const f32x4* src = pex + ((pair * 2 + qb) * 4) * 64 + lane;
    float ds[16];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4 p4 = src[64 * m];
      const f32x4 d4 = *(const f32x4*)(st + BM + 32 * qb + 8 * m + 4 * hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (DROP) {
          // dS = P (keep * dP / (1 - p) - delta): the scaled dP, its bits
          // cleared where dropped.
          const float t = dp[4 * m + e] * drop.inv_keep;
          const float g = __uint_as_float(__float_as_uint(t) & keep_mask_elem(kf[m], e));
          ds[4 * m + e] = p4[e] * (g - d4[e]);
        } else {
          ds[4 * m + e] = p4[e] * (dp[4 * m + e] - d4[e]);
        }
      }
    }
    u32x4 sp[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) sp[h][e] = TT::pack2(ds[8 * h + 2 * e], ds[8 * h + 2 * e + 1]);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc[db] = TT::mma(rd_tr<D>(qt, 32 * qb + 16 * h, ldo, db), sp[h], acc[db]);
  };

  // One query tile of one role: phase 1, barrier (P visible), phase 2.
  auto iteration = [&] __device__ (auto is_a, int u, const char* qt, const char* gt, const float* st)
      __attribute__((always_inline)) {
    if constexpr (decltype(is_a)::value) {
      const int i = item_tile(u), h = item_head(u);
      const bool masked = (i * BM + prm.diag < k0 + BK) || (i * BM + BM > N) || (k0 + BK > N);
      u32x4 pp[2][2];
      if (masked) {
        phase_a1(std::true_type{}, i, h, qt, st, 0, pp[0]);
        phase_a1(std::true_type{}, i, h, qt, st, 1, pp[1]);
      } else {
        phase_a1(std::false_type{}, i, h, qt, st, 0, pp[0]);
        phase_a1(std::false_type{}, i, h, qt, st, 1, pp[1]);
      }
      __syncthreads();
      phase_a2(gt, 0, pp[0]);
      phase_a2(gt, 1, pp[1]);
    } else {
      f32x16 dp[2];
      u32x4 kf[2] = {};
      const int i = DROP ? item_tile(u) : 0, h = DROP ? item_head(u) : 0;
      phase_b1(gt, 0, dp[0], i, h, kf[0]);
      phase_b1(gt, 1, dp[1], i, h, kf[1]);
      __syncthreads();
      phase_b2(qt, st, 0, dp[0], kf[0]);
      phase_b2(qt, st, 1, dp[1], kf[1]);
    }
  };

  // Double-buffered query tiles, two per loop iteration so that every LDS
  // buffer is named statically. The barrier at the end of an iteration
  // makes the next tile (loaded during this one) visible and frees this
  // tile's buffers and the P exchange area. The two roles run separate
  // copies of the loop with the same barriers.
  auto run = [&] __device__ (auto is_a) __attribute__((always_inline)) {
    if (n_items > 0) {
      store_stats(st0, load_qtile(0, qt0, gt0));
      wait_vmem();
      __syncthreads();
    }
    for (int u = 0; u < n_items; u += 2) {
      float v1 = 0.f;
      if (u + 1 < n_items) v1 = load_qtile(u + 1, qt1, gt1);
      iteration(is_a, u, qt0, gt0, st0);
      store_stats(st1, v1);
      wait_vmem();
      __syncthreads();
      if (u + 1 >= n_items) break;
      float v0 = 0.f;
      if (u + 2 < n_items) v0 = load_qtile(u + 2, qt0, gt0);
      iteration(is_a, u + 1, qt1, gt1, st1);
      store_stats(st0, v0);
      wait_vmem();
      __syncthreads();
    }
  };
  if (role_a) run(std::true_type{});
  else run(std::false_type{});

  // dK = scale * acc (role B), dV = acc (role A), rounded to the dtype. Lane
  // lq holds key kw0 + lq; register r holds dim 32 db + 8(r/4) + 4 hi + r%4.
  // The rows leave through LDS (store_tile_rows), each wave's tile in half of
  // one query tile buffer once every wave is done with them.
  __syncthreads();
  {
    const int bsel = w >> 1;
    char* buf = bsel == 0 ? qt0 : bsel == 1 ? qt1 : bsel == 2 ? gt0 : gt1;
    const float sc = role_a ? (DROP ? drop.inv_keep : 1.f) : prm.grad_scale;
    store_tile_rows<TT, D>(acc, sc, buf + (w & 1) * 32 * (2 * D),
                           (role_a ? prm.dv : prm.dk) + sr0.kvbase + (size_t)kw0 * sr0.kvstride,
                           sr0.kvstride, N - kw0, lane);
  }
}

// ---------------------------------------------------------------- dQ

template <typename TT, int D, bool DROP, bool COMPACT>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(const BwdParams prm) {
  constexpr int BM = kBwdQueryTile;  // query rows per workgroup: 32 per wave
  static_assert(BM == 32 * kWaves, "one 32-row block per wave");
  constexpr int BN = 64;           // keys per LDS tile
  constexpr int ROWB = 2 * D;
  constexpr int TILEB = BN * ROWB;
  constexpr int DB = D / 32;
  constexpr int KK = D / 16;
  __shared__ __attribute__((aligned(1024))) char kb0[TILEB];
  __shared__ __attribute__((aligned(1024))) char kb1[TILEB];
  __shared__ __attribute__((aligned(1024))) char vb0[TILEB];
  __shared__ __attribute__((aligned(1024))) char vb1[TILEB];
  // With dropout: each wave's area for the keep bytes' quad transpose.
  __shared__ __attribute__((aligned(16))) uint32_t dxa[DROP ? kWaves * kQuadXWords : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lq = lane & 31, hi = lane >> 5;
  const float c = prm.c;
  const float dq_scale = prm.grad_scale;
  const uint32_t qsign = prm.qsign;
  const DropParams& drop = prm.drop;
  // One (sequence b, query head h, query tile); units (b, h) numbered
  // head-major, heads pinned to XCDs, heaviest causal query tiles first.
  // Unit-major (the default): each XCD runs one unit's tiles after another,
  // which keeps that unit's K/V in its L2. Round-major (grids of at most two
  // workgroups per CU): round r takes every unit's r-th tile counted back
  // from the end of its sequence, the forward's order, which pairs heavy and
  // light tiles on each CU exactly. Head h reads K/V head h / group.
  // COMPACT: a grid of only real query tiles, in the unit-major order.
  int unit, round;
  if constexpr (COMPACT) {
    const int g8 = prm.heads >> 3;
    int j, b;
    if (!bwd_packed_compact_wave(prm.cu, prm.batch, prm.total, prm.seqlen, BM, g8,
                                 (int)(blockIdx.x >> 3), lane, j, b, round))
      return;  // past the batch's last query tile
    unit = ((int)(blockIdx.x & 7) * g8 + j) * prm.batch + b;
  } else {
    bwd_unit_slot(blockIdx.x, gridDim.x, prm.round_major != 0, prm.batch * prm.heads, prm.n_tiles,
                  unit, round);
  }
  const int h = unit / prm.batch, bidx = unit - h * prm.batch;
  const int bh = bidx * prm.heads + h;
  const SeqRows sr = seq_rows<D>(prm, bidx, h, h / prm.group);
  const int N = sr.N;
  // Unit-major counts from the longest sequence's end (its empty slots
  // then sit at the start of the unit's range), round-major from this
  // sequence's own end.
  // (The compact order's rank r is query tile n_b - 1 - r of its unit.)
  const int qt = COMPACT ? (N + BM - 1) / BM - 1 - round
                         : bwd_dq_tile(round, prm.round_major != 0, prm.n_tiles, N, BM);
  if (qt < 0) return;  // a slot past the end of a shorter sequence
  const int q0 = qt * BM;
  LdsOffsets<D> ldo;
  ldo.init(lane);
  const uint16_t* Kh = prm.k + sr.kvbase;
  const uint16_t* Vh = prm.v + sr.kvbase;

  // This wave's 32 rows of Q (sign-flipped for negative scale) and dO as B
  // operands of S^T = K Q^T and dP^T = V dO^T, and the rows' statistics.
  const int qw0 = q0 + 32 * w;
  const int qi = qw0 + lq;
  // All loads go out together: rows past N read row N - 1 and are zeroed
  // afterwards (under a per-row branch the compiler waited for the first
  // loads before issuing the rest).
  const bool row_ok = qi < N;
  const int qc = min(qi, N - 1);
  u32x4 qf[KK], gf[KK];
  {
    const size_t roff = sr.qbase + (size_t)qc * sr.qstride + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qf[kk] = *(const u32x4*)(prm.q + roff + 16 * kk);
      gf[kk] = *(const u32x4*)(prm.dout + roff + 16 * kk);
    }
    const uint32_t qmask = row_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qf[kk] = (qf[kk] ^ qsign) & qmask;
      gf[kk] = gf[kk] & qmask;
    }
  }
  const float l2r = prm.lse2[sr.sbase + qc], dlr = prm.delta[sr.sbase + qc];
  const float l2 = row_ok ? l2r : 0.f;
  const float dl = row_ok ? dlr : 0.f;

  f32x16 acc[DB];  // dQ^T: lane = query, register = dim
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  const int kv_end = min(N, q0 + BM + prm.diag);
  const int ntile = (kv_end + BN - 1) / BN;
  const int wave_end = min(N, qw0 + 32 + prm.diag);
  const int last_b = qw0 < N ? (wave_end - 1) / 32 : -1;  // last 32-key block of this wave
  int first_edge = (N % 32) ? (N - 1) / 32 : (kv_end + 31) / 32;
  first_edge = min(first_edge, (qw0 + prm.diag) / 32);

  // One 32-key block (half of the tile in kt/vt).
  auto block = [&] __device__ (auto masked, int b, const char* kt, const char* vt)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(masked)::value;
    const int half = b & 1;
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
    // The two products: without dropout left to the compiler's interleave
    // (the whole training backward 0.2-0.8 % faster than with them fenced
    // apart, in interleaved runs on two boxes); with dropout fenced, so that
    // one set of operand fragments
    // is live at a time (unfenced, the keep bytes' registers push it into
    // spills).
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) s = TT::mma(rd_row<D>(kt, 32 * half, ldo, kk), qf[kk], s);
    if constexpr (DROP) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) dp = TT::mma(rd_row<D>(vt, 32 * half, ldo, kk), gf[kk], dp);
    if constexpr (DROP) __builtin_amdgcn_sched_barrier(0);
    float ds[16];
    u32x4 kb = {};
    if constexpr (DROP) kb = keep_bytes_rows(drop, bh, qi, 32 * b, hi, lane, dxa + w * kQuadXWords);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = fast_exp2(fmaf(s[r], c, -l2));
      if (MASK) {
        const int kidx = 32 * b + 8 * (r >> 2) + 4 * hi + (r & 3);
        const bool ok = kidx < N && kidx <= qi + prm.diag;
        p = ok ? p : 0.f;
      }
      if constexpr (DROP) {
        // dS = P (keep * dP / (1 - p) - delta)
        ds[r] = p * ((byte_kept(kb, r, drop.thr) ? dp[r] * drop.inv_keep : 0.f) - dl);
      } else {
        ds[r] = p * (dp[r] - dl);
      }
    }
    u32x4 sp[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) sp[h][e] = TT::pack2(ds[8 * h + 2 * e], ds[8 * h + 2 * e + 1]);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc[db] = TT::mma(rd_tr<D>(kt, 32 * half + 16 * h, ldo, db), sp[h], acc[db]);
  };
  auto any_block = [&] __device__ (int b, const char* kt, const char* vt) __attribute__((always_inline)) {
    if (b > last_b) return;
    if (b >= first_edge) block(std::true_type{}, b, kt, vt);
    else block(std::false_type{}, b, kt, vt);
  };

  load_rows64<D>(Kh, sr.kvstride, 0, N, kb0, w, lane);
  load_rows64<D>(Vh, sr.kvstride, 0, N, vb0, w, lane);
  wait_vmem();
  __syncthreads();
  for (int t = 0; t < ntile; t += 2) {
    if (t + 1 < ntile) {
      load_rows64<D>(Kh, sr.kvstride, (t + 1) * BN, N, kb1, w, lane);
      load_rows64<D>(Vh, sr.kvstride, (t + 1) * BN, N, vb1, w, lane);
    }
    any_block(2 * t, kb0, vb0);
    any_block(2 * t + 1, kb0, vb0);
    wait_vmem();
    __syncthreads();
    if (t + 1 >= ntile) break;
    if (t + 2 < ntile) {
      load_rows64<D>(Kh, sr.kvstride, (t + 2) * BN, N, kb0, w, lane);
      load_rows64<D>(Vh, sr.kvstride, (t + 2) * BN, N, vb0, w, lane);
    }
    any_block(2 * t + 2, kb1, vb1);
    any_block(2 * t + 3, kb1, vb1);
    wait_vmem();
    __syncthreads();
  }

  // dQ = scale * acc, rounded to the dtype: lane lq holds query qi; register
  // r holds dim 32 db + 8(r/4) + 4 hi + r%4. The rows leave through LDS
  // (store_tile_rows), each wave's tile in half of one K/V tile buffer once
  // every wave is done with them.
  __syncthreads();
  {
    const int bsel = w >> 1;
    char* buf = bsel == 0 ? kb0 : bsel == 1 ? kb1 : bsel == 2 ? vb0 : vb1;
    store_tile_rows<TT, D>(acc, dq_scale, buf + (w & 1) * 32 * (2 * D),
                           prm.dq + sr.qbase + (size_t)qw0 * sr.qstride, sr.qstride, N - qw0,
                           lane);
  }
}

template <typename TT, int D>
hipError_t launch_typed(const BwdArgs& a, const BwdWorkspace& ws) {
  char* wsb = (char*)a.workspace;
  float* delta = (float*)(wsb + ws.delta_off);
  float* lse2 = (float*)(wsb + ws.lse2_off);
  const bool packed = a.cu_seqlens != nullptr;
  const int64_t rows = packed ? a.H * a.total : a.B * a.H * a.N;

  const int64_t pre_threads = rows * (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<TT, D>), dim3((unsigned)((pre_threads + 255) / 256)),
                     dim3(256), 0, a.stream, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse,
                     delta, lse2, rows, packed ? a.total : (int64_t)0, (int)a.H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const float c = fabsf(a.scale) * kLog2e;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  // For scale < 0 the scores are formed from -K (dK/dV kernel) or -Q (dQ
  // kernel) with |scale|; the gradients dK = scale dS^T Q and dQ = scale dS K
  // use the unflipped operands.
  const int64_t hkv = a.H_kv > 0 ? a.H_kv : a.H;
  BwdParams prm{};
  prm.q = (const uint16_t*)a.q;
  prm.k = (const uint16_t*)a.k;
  prm.v = (const uint16_t*)a.v;
  prm.dout = (const uint16_t*)a.dout;
  prm.lse2 = lse2;
  prm.delta = delta;
  prm.dq = (uint16_t*)a.dq;
  prm.dk = (uint16_t*)a.dk;
  prm.dv = (uint16_t*)a.dv;
  prm.cu = a.cu_seqlens;
  prm.seqlen = (int)a.N;
  prm.total = packed ? (int)a.total : 0;
  prm.batch = (int)a.B;
  prm.heads = (int)a.H;
  prm.group = (int)(a.H / hkv);
  prm.c = c;
  prm.grad_scale = a.scale;
  prm.qsign = qsign;
  prm.drop = a.drop;

  // Grids and work orders (round-major for small causal grids): bwd_shape.
  const BwdShape sh = bwd_shape(a.B, a.H, hkv, a.N, a.causal != 0);
  // Packed batches: grids of only real tiles where the limits allow.
  const bool c1 = packed && bwd_packed_compact_ok(a.B, hkv, sh.rm_dkdv);
  const bool c2 = packed && bwd_packed_compact_ok(a.B, a.H, sh.rm_dq);
  const dim3 g1((unsigned)(c1 ? bwd_packed_compact_grid(a.B, a.total, hkv, kBwdKeyTile, sh.n_ktiles)
                              : sh.grid_dkdv));
  const dim3 g2((unsigned)(c2 ? bwd_packed_compact_grid(a.B, a.total, a.H, kBwdQueryTile,
                                                        sh.n_qtiles)
                              : sh.grid_dq));
  prm.diag = a.causal ? 0 : (int)a.N;
  auto go = [&](auto drop) -> hipError_t {
    constexpr bool DR = decltype(drop)::value;
    BwdParams p1 = prm;
    p1.n_tiles = sh.n_ktiles;
    p1.round_major = sh.rm_dkdv;
    if (c1)
      hipLaunchKernelGGL((bwd_dkdv_kernel<TT, D, DR, true>), g1, dim3(kThreads), 0, a.stream, p1);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<TT, D, DR, false>), g1, dim3(kThreads), 0, a.stream, p1);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    BwdParams p2 = prm;
    p2.n_tiles = sh.n_qtiles;
    p2.round_major = sh.rm_dq;
    if (c2)
      hipLaunchKernelGGL((bwd_dq_kernel<TT, D, DR, true>), g2, dim3(kThreads), 0, a.stream, p2);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<TT, D, DR, false>), g2, dim3(kThreads), 0, a.stream, p2);
    return hipGetLastError();
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  return a.drop.thr != 0 ? go(T_{}) : go(F_{});
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, const BwdWorkspace& ws) {
  if (a.dtype == FA_BF16)
    return a.D == 64 ? launch_typed<Bf16, 64>(a, ws) : launch_typed<Bf16, 128>(a, ws);
  return a.D == 64 ? launch_typed<F16, 64>(a, ws) : launch_typed<F16, 128>(a, ws);
}

}  // namespace fa
