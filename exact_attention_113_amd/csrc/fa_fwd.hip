// Fused attention forward for bf16/fp16 inputs on gfx950.
//
// One workgroup owns 256 (or 128) query rows of one (batch, head) and streams
// the key/value rows through LDS, keeping per query row a running maximum,
// a running sum of exponentials and an unnormalised fp32 output accumulator
// (online softmax: "From Self-Attention to FlashAttention", section 2;
// "FlashAttention in ops-transformer", "Core idea" and "Online softmax").
// Scores and probabilities live only in registers; O and the row
// logsumexp are the only results written back (the flash data flow of
// section 1 of the first page: only O goes back to HBM).
//
// Waves. Eight waves, two per SIMD, each owning 32 consecutive query rows
// and all of their keys; for short sequences, two waves per 32 rows, each
// taking every other 32-key block, merged at the end.
// Scores are computed transposed, S^T = K Q^T (32x32x16 MFMA, fp32
// accumulate): lane j and j + 32 share one query and each holds 16 of a
// 32-key block's scores, so row maxima and sums are in-register reductions
// plus one exchange of the wave halves. The output is accumulated
// transposed as well, O^T = V^T P^T, whose B operand is the probability
// tile as the score MFMA left it in registers.
//
// Pipeline. Keys are processed in 32-key blocks. Step b issues the score
// MFMAs of block b + 1 and the P V MFMAs of block b - 1 and, in between
// them, the softmax of block b: the softmax depends on neither MFMA group,
// so the matrix core and the vector ALU of a SIMD work at the same time,
// within a wave and across the two waves sharing the SIMD. The accumulator
// is rescaled lazily: a row's reference maximum moves only when a block's
// maximum exceeds it by more than kTau (log2 units), so probabilities are
// bounded by 2^kTau; the rescale (a rare, wave-uniform branch) is applied
// before the next P V product.
//
// Memory path. K and V tiles of 64 keys go from global memory straight
// into LDS with global_load_lds_dwordx4 (no staging registers), double
// buffered, one barrier per tile (at D = 64: four buffers per tensor, one
// barrier per two tiles). The tile buffers are separate LDS arrays
// addressed statically (the tile loop is unrolled), so the compiler can
// tell that the operand reads of one buffer do not wait for the direct
// loads still landing in another. O leaves through LDS as whole rows. Each 16-byte chunk of a row is
// stored at an XOR-swizzled position so that the MFMA operand reads hit
// distinct LDS banks. V stays row-major in LDS; its transposed A operand
// is read with ds_read_b64_tr_b16, which hands lane i of each 16-lane group
// element i%4 of the chunks addressed by lanes 4j + i/4 (j = 0..3).
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

// Workgroups of eight waves, one per CU. Each wave takes 32 rows and all of
// their keys (256 rows per workgroup) when the grid is large enough: causal
// attention needs more such workgroups than the 256 CUs (a second round, so
// that light tiles of the causal triangle follow the heavy ones), full
// attention, whose workgroups all take equally long, more than half as many.
// Otherwise (short grids) a workgroup takes 128 rows and the two waves of
// each 32-row group split the keys (KS = 2): the key loop, the critical path
// of such grids, halves, and a SIMD still runs two waves. Measured (D128):
// causal B1 H32 N2048 (256 tiles) 54.9 us split against 57.7 whole; causal
// grids of 384 tiles 13-19 % faster whole (B1 H48 N2048 81 against 66 us);
// B1 H32 N4096 (512 tiles) 161 split against 133 whole; full attention B1
// H32 N1024 (128 tiles) 27.1 split against 32.4 whole, N1536 (192 tiles)
// 63.4 against 51.2, N2048 88.1 against 73.8. (Four-wave workgroups of 128
// rows with whole key ranges, one wave per SIMD, measured 8 % slower than
// the split at causal N = 1024 and 15 % at B2 H8 N512 D64.)
// At head dim 64 the shortest grids split the keys four ways (64-row
// workgroups, 128-key tiles). (The grid rule, kMaxSplitCausal,
// kMaxSplitFull and kMaxSplit4, is fwd_shape in fa_sched.h.)
constexpr int kBN = 64;                 // keys per LDS tile (whole key ranges, two splits)
constexpr int kKB = 32;                 // keys per pipeline step
constexpr float kTau = 8.0f;
constexpr float kSumCap = 256.0f;       // 2^kTau

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
using False = std::false_type;
using True = std::true_type;
// Softmax kind of a step: False = interior block, True = block with masked
// keys, Unmasked = full softmax without masks (a row's first block).
struct Unmasked : std::false_type {};

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Kernel arguments. Dense: Q, K, V, O are [B, H, N, D] and LSE [B, H, N].
// Packed variable-length batches (cu != null): Q and O are [total, H, D], K
// and V [total, H / group, D], LSE [H, total]; sequence b holds tokens
// [cu[b], cu[b+1]). Query head h reads K/V head h / group in both layouts.
struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* cu;  // sequence starts (batch + 1 entries) or null
  int seqlen;         // dense: N; packed: the longest sequence
  int total;          // packed: tokens in the batch
  int heads;          // query heads
  int group;          // query heads per K/V head
  int n_qtiles;
  int bh_count;
  int pair_order;     // pairwise XCD order of the tiles (fwd_tile_of)
  int lpt;            // packed: only real tiles, heaviest first (fwd_packed_lpt_wave)
  float c;
  uint32_t qsign;
  DropParams drop;    // dense batches only
  // Query i sees keys 0 .. i + diag: 0 for causal attention, at least the
  // sequence length (every key) otherwise.
  int diag;
};

// Causal and full attention run the same code: full attention is the causal
// mask moved past the last key (diag >= N), which leaves only the tail of
// the keys to mask. (A separate full-attention instantiation, with its mask
// folded away at compile time, came out of register allocation with spills
// in the key loop and ran 1.46x slower at N = 4096, D = 128.)
template <typename TT, int D, int NW, bool DROP, int KS>
__global__ __launch_bounds__(64 * NW, 1) void fwd_kernel(const FwdParams prm) {
  // KS = 2 or 4 (short sequences): the waves form NW / KS row groups of 32
  // rows, and the KS waves of a group take every KS-th 32-key block of its
  // keys, cutting the key loop's length KS-fold; their partial results are
  // merged at the end (the same rescale-and-add as between blocks of the
  // online softmax). A K/V tile then holds one block per split.
  constexpr int NRG = NW / KS;                // row groups of 32 query rows
  constexpr int kBM = 32 * NRG;               // query rows per workgroup
  constexpr int BN = KS == 4 ? 128 : kBN;     // keys per LDS tile
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int ROWB = 2 * D;                 // bytes per row
  constexpr int TILEB = BN * ROWB;            // bytes per K or V tile
  constexpr int RPI = 64 / CH;                // rows per wave-wide direct load (1 KiB)
  constexpr int LPW = BN / (NW * RPI);        // direct loads per wave, tile and tensor
  constexpr int DB = D / 32;                  // 32-row blocks of the head dim
  constexpr int KK = D / 16;                  // k-steps of the score MFMA
  static_assert(LPW >= 1, "tile too small for one direct load per wave");
  __shared__ __attribute__((aligned(1024))) char kb0[TILEB];
  __shared__ __attribute__((aligned(1024))) char kb1[TILEB];
  __shared__ __attribute__((aligned(1024))) char vb0[TILEB];
  __shared__ __attribute__((aligned(1024))) char vb1[TILEB];
  // Whole key ranges at D = 64 (GROUP2): four K and four V tile buffers and
  // one barrier per two tiles. (At D = 128 the per-tile barrier measured
  // faster: 141 against 144 us at B1 H32 N4096 causal; at D = 64 the group
  // of four steps measured 93 against 99.5 us.)
  constexpr bool GROUP2 = KS == 1 && D == 64;
  constexpr int TILEB2 = GROUP2 ? TILEB : 1024;
  __shared__ __attribute__((aligned(1024))) char kb2[TILEB2];
  __shared__ __attribute__((aligned(1024))) char kb3[TILEB2];
  __shared__ __attribute__((aligned(1024))) char vb2[TILEB2];
  __shared__ __attribute__((aligned(1024))) char vb3[TILEB2];
  // Merge of the key splits: reference and sum share of each wave but the
  // first of its row group.
  constexpr int NX = KS > 1 ? NRG * (KS - 1) : 1;
  __shared__ float xm[NX][64], xl[NX][64];
  // With dropout: each wave's area for the keep bytes' quad transpose.
  __shared__ __attribute__((aligned(16))) uint32_t dxa[DROP ? NW * kQuadXWords : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lq = lane & 31, hi = lane >> 5;
  const int rg = w % NRG, kh = w / NRG;  // row group; key split (KS > 1)

  const float c = prm.c;
  const uint32_t qsign = prm.qsign;
  // This workgroup's (sequence bidx, head h, query tile qt).
  const int batch = prm.bh_count / prm.heads;
  int qt, h, bidx;
  if (prm.lpt) {
    int hl;
    if (!fwd_packed_lpt_wave(prm.cu, batch, prm.total, prm.seqlen, kBM, prm.n_qtiles,
                             prm.heads >> 3, (int)(blockIdx.x >> 3), lane, bidx, hl, qt))
      return;  // past the batch's last tile
    h = (int)(blockIdx.x & 7) * (prm.heads >> 3) + hl;
  } else {
    int p;
    fwd_tile_of(blockIdx.x, prm.n_qtiles, prm.bh_count, prm.pair_order != 0, qt, p);
    h = p / batch;
    bidx = p - h * batch;
  }
  // This (sequence, head): its length N, the element offsets of its first
  // Q/O and K/V rows and of its LSE entries, and the row strides.
  const int bh = bidx * prm.heads + h;
  const int hkv = prm.heads / prm.group, hk = h / prm.group;
  int N;
  size_t qbase, kvbase, lbase;
  size_t sq, skv;
  if (prm.cu) {
    int s0;
    seq_span(prm.cu, bidx, prm.total, prm.seqlen, s0, N);
    qbase = ((size_t)s0 * prm.heads + h) * D;
    kvbase = ((size_t)s0 * hkv + hk) * D;
    lbase = (size_t)h * prm.total + s0;
    sq = (size_t)prm.heads * D;
    skv = (size_t)hkv * D;
  } else {
    N = prm.seqlen;
    qbase = (size_t)bh * N * D;
    kvbase = ((size_t)bidx * hkv + hk) * N * D;
    lbase = (size_t)bh * N;
    sq = skv = D;
  }
  // Without the whole-batch order, packed batches count a sequence's tiles
  // back from its own last one, so that the slots past the end of shorter
  // sequences (no work) come last in the dispatch order instead of first.
  if (!prm.lpt) {
    qt = fwd_seq_tile(qt, prm.n_qtiles, N, kBM, prm.cu != nullptr);
    if (qt < 0) return;
  }
  const int q0 = qt * kBM;
  const uint16_t* Qh = prm.q + qbase;
  const uint16_t* Kh = prm.k + kvbase;
  const uint16_t* Vh = prm.v + kvbase;

  // This wave's 32 query rows and their B operands of S^T = K Q^T:
  // lane (query lq, half hi), k-step kk -> Q[row][16*kk + 8*hi + 0..7].
  const int qw0 = q0 + 32 * rg;
  const int qi = qw0 + lq;
  // All eight loads go out together (rows past N read row N - 1 and are
  // zeroed afterwards: a load under a per-row branch made the compiler wait
  // for the first ones before issuing the rest).
  u32x4 qf[KK];
  const uint16_t* qrow = Qh + (size_t)min(qi, N - 1) * sq + 8 * hi;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const u32x4*)(qrow + 16 * kk);
  const uint32_t qmask = qi < N ? 0xffffffffu : 0u;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = (qf[kk] ^ qsign) & qmask;  // sign flip for negative scale (exact)

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float mref = -INFINITY;  // reference maximum of the row, log2 units
  float lsum = 0.f;        // this lane's share of the row sum
  float alpha = 1.f;       // pending rescale factor of the accumulator
  bool rescale = false;    // wave-uniform: some lane's alpha differs from 1

  // Key range of the workgroup and of this wave: up to the last visible key
  // of its last row.
  const int diag = prm.diag;
  const int kv_end = min(N, q0 + kBM + diag);
  const int nb = (kv_end + kKB - 1) / kKB;  // 32-key steps of the workgroup
  const int ntile = (kv_end + BN - 1) / BN;
  const int wave_end = min(N, qw0 + 32 + diag);
  // Last step this wave computes (-1: every row of the wave is past N).
  const int last_b = qw0 < N ? (wave_end - 1) / kKB : -1;
  // First step whose scores need a mask: the block holding this wave's
  // first diagonal key, or the partial block at the end of the keys.
  int first_edge = (N % kKB) ? (N - 1) / kKB : nb;
  first_edge = min(first_edge, (qw0 + diag) / kKB);
  // Steps [1, interior_end) need neither masks nor drains.
  const int interior_end = min(last_b + 1, first_edge);

  // V chunk swizzle: the transposing reads of one half-wave cover four
  // consecutive rows (r & 3 = 0..3) and four 16-byte chunks of each; the
  // XOR spreads those rows over all 64 banks (256-byte rows, D = 128) or
  // over both bank halves they alternate between (128-byte rows, D = 64).
  auto vswz = [](int r) __attribute__((always_inline)) {
    return CH == 16 ? 4 * (r & 3) : 2 * (r & 3);
  };

  // Direct global->LDS load of rows [t*BN, t*BN + BN) of X into dst.
  // Lane l of load i writes row R0 + l/CH at chunk position l%CH, fetching
  // the chunk that the swizzle puts there; rows past N repeat row N-1
  // (their scores are masked).
  auto load_tile = [&](const uint16_t* Xh, int t, char* dst, bool is_v)
      __attribute__((always_inline)) {
    const int k0 = t * BN;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int R0 = (w * LPW + i) * RPI;
      const int r = R0 + lane / CH, p = lane % CH;
      const int cg = is_v ? (p ^ vswz(r)) : (p ^ (r % CH));
      const int grow = min(k0 + r, N - 1);
      __builtin_amdgcn_global_load_lds(Xh + (size_t)grow * skv + cg * 8,
                                       (lds_void*)(dst + R0 * ROWB), 16, 0, 0);
    }
  };

  // Per-lane parts of the LDS operand addresses.
  const int kxor = lq % CH;
  const int koff = lq * ROWB;
  const int tj = (lane & 15) >> 2, tm = lane & 3, dsub = (lane >> 4) & 1;
  const int vlane = (4 * hi + tj) * ROWB + 8 * (tm & 1);
  const int vx = (2 * dsub + (tm >> 1)) ^ vswz(tj);

  // Scores of the 32-key half `half` of the K tile in kt: S^T = K Q^T.
  auto scores = [&](const char* kt, int half, f32x16& s) __attribute__((always_inline)) {
    const char* row = kt + 32 * half * ROWB + koff;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 a = *(const u32x4*)(row + 16 * ((2 * kk + hi) ^ kxor));
      s = TT::mma(a, qf[kk], s);
    }
  };

  // O^T += V^T P^T for the 32-key half `half` of the V tile in vt. Slot e
  // of lane half hi in k-step h of the B operand is key
  // 16*h + 4*hi + (e<4 ? e : e+4) of that half.
  auto pv = [&](const char* vt, int half, const u32x4 (&pf)[2]) __attribute__((always_inline)) {
    const char* base0 = vt + 32 * half * ROWB + vlane;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char* base = base0 + 16 * h * ROWB + 16 * ((4 * db) ^ vx);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)base);
        const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * ROWB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 u2 = __builtin_bit_cast(u32x2, up);
        const u32x4 a = {l2[0], l2[1], u2[0], u2[1]};
        oacc[db] = TT::mma(a, pf[h], oacc[db]);
      }
  };

  // Dropout on the P V operand only: the row sum (and so LSE) keeps every
  // probability, the kept ones enter P V unscaled and O is scaled by
  // 1 / (1 - p) at the end.
  auto drop_operand = [&](int b, const float (&p)[16], u32x4 (&pf)[2])
      __attribute__((always_inline)) {
    // Elements 8 h + 2 e and 8 h + 2 e + 1 are bytes 2 (e % 2) and
    // 2 (e % 2) + 1 of flag word 2 h + e / 2; a dropped one's half is cleared.
    const u32x4 g = keep_flags_rows(prm.drop, bh, qi, kKB * b, hi, lane, dxa + w * kQuadXWords);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * h + 2 * e;
        pf[h][e] = TT::pack2(p[r], p[r + 1]) & keep_mask_pair(g[2 * h + (e >> 1)], e & 1);
      }
  };

  // Softmax of block b: mask (edge steps), row max, lazy reference update,
  // probabilities packed as the B operands of the P V product, row sum.
  auto softmax_full = [&](auto edge, int b, f32x16& s, u32x4 (&pf)[2])
      __attribute__((always_inline)) {
    constexpr bool EDGE = decltype(edge)::value;
    // Edge steps: a key past N or past the row's diagonal is excluded. Its
    // score becomes -inf for the maximum and its probability exactly 0
    // (not exp2(-inf * c), which is NaN when the scale is 0).
    uint32_t okm = 0xffffu;
    if (EDGE) {
      okm = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kKB * b + 8 * (r >> 2) + 4 * hi + (r & 3);
        const bool ok = key < N && key <= qi + diag;
        okm |= ok ? (1u << r) : 0u;
        s[r] = ok ? s[r] : -INFINITY;
      }
    }
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = half_swap_max(mx);
    // Block maximum in log2 units; a fully masked block stays -inf.
    const float tmx = (EDGE && mx == -INFINITY) ? -INFINITY : mx * c;
    const bool need = tmx > mref + kTau;
    const float mnew = need ? tmx : mref;
    const float a = need ? fast_exp2(mref - mnew) : 1.f;  // exp2(-inf) = 0 at the start
    alpha = a;
    mref = mnew;
    const float nm = -mnew;
    float p[16];
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = fast_exp2(fmaf(s[r], c, nm));
      if (EDGE) x = ((okm >> r) & 1u) ? x : 0.f;
      p[r] = x;
      sum += x;
    }
    lsum = fmaf(lsum, a, sum);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) pf[h][e] = TT::pack2(p[8 * h + 2 * e], p[8 * h + 2 * e + 1]);
    if constexpr (DROP) drop_operand(b, p, pf);
    rescale = wave_any(need);
  };

  // Softmax of an interior block once the row's reference is set: the
  // probabilities are taken against the current reference without a block
  // maximum. A lane whose 16 probabilities sum to at most 2^kTau has none
  // above 2^kTau, which is all the lazy rescaling needs; only when some lane
  // of the wave exceeds that (a new, much larger maximum, or overflow to
  // inf) is the block redone by the full softmax above, which moves the
  // reference. The fast path ends with its results pinned so that they are
  // computed here, interleaved with this step's MFMAs, and not moved past
  // the rare branch.
  auto softmax = [&](auto edge, int b, f32x16& s, u32x4 (&pf)[2]) __attribute__((always_inline)) {
    using E = decltype(edge);
    if constexpr (std::is_same<E, Unmasked>::value) {
      softmax_full(False{}, b, s, pf);
    } else if constexpr (E::value) {
      softmax_full(True{}, b, s, pf);
    } else {
      const float nm = -mref;
      float p[16];
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(fmaf(s[r], c, nm));
        sum += p[r];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) pf[h][e] = TT::pack2(p[8 * h + 2 * e], p[8 * h + 2 * e + 1]);
      if constexpr (DROP) drop_operand(b, p, pf);
      const float lprev = lsum;
      lsum = lprev + sum;
      rescale = false;
      asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(lsum));
      if (wave_any(!(sum <= kSumCap))) {
        lsum = lprev;
        softmax_full(False{}, b, s, pf);
      }
    }
  };

  // Apply the pending rescale to the accumulator (before the next P V).
  auto apply_rescale = [&]() __attribute__((always_inline)) {
    if (rescale) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
  };

  // Two score buffers and two probability buffers, used alternately by
  // odd and even steps so that every index below is a compile-time one.
  f32x16 sA, sB;
  u32x4 pA[2], pB[2];

  // One pipeline step: scores of block b+1 (K tile kt), P V of block b-1
  // (V tile vt), softmax of block b. `cur` holds S(b) on entry, `nxt`
  // receives S(b+1); `pprev` holds P(b-1), `pcur` receives P(b). The scores
  // of the block after a wave's last one are computed and never used (they
  // read a stale but in-bounds LDS buffer), which keeps the step free of
  // branches.
  auto step = [&](auto edge, auto has_pv, int b, const char* kt, const char* vt, f32x16& cur,
                  f32x16& nxt, const u32x4 (&pprev)[2], u32x4 (&pcur)[2])
      __attribute__((always_inline)) {
    apply_rescale();
    scores(kt, KS == 1 ? (b + 1) & 1 : kh, nxt);
    if constexpr (decltype(has_pv)::value) pv(vt, KS == 1 ? (b - 1) & 1 : kh, pprev);
    softmax(edge, b, cur, pcur);
  };
  // A step of a wave whose rows may need masks or be done: the full step
  // while b is one of its steps, the last block's P V right after its last
  // step, nothing afterwards (it still takes part in the barriers).
  auto any_step = [&](int b, const char* kt, const char* vt, f32x16& cur, f32x16& nxt,
                      const u32x4 (&pprev)[2], u32x4 (&pcur)[2]) __attribute__((always_inline)) {
    if (b <= last_b) {
      if (b >= first_edge) step(True{}, True{}, b, kt, vt, cur, nxt, pprev, pcur);
      else step(False{}, True{}, b, kt, vt, cur, nxt, pprev, pcur);
    } else if (b == last_b + 1) {
      apply_rescale();
      pv(vt, (b - 1) & 1, pprev);
    }
  };
  // Steps 2T+1 and 2T+2 read K tile T+1 (kt) and V tile T (vt): S(2T+1)
  // is in sB and P(2T) in pA on entry.
  auto tile_steps = [&](int T, const char* kt, const char* vt) __attribute__((always_inline)) {
    const int b = 2 * T + 1;
    if (b + 1 < interior_end) {
      step(False{}, True{}, b, kt, vt, sB, sA, pA, pB);
      step(False{}, True{}, b + 1, kt, vt, sA, sB, pB, pA);
    } else {
      any_step(b, kt, vt, sB, sA, pA, pB);
      if (b + 1 < nb) any_step(b + 1, kt, vt, sA, sB, pB, pA);
    }
  };
  // Barrier before step 2T+1: K tile T and V tile T-1 are no longer read
  // and the loads issued at the previous barrier have landed; then K tile
  // T+2 and V tile T+1 go out (into the buffers just freed).
  auto tile_barrier = [&](int T, char* kdst, char* vdst) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (T + 2 < ntile) load_tile(Kh, T + 2, kdst, false);
    if (T + 1 < ntile) load_tile(Vh, T + 1, vdst, true);
  };

  // Prologue: K tiles 0 and 1 and V tile 0 (GROUP2: also K tile 2 and V
  // tile 1, which the first group of four steps reads).
  load_tile(Kh, 0, kb0, false);
  load_tile(Vh, 0, vb0, true);
  if (ntile > 1) load_tile(Kh, 1, kb1, false);
  if constexpr (GROUP2) {
    if (ntile > 2) load_tile(Kh, 2, kb2, false);
    if (ntile > 1) load_tile(Vh, 1, vb1, true);
  }
  wait_vmem();
  __syncthreads();

  if constexpr (KS == 1) {
    // The scores of block 0 and step 0 (no P V yet).
    if (last_b >= 0) {
      scores(kb0, 0, sA);
      // Edge variant even without masks: the reference is not set yet, so
      // step 0 takes the full softmax (with masks only where needed).
      if (first_edge == 0) step(True{}, False{}, 0, kb0, vb0, sA, sB, pB, pA);
      else step(Unmasked{}, False{}, 0, kb0, vb0, sA, sB, pB, pA);
    }

    if constexpr (!GROUP2) {
      // Two tiles per iteration so that every buffer is named statically:
      // even tiles T read K from kb1 and V from vb0, odd tiles K from kb0 and
      // V from vb1.
      for (int T = 0; 2 * T + 1 < nb; T += 2) {
        tile_barrier(T, kb0, vb1);
        tile_steps(T, kb1, vb0);
        if (2 * T + 3 < nb) {
          tile_barrier(T + 1, kb1, vb0);
          tile_steps(T + 1, kb0, vb1);
        }
      }
    } else {
      // K tile t lives in kb[t % 4] and V tile t in vb[t % 4]. Group G is
      // steps 4G+1 .. 4G+4: K tiles 2G+1, 2G+2 and V tiles 2G, 2G+1. The
      // barrier before it frees the tiles group G-1 read and sends K tiles
      // 2G+3, 2G+4 and V tiles 2G+2, 2G+3 there (read by group G+1). Two
      // groups per iteration so that every buffer is named statically.
      auto group_barrier = [&](int G, char* k0d, char* k1d, char* v0d, char* v1d)
          __attribute__((always_inline)) {
        wait_vmem();
        __syncthreads();
        if (2 * G + 3 < ntile) load_tile(Kh, 2 * G + 3, k0d, false);
        if (2 * G + 4 < ntile) load_tile(Kh, 2 * G + 4, k1d, false);
        if (2 * G + 2 < ntile) load_tile(Vh, 2 * G + 2, v0d, true);
        if (2 * G + 3 < ntile) load_tile(Vh, 2 * G + 3, v1d, true);
      };
      for (int G = 0; 4 * G + 1 < nb; G += 2) {
        group_barrier(G, kb3, kb0, vb2, vb3);
        tile_steps(2 * G, kb1, vb0);
        if (4 * G + 3 < nb) tile_steps(2 * G + 1, kb2, vb1);
        if (4 * G + 5 < nb) {
          group_barrier(G + 1, kb1, kb2, vb0, vb1);
          tile_steps(2 * G + 2, kb3, vb2);
          if (4 * G + 7 < nb) tile_steps(2 * G + 3, kb0, vb3);
        }
      }
    }
    // The last step's P V when it was the workgroup's last step (its V tile
    // is visible after this barrier).
    wait_vmem();
    __syncthreads();
    if (last_b == nb - 1 && last_b >= 0) {
      apply_rescale();
      const u32x4(&pl)[2] = (last_b & 1) ? pB : pA;
      const int vt = (last_b >> 1) & (GROUP2 ? 3 : 1);
      if (vt == 0) pv(vb0, last_b & 1, pl);
      else if (vt == 1) pv(vb1, last_b & 1, pl);
      else if (vt == 2) pv(vb2, last_b & 1, pl);
      else pv(vb3, last_b & 1, pl);
    }

    // O = acc / sum rounded to the dtype; LSE = ln 2 * (ref + log2 sum).
    const float ltot = half_swap_sum(lsum);
    const float inv = (DROP ? prm.drop.inv_keep : 1.f) / ltot;
    if (qi < N && hi == 0) prm.lse[lbase + qi] = kLn2 * (mref + __log2f(ltot));
    // O leaves through LDS as whole rows (store_tile_rows), each wave's tile
    // in half of one tile buffer, free once every wave has finished its last
    // P V product.
    __syncthreads();
    char* stage;
    {
      const int bsel = w >> 1;
      char* buf = bsel == 0 ? kb0 : bsel == 1 ? kb1 : bsel == 2 ? vb0 : vb1;
      stage = buf + (w & 1) * 32 * ROWB;
    }
    store_tile_rows<TT, D>(oacc, inv, stage, prm.o + qbase + (size_t)qw0 * sq, sq, N - qw0, lane);
  } else {
    // Key splits: this wave's step j computes block KS j + kh, the kh-th
    // 32-key block of K/V tile j, so one step per tile. K tile t lives in
    // kb[t % 2] and V tile t in vb[t % 2]; step j reads K tile j + 1 and V
    // tile j - 1, and the barrier before it sends K tile j + 2 and V tile j
    // into the buffers step j - 1 was the last to read. K tile 2 goes out
    // once every wave has taken block kh's scores from K tile 0.
    const int jl = last_b >= kh ? (last_b - kh) / KS : -1;  // this wave's last step
    const int jmax = (nb - 1) / KS;                         // the workgroup's last block step
    if (jl >= 0) scores(kb0, kh, sA);
    __syncthreads();
    if (ntile > 2) load_tile(Kh, 2, kb0, false);
    if (jl >= 0) {
      if (first_edge <= kh) step(True{}, False{}, kh, kb1, vb0, sA, sB, pB, pA);
      else step(Unmasked{}, False{}, kh, kb1, vb0, sA, sB, pB, pA);
    }
    auto half_step = [&](int j, const char* kt, const char* vt, f32x16& cur, f32x16& nxt,
                         const u32x4(&pprev)[2], u32x4(&pcur)[2]) __attribute__((always_inline)) {
      const int b = KS * j + kh;
      if (j <= jl) {
        if (b >= first_edge) step(True{}, True{}, b, kt, vt, cur, nxt, pprev, pcur);
        else step(False{}, True{}, b, kt, vt, cur, nxt, pprev, pcur);
      } else if (j == jl + 1) {
        apply_rescale();
        pv(vt, kh, pprev);
      }
    };
    for (int j = 1; j <= jmax + 1; j += 2) {
      wait_vmem();
      __syncthreads();
      if (j + 2 < ntile) load_tile(Kh, j + 2, kb1, false);
      if (j < ntile) load_tile(Vh, j, vb1, true);
      half_step(j, kb0, vb0, sB, sA, pA, pB);
      if (j + 1 <= jmax + 1) {
        wait_vmem();
        __syncthreads();
        if (j + 3 < ntile) load_tile(Kh, j + 3, kb0, false);
        if (j + 1 < ntile) load_tile(Vh, j + 1, vb0, true);
        half_step(j + 1, kb1, vb1, sA, sB, pB, pA);
      }
    }

    // The waves of splits 1 .. KS-1 hand their reference maximum, sum share
    // and accumulator to the wave of split 0 with the same rows, each through
    // a slot of its own in the tile buffers (free once every wave is past
    // its last P V); that wave rescales all of them to the largest
    // reference, adds, and stores.
    wait_vmem();
    __syncthreads();
    constexpr int SLOTB = DB * 16 * 64 * 4;  // bytes of one wave's accumulator
    constexpr int PERBUF = TILEB / SLOTB;    // slots per tile buffer
    static_assert(PERBUF >= 1 && 4 * PERBUF >= NRG * (KS - 1), "merge slots exceed the buffers");
    auto slot_ptr = [&](int sl) __attribute__((always_inline)) {
      const int bsel = sl / PERBUF;
      char* buf = bsel == 0 ? kb0 : bsel == 1 ? kb1 : bsel == 2 ? vb0 : vb1;
      return (float*)(buf + (sl % PERBUF) * SLOTB);
    };
    if (kh > 0) {
      const int sl = rg * (KS - 1) + kh - 1;
      float* xo = slot_ptr(sl);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(f32x4*)(xo + 4 * ((db * 4 + r4) * 64 + lane)) =
              f32x4{oacc[db][4 * r4], oacc[db][4 * r4 + 1], oacc[db][4 * r4 + 2],
                    oacc[db][4 * r4 + 3]};
      xm[sl][lane] = mref;
      xl[sl][lane] = lsum;
    }
    __syncthreads();
    if (kh == 0) {
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
        const int sl = rg * (KS - 1) + x;
        const float m1 = xm[sl][lane];
        const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
        lsum = fmaf(xl[sl][lane], a1, lsum);
        const float* xo = slot_ptr(sl);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 o1 = *(const f32x4*)(xo + 4 * ((db * 4 + r4) * 64 + lane));
#pragma unroll
            for (int e = 0; e < 4; ++e)
              oacc[db][4 * r4 + e] = fmaf(o1[e], a1, oacc[db][4 * r4 + e]);
          }
        // One partner's accumulator at a time in registers.
        asm volatile("" ::: "memory");
      }
      mref = mm;
      const float ltot = half_swap_sum(lsum);
      const float inv = (DROP ? prm.drop.inv_keep : 1.f) / ltot;
      if (qi < N && hi == 0) prm.lse[lbase + qi] = kLn2 * (mref + __log2f(ltot));
      // The wave has read all of its row group's slots: it stages its rows
      // in the first of them (store_tile_rows).
      store_tile_rows<TT, D>(oacc, inv, (char*)slot_ptr(rg * (KS - 1)),
                             prm.o + qbase + (size_t)qw0 * sq, sq, N - qw0, lane);
    }
  }
}

template <typename TT, int D>
hipError_t launch_half(const FwdArgs& a) {
  FwdParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k;
  p.v = (const uint16_t*)a.v;
  p.o = (uint16_t*)a.o;
  p.lse = a.lse;
  p.cu = a.cu_seqlens;
  p.seqlen = (int)a.N;  // dense N, or the longest packed sequence
  p.total = (int)a.total;
  p.heads = (int)a.H;
  p.group = (int)(a.H / a.H_kv);
  p.bh_count = (int)(a.B * a.H);
  p.c = fabsf(a.scale) * kLog2e;
  p.qsign = a.scale < 0.f ? 0x80008000u : 0u;
  p.drop = a.drop;
  p.diag = a.causal ? 0 : (int)a.N;
  const FwdShape sh = fwd_shape(p.bh_count, a.N, a.causal != 0, D);
  p.n_qtiles = sh.n_qtiles;
  p.pair_order = sh.pairs && a.cu_seqlens == nullptr;
  p.lpt = a.cu_seqlens != nullptr && fwd_packed_lpt_ok(a.B, a.H, sh.n_qtiles);
  const int64_t grid_size =
      p.lpt ? fwd_packed_lpt_grid(a.B, a.total, a.H, sh.bm, sh.n_qtiles) : sh.grid;
  auto go = [&](auto ks) {
    constexpr int KS = decltype(ks)::value;
    const dim3 grid((unsigned)grid_size);
    if (a.drop.thr != 0)
      hipLaunchKernelGGL((fwd_kernel<TT, D, 8, true, KS>), grid, dim3(512), 0, a.stream, p);
    else
      hipLaunchKernelGGL((fwd_kernel<TT, D, 8, false, KS>), grid, dim3(512), 0, a.stream, p);
  };
  if (sh.ks == 1) go(std::integral_constant<int, 1>{});
  else if (sh.ks == 2 || D != 64) go(std::integral_constant<int, 2>{});
  else if constexpr (D == 64) go(std::integral_constant<int, 4>{});
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
