// Attention of a few new tokens against a key/value cache (decode), bf16 /
// fp16 on gfx950.
//
// Each step of token-by-token generation brings only the new tokens' queries
// but reads the whole, growing cache ("Flash Attention algorithm design and
// I/O optimisation", "Training and inference value"), so the work is bound
// by streaming K and V from HBM once. New token t of a sequence with L cached
// tokens sits at position L - s_q + t and sees cache keys 0 .. L - s_q + t.
//
// Work split (split-KV). One workgroup takes one (sequence, K/V head, key
// chunk): all query heads of the group sharing that K/V head and all s_q new
// tokens become the rows of one 32-row MFMA tile, so every K/V byte is read
// once per step. Its four waves take every fourth 32-key block of the chunk
// and keep their own online-softmax state (running maximum, running sum,
// fp32 accumulator: "From Self-Attention to FlashAttention", section 2). Each
// wave loads its blocks itself, one block ahead: K straight into registers
// (the score MFMA's A operand) and V through its own double-buffered LDS
// region (direct global->LDS loads; the P V product reads it transposed),
// so the key loop needs no workgroup barrier, and two workgroups fit on a
// CU to keep enough bytes in flight for HBM. At
// the end the four partial states are merged through LDS with the same
// rescale-and-add, and the chunk's (O, LSE) is written: straight to the
// output when the cache is one chunk, else to a workspace that
// decode_merge_kernel combines over the chunks by LSE.
//
// Products follow the forward kernel: S^T = K Q^T and O^T = V^T P^T on
// 32x32x16 MFMAs, V read transposed from LDS with ds_read_b64_tr_b16. The
// head dim is split between the two lane halves of the score MFMA as
// d = (D/2) * half + 8 * step + element, the same for K and Q, so that each
// lane reads one contiguous half row of K.
#include <utility>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDKB = 32;  // keys per block

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Loads whose completion the kernel tracks itself. The compiler's own
// counting of outstanding loads turns conservative (a wait for all of them)
// once direct global->LDS loads are in flight, which would serialise the
// one-block-ahead prefetch; these are issued as plain instructions instead,
// and every value they produce passes through an explicit s_waitcnt that
// names it as an operand before its first use.
template <int I>
__device__ __forceinline__ void load16_async(u32x4& dst, const uint16_t* p) {
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=v"(dst) : "v"(p), "n"(16 * I));
}
template <int KK, int... I>
__device__ __forceinline__ void load_row_async(u32x4 (&dst)[KK], const uint16_t* p,
                                               std::integer_sequence<int, I...>) {
  (load16_async<I>(dst[I], p), ...);
}
// Wait until at most N vector-memory loads are outstanding; `k` are the
// registers the waited loads wrote.
template <int N>
__device__ __forceinline__ void wait_vm(u32x4 (&k)[8]) {
  asm volatile("s_waitcnt vmcnt(%8)"
               : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]), "+v"(k[4]), "+v"(k[5]),
                 "+v"(k[6]), "+v"(k[7])
               : "n"(N)
               : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm(u32x4 (&k)[4]) {
  asm volatile("s_waitcnt vmcnt(%4)"
               : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3])
               : "n"(N)
               : "memory");
}
// The LDS reads are complete (s_waitcnt lgkmcnt(0) just before); this ties
// their registers to that point so no use moves above it.
__device__ __forceinline__ void wait_lgkm_tied(u32x4 (&a)[8]) {
  asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
               "+v"(a[6]), "+v"(a[7]));
}
__device__ __forceinline__ void wait_lgkm_tied(u32x4 (&a)[4]) {
  asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
}
__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

struct DecParams {
  const uint16_t* q;        // [B, s_q, H, D]
  const uint16_t* k;        // [B, cap, H_kv, D]
  const uint16_t* v;        // [B, cap, H_kv, D]
  uint16_t* o;              // [B, s_q, H, D]
  float* lse;               // [B, H, s_q]
  const int32_t* seqlens;   // [B] cached tokens per sequence
  float* part_o;            // [B, H, s_q, n_splits, D] (split mode)
  float* part_lse;          // [B, H, s_q, n_splits]    (split mode)
  int batch, s_q, cap, max_len, heads, hkv, group, n_splits, chunk;
  float c;                  // |scale| * log2(e)
  uint32_t qsign;           // sign flip of Q for a negative scale
};

template <typename TT, int D>
__global__ __launch_bounds__(kDecThreads, 2) void decode_kernel(const DecParams prm) {
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int ROWB = 2 * D;              // bytes per row
  constexpr int BLKB = kDKB * ROWB;        // bytes of one K or V block
  constexpr int RPI = 64 / CH;             // rows per wave-wide direct load
  constexpr int LPB = kDKB / RPI;          // direct loads per block and tensor
  constexpr int DB = D / 32;               // 32-row blocks of the head dim
  constexpr int KK = D / 16;               // k-steps of the score MFMA
  constexpr int OC = D / 4;                // 16-byte chunks of an fp32 output row
  constexpr int SLAB = 32 * D * 4;         // one wave's fp32 rows in the merge
  static_assert(kDecWaves * BLKB >= 2 * SLAB, "merge buffer too small");
  // Per wave: one V block per buffer. The merge reuses both buffers, two
  // waves' slabs in each.
  __shared__ __attribute__((aligned(1024))) char vb0[kDecWaves * BLKB];
  __shared__ __attribute__((aligned(1024))) char vb1[kDecWaves * BLKB];
  __shared__ float stat_m[kDecWaves][32];
  __shared__ float stat_l[kDecWaves][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lq = lane & 31, hi = lane >> 5;

  int b, hk, split;
  if (prm.batch <= kDecodeOrderMaxBatch) {
    // Active chunks first (decode_active_unit_wave); past them, nothing to do.
    hk = (int)(blockIdx.x % prm.hkv);
    if (!decode_active_unit_wave(prm.seqlens, prm.batch, prm.max_len, prm.chunk, prm.n_splits,
                                 (int)(blockIdx.x / prm.hkv), lane, b, split))
      return;
  } else {
    decode_unit(blockIdx.x, prm.n_splits, prm.hkv, b, hk, split);
  }
  const int L = min(max(prm.seqlens[b], 0), prm.max_len);
  const int k_lo = split * prm.chunk;
  const int k_hi = min(L, k_lo + prm.chunk);
  // Chunks past the cached keys write nothing: the merge weighs only the
  // first ones.
  if (split >= decode_active_chunks(L, prm.chunk, prm.n_splits)) return;
  const int nblk = k_hi > k_lo ? (k_hi - k_lo + kDKB - 1) / kDKB : 0;
  const int rows = prm.group * prm.s_q;

  // Row lq of the tile: query head hk * group + lq / s_q, new token lq % s_q.
  const int gq = lq / prm.s_q, tq = lq - gq * prm.s_q;
  const int h = hk * prm.group + gq;
  const bool row_ok = lq < rows;
  // Keys visible to this row within the chunk: [k_lo, lim).
  const int lim = min(min(L, L - prm.s_q + tq + 1), k_hi);

  // All loads go out together: lanes past the tile's rows read row 0 and are
  // zeroed afterwards (a load under a per-row branch made the compiler wait
  // for the first ones before issuing the rest).
  u32x4 qf[KK];
  {
    const int lqc = row_ok ? lq : 0;
    const int gqc = lqc / prm.s_q, tqc = lqc - gqc * prm.s_q;
    const uint16_t* qrow =
        prm.q + ((size_t)(b * prm.s_q + tqc) * prm.heads + hk * prm.group + gqc) * D + (D / 2) * hi;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const u32x4*)(qrow + 8 * kk);
    const uint32_t qmask = row_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = (qf[kk] ^ prm.qsign) & qmask;
  }
  wait_vm<0>(qf);

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float mrun = -INFINITY;  // running maximum, log2 units
  float lsum = 0.f;        // this lane's share of the running sum

  const size_t kv_stride = (size_t)prm.hkv * D;  // elements between cache rows
  const uint16_t* Kb = prm.k + ((size_t)b * prm.cap * prm.hkv + hk) * D;
  const uint16_t* Vb = prm.v + ((size_t)b * prm.cap * prm.hkv + hk) * D;

  auto vswz = [](int r) __attribute__((always_inline)) {
    return CH == 16 ? 4 * (r & 3) : 2 * (r & 3);
  };
  // Block j's loads: K row lq's half `hi` into registers (the score MFMA's
  // A operand), the 32 V rows into this wave's LDS region by direct loads.
  // Rows past the cache length repeat its last row (their scores are
  // masked). With live = false every lane reads the last row: a load that
  // keeps the loop free of branches (and so keeps the compiler's memory
  // counters exact) but whose data is never used.
  auto load_block = [&](int j, bool live, u32x4 (&kr)[KK], char* vdst)
      __attribute__((always_inline)) {
    const int key0 = k_lo + kDKB * j;
    const uint16_t* krow =
        Kb + (size_t)(live ? min(key0 + lq, L - 1) : L - 1) * kv_stride + (D / 2) * hi;
    load_row_async<KK>(kr, krow, std::make_integer_sequence<int, KK>{});
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      const int R0 = i * RPI;
      const int r = R0 + lane / CH, p = lane % CH;
      const int row = live ? min(key0 + r, L - 1) : L - 1;
      const void* vsrc = Vb + (size_t)row * kv_stride + (p ^ vswz(r)) * 8;
      __builtin_amdgcn_global_load_lds(vsrc, (lds_void*)(vdst + R0 * ROWB), 16, 0, 0);
    }
  };

  const int tj = (lane & 15) >> 2, tm = lane & 3, dsub = (lane >> 4) & 1;
  const int vlane = (4 * hi + tj) * ROWB + 8 * (tm & 1);
  const int vx = (2 * dsub + (tm >> 1)) ^ vswz(tj);

  // One 32-key block: scores, masked online softmax, P V.
  auto compute_block = [&](int j, const u32x4 (&kr)[KK], const char* vt)
      __attribute__((always_inline)) {
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) s = TT::mma(kr[kk], qf[kk], s);
    const int key0 = k_lo + kDKB * j;
    uint32_t okm = 0;
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      const bool ok = key < lim;
      okm |= ok ? (1u << r) : 0u;
      mx = ok ? fmaxf(mx, s[r]) : mx;
    }
    mx = half_swap_max(mx);
    const float tmx = mx == -INFINITY ? -INFINITY : mx * prm.c;
    const float mnew = fmaxf(mrun, tmx);
    // Nothing visible yet: keep alpha = 1 (the state is still empty).
    const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mrun - mnew);
    const float nm = -mnew;
    float p[16];
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = fast_exp2(fmaf(s[r], prm.c, nm));
      p[r] = ((okm >> r) & 1u) ? x : 0.f;
      sum += p[r];
    }
    lsum = fmaf(lsum, alpha, sum);
    mrun = mnew;
    if (wave_any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    u32x4 pf[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 4; ++e) pf[hh][e] = TT::pack2(p[8 * hh + 2 * e], p[8 * hh + 2 * e + 1]);
    // V's transposed reads (the direct loads that filled this buffer are
    // complete: the loop waited for them).
    u32x4 va[2 * DB];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t base = (uint32_t)(uintptr_t)(lds_void*)(vt + vlane + 16 * hh * ROWB +
                                                               16 * ((4 * db) ^ vx));
        const u32x2 lo = lds_read_tr16(base);
        const u32x2 up = lds_read_tr16(base + 8 * ROWB);
        va[hh * DB + db] = u32x4{lo[0], lo[1], up[0], up[1]};
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    wait_lgkm_tied(va);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = TT::mma(va[hh * DB + db], pf[hh], oacc[db]);
  };

  // This wave's blocks w, w + 4, ...: block i of the wave in register set
  // and V buffer i % 2, the next one loading while the current one is
  // computed (past the last block, a dummy load takes its place). A wave
  // reads only what it loaded itself, so waiting until at most the next
  // block's KK + LPB loads are in flight is the only sync; the LDS reads of
  // a buffer are complete before the next direct load into it is issued.
  u32x4 kA[KK], kB[KK];
  char* v0 = vb0 + w * BLKB;
  char* v1 = vb1 + w * BLKB;
  const int ni = nblk > w ? (nblk - w + kDecWaves - 1) / kDecWaves : 0;
  if (ni > 0) load_block(w, true, kA, v0);
  for (int i = 0; i < ni; i += 2) {
    load_block(w + kDecWaves * (i + 1), i + 1 < ni, kB, v1);
    wait_vm<KK + LPB>(kA);  // block i (K in kA, V in v0) has landed
    compute_block(w + kDecWaves * i, kA, v0);
    load_block(w + kDecWaves * (i + 2), i + 2 < ni, kA, v0);
    wait_vm<KK + LPB>(kB);
    if (i + 1 < ni) compute_block(w + kDecWaves * (i + 1), kB, v1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Merge the four waves' states: maximum M over the waves, each wave's
  // weight 2^(m_w - M) (0 for a wave that saw no key), total sum, and the
  // weighted accumulators summed through LDS.
  const float lrow = half_swap_sum(lsum);
  __syncthreads();  // every wave is done with its LDS blocks
  if (hi == 0) {
    stat_m[w][lq] = mrun;
    stat_l[w][lq] = lrow;
  }
  __syncthreads();
  auto row_stats = [&](int row, float& M, float& Ltot) __attribute__((always_inline)) {
    M = -INFINITY;
#pragma unroll
    for (int x = 0; x < kDecWaves; ++x) M = fmaxf(M, stat_m[x][row]);
    Ltot = 0.f;
#pragma unroll
    for (int x = 0; x < kDecWaves; ++x)
      Ltot += stat_m[x][row] == -INFINITY ? 0.f : fast_exp2(stat_m[x][row] - M) * stat_l[x][row];
  };
  {
    float M, Ltot;
    row_stats(lq, M, Ltot);
    const float f = mrun == -INFINITY ? 0.f : fast_exp2(mrun - M);
    // Row lq of wave w's slab, 16-byte chunk c stored at c ^ (lq % OC) so
    // that the 32 rows written together spread over the banks.
    float* ob = (float*)((w < 2 ? vb0 : vb1) + (w & 1) * SLAB) + (size_t)lq * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = oacc[db][4 * g4 + e] * f;
        const int cidx = 8 * db + 2 * g4 + hi;
        *(f32x4*)(ob + 4 * (cidx ^ (lq % OC))) = x;
      }
  }
  __syncthreads();
  {
    constexpr int SEG = D / 8;  // output elements per thread
    const int row = tid >> 3, d0 = (tid & 7) * SEG;
    if (row < rows) {
      float M, Ltot;
      row_stats(row, M, Ltot);
      const float inv = Ltot > 0.f ? 1.f / Ltot : 0.f;
      float acc[SEG];
#pragma unroll
      for (int e = 0; e < SEG; ++e) acc[e] = 0.f;
#pragma unroll
      for (int x = 0; x < kDecWaves; ++x) {
        const float* src = (const float*)((x < 2 ? vb0 : vb1) + (x & 1) * SLAB) + (size_t)row * D;
#pragma unroll
        for (int e = 0; e < SEG; e += 4) {
          const f32x4 y = *(const f32x4*)(src + 4 * (((d0 + e) / 4) ^ (row % OC)));
          acc[e] += y[0];
          acc[e + 1] += y[1];
          acc[e + 2] += y[2];
          acc[e + 3] += y[3];
        }
      }
      const int rg = row / prm.s_q, rt = row - rg * prm.s_q;
      const int rh = hk * prm.group + rg;
      const float lse_row = Ltot > 0.f ? kLn2 * (M + __log2f(Ltot)) : -INFINITY;
      if (prm.n_splits == 1) {
        uint16_t* orow = prm.o + ((size_t)(b * prm.s_q + rt) * prm.heads + rh) * D + d0;
#pragma unroll
        for (int e = 0; e < SEG; e += 8) {
          u32x4 out;
#pragma unroll
          for (int u = 0; u < 4; ++u) out[u] = TT::pack2(acc[e + 2 * u] * inv, acc[e + 2 * u + 1] * inv);
          *(u32x4*)(orow + e) = out;
        }
        if ((tid & 7) == 0) prm.lse[((size_t)b * prm.heads + rh) * prm.s_q + rt] = lse_row;
      } else {
        const size_t prow = ((size_t)(b * prm.heads + rh) * prm.s_q + rt) * prm.n_splits + split;
        float* po = prm.part_o + prow * D + d0;
#pragma unroll
        for (int e = 0; e < SEG; e += 4) {
          f32x4 y = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
          *(f32x4*)(po + e) = y;
        }
        if ((tid & 7) == 0) prm.part_lse[prow] = lse_row;
      }
    }
  }
}

// Decode with at most 16 query rows per (sequence, K/V head): the rows are
// the N side of 16x16x32 MFMAs (S^T = K Q^T and O^T = V^T P^T as above),
// which halves the accumulator, the Q fragments and the per-block softmax
// of the 32-row tile. V is loaded into registers like K and copied to a
// per-wave LDS stage just before its transposed reads, so that both of a
// block's tensors are held in registers while in flight: a wave refills a
// block's registers as soon as its scores are computed and its V is
// staged, which keeps two blocks in flight during the rest of the step
// (the 32-row kernel has room for one). All loads are ordinary ones whose
// completion the compiler tracks.
//
// Layouts (lane l, q = l % 16, row group g = l / 16 of the wave):
//  - score MFMA: A = K rows key0 + 16 t + q, B = Q row q; the head dim is
//    split as d = (D/4) g + 8 s + e for k-step s and element e, the same for
//    K and Q, so each lane reads one contiguous quarter row. The result
//    gives lane l the scores of query q against keys key0 + 16 t + 4 g + r.
//  - P V MFMA: B = P^T with lane l holding keys key0 + 4 g + r (elements
//    0..3) and key0 + 16 + 4 g + r (elements 4..7), which is exactly what
//    the score MFMAs left in the lane; A = V^T read transposed from the
//    stage with the same key order; the result gives lane l the output
//    elements d = 16 i + 4 g + r of query q.
template <typename TT, int D>
__global__ __launch_bounds__(kDecThreads, 2) void decode16_kernel(const DecParams prm) {
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int ROWB = 2 * D;      // bytes per row
  constexpr int KS = D / 32;       // k-steps of a score MFMA
  constexpr int DT = D / 16;       // 16-element tiles of the head dim
  constexpr int QW = D / 4;        // head-dim elements per row group in the score MFMA
  constexpr int RPL = 64 / CH;     // V rows per wave-wide load
  constexpr int VL = kDKB / RPL;   // V loads per lane and block
  constexpr int STAGE = kDKB * ROWB;
  constexpr int OC = D / 4;        // 16-byte chunks of an fp32 output row
  static_assert(16 * D * 4 <= STAGE, "merge slab exceeds a wave's stage");
  __shared__ __attribute__((aligned(1024))) char vst[kDecWaves * STAGE];
  __shared__ float stat_m[kDecWaves][16];
  __shared__ float stat_l[kDecWaves][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 15, g = lane >> 4;

  int b, hk, split;
  if (prm.batch <= kDecodeOrderMaxBatch) {
    // Active chunks first (decode_active_unit_wave); past them, nothing to do.
    hk = (int)(blockIdx.x % prm.hkv);
    if (!decode_active_unit_wave(prm.seqlens, prm.batch, prm.max_len, prm.chunk, prm.n_splits,
                                 (int)(blockIdx.x / prm.hkv), lane, b, split))
      return;
  } else {
    decode_unit(blockIdx.x, prm.n_splits, prm.hkv, b, hk, split);
  }
  const int L = min(max(prm.seqlens[b], 0), prm.max_len);
  const int k_lo = split * prm.chunk;
  const int k_hi = min(L, k_lo + prm.chunk);
  // Chunks past the cached keys write nothing: the merge weighs only the
  // first ones.
  if (split >= decode_active_chunks(L, prm.chunk, prm.n_splits)) return;
  const int nblk = k_hi > k_lo ? (k_hi - k_lo + kDKB - 1) / kDKB : 0;
  const int rows = prm.group * prm.s_q;

  // Query row q: head hk * group + q / s_q, new token q % s_q; it sees the
  // keys [k_lo, lim) of the chunk.
  const int gq = q / prm.s_q, tq = q - gq * prm.s_q;
  const bool row_ok = q < rows;
  const int lim = min(min(L, L - prm.s_q + tq + 1), k_hi);

  const size_t kv_stride = (size_t)prm.hkv * D;
  const uint16_t* Kb = prm.k + ((size_t)b * prm.cap * prm.hkv + hk) * D;
  const uint16_t* Vb = prm.v + ((size_t)b * prm.cap * prm.hkv + hk) * D;
  // Rows past the cache read its last row (their scores are masked); the
  // capacity is at least one row.
  const int last = max(L - 1, 0);
  char* stage = vst + w * STAGE;
  auto swz = [](int r) __attribute__((always_inline)) {
    return CH == 16 ? 4 * (r & 3) : 2 * (r & 3);
  };

  struct Blk {
    u32x4 k[2][KS];
    u32x4 v[VL];
  };
  auto load_block = [&](int j, Blk& x) __attribute__((always_inline)) {
    const int key0 = k_lo + kDKB * j;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t* kr = Kb + (size_t)min(key0 + 16 * t + q, last) * kv_stride + QW * g;
#pragma unroll
      for (int st = 0; st < KS; ++st) x.k[t][st] = *(const u32x4*)(kr + 8 * st);
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int r = RPL * i + lane / CH, c = lane % CH;
      x.v[i] = *(const u32x4*)(Vb + (size_t)min(key0 + r, last) * kv_stride + 8 * c);
    }
  };

  u32x4 qf[KS];
  f32x4 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY;  // running maximum of query q, log2 units
  float lsum = 0.f;        // this lane's share of the running sum

  // Transposed-read address of row group g, lane x = l % 16: row 4 g + x / 4
  // (the second read 16 rows further), head-dim elements 4 (x % 4) .. + 3 of
  // tile i, i.e. 16-byte chunk 2 i + (x % 4) / 2 at byte 8 (x % 2).
  const int trow = 4 * g + ((lane & 15) >> 2);
  const int tcol = ((lane & 15) >> 1) & 1;
  const uint32_t tbase = (uint32_t)(uintptr_t)(lds_void*)(stage + trow * ROWB + 8 * (lane & 1));

  // One block: stage V, scores, refill the block's registers (when `next`
  // names a block), masked online softmax, P V.
  auto compute_block = [&](int j, Blk& x, int next) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int r = RPL * i + lane / CH, c = lane % CH;
      *(u32x4*)(stage + r * ROWB + 16 * (c ^ swz(r))) = x.v[i];
    }
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) s[t] = TT::mma16(x.k[t][st], qf[st], s[t]);
    }
    if (next >= 0) load_block(next, x);
    const int key0 = k_lo + kDKB * j;
    uint32_t okm = 0;
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = key0 + 16 * t + 4 * g + r < lim;
        okm |= ok ? (1u << (4 * t + r)) : 0u;
        mx = ok ? fmaxf(mx, s[t][r]) : mx;
      }
    mx = quad_max(mx);
    const float tmx = mx == -INFINITY ? -INFINITY : mx * prm.c;
    const float mnew = fmaxf(mrun, tmx);
    // Nothing visible yet: keep alpha = 1 (the state is still empty).
    const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mrun - mnew);
    const float nm = -mnew;
    float p[8];
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(fmaf(s[t][r], prm.c, nm));
        p[4 * t + r] = ((okm >> (4 * t + r)) & 1u) ? e : 0.f;
        sum += p[4 * t + r];
      }
    lsum = fmaf(lsum, alpha, sum);
    mrun = mnew;
    if (wave_any(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < DT; ++i) oacc[i] *= alpha;
    }
    const u32x4 pf = {TT::pack2(p[0], p[1]), TT::pack2(p[2], p[3]), TT::pack2(p[4], p[5]),
                      TT::pack2(p[6], p[7])};
#pragma unroll
    for (int i = 0; i < DT; ++i) {
      const uint32_t a = tbase + 16 * ((2 * i + tcol) ^ swz(trow));
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)a);
      const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(a + 16 * ROWB));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), u2 = __builtin_bit_cast(u32x2, up);
      const u32x4 va = {l2[0], l2[1], u2[0], u2[1]};
      oacc[i] = TT::mma16(va, pf, oacc[i]);
    }
  };

  // This wave's blocks w, w + 4, ...: block i in register set i % 2. Both
  // first blocks are issued at once, then Q (after them: the compiler's wait
  // for Q covers both, so Q adds no round trip of its own); each block's
  // set is refilled with the block two further on while that block is
  // computed.
  const int ni = nblk > w ? (nblk - w + kDecWaves - 1) / kDecWaves : 0;
  if (ni > 0) {
    Blk A, B;
    load_block(w, A);
    load_block(w + kDecWaves, B);
    asm volatile("" ::: "memory");
    {
      const int qc = row_ok ? q : 0;
      const int gqc = qc / prm.s_q, tqc = qc - gqc * prm.s_q;
      const uint16_t* qrow =
          prm.q + ((size_t)(b * prm.s_q + tqc) * prm.heads + hk * prm.group + gqc) * D + QW * g;
#pragma unroll
      for (int st = 0; st < KS; ++st) qf[st] = *(const u32x4*)(qrow + 8 * st);
      const uint32_t qmask = row_ok ? 0xffffffffu : 0u;
#pragma unroll
      for (int st = 0; st < KS; ++st) qf[st] = (qf[st] ^ prm.qsign) & qmask;
    }
    // Inside the loop both sets are always refilled, so the loads in flight
    // at its head are the same on every pass and the compiler's waits stay
    // exact; the last two or three blocks follow it.
    int i = 0;
    for (; i + 3 < ni; i += 2) {
      compute_block(w + kDecWaves * i, A, w + kDecWaves * (i + 2));
      compute_block(w + kDecWaves * (i + 1), B, w + kDecWaves * (i + 3));
    }
    if (i + 2 < ni) {
      compute_block(w + kDecWaves * i, A, w + kDecWaves * (i + 2));
      compute_block(w + kDecWaves * (i + 1), B, -1);
      compute_block(w + kDecWaves * (i + 2), A, -1);
    } else {
      compute_block(w + kDecWaves * i, A, -1);
      if (i + 1 < ni) compute_block(w + kDecWaves * (i + 1), B, -1);
    }
  }

  // Merge the four waves' states as in the 32-row kernel; each wave's
  // weighted accumulator goes to its own stage (16 fp32 rows).
  const float lrow = quad_sum(lsum);
  if (g == 0) {
    stat_m[w][q] = mrun;
    stat_l[w][q] = lrow;
  }
  __syncthreads();
  auto row_stats = [&](int row, float& M, float& Ltot) __attribute__((always_inline)) {
    M = -INFINITY;
#pragma unroll
    for (int x = 0; x < kDecWaves; ++x) M = fmaxf(M, stat_m[x][row]);
    Ltot = 0.f;
#pragma unroll
    for (int x = 0; x < kDecWaves; ++x)
      Ltot += stat_m[x][row] == -INFINITY ? 0.f : fast_exp2(stat_m[x][row] - M) * stat_l[x][row];
  };
  {
    float M, Ltot;
    row_stats(q, M, Ltot);
    const float f = mrun == -INFINITY ? 0.f : fast_exp2(mrun - M);
    // Row q of the slab, 16-byte chunk c stored at c ^ (q % OC).
    float* ob = (float*)stage + (size_t)q * D;
#pragma unroll
    for (int i = 0; i < DT; ++i) *(f32x4*)(ob + 4 * ((4 * i + g) ^ (q % OC))) = oacc[i] * f;
  }
  __syncthreads();
  {
    constexpr int SEG = D / 16;  // output elements per thread
    const int row = tid >> 4, d0 = (tid & 15) * SEG;
    if (row < rows) {
      float M, Ltot;
      row_stats(row, M, Ltot);
      const float inv = Ltot > 0.f ? 1.f / Ltot : 0.f;
      float acc[SEG];
#pragma unroll
      for (int e = 0; e < SEG; ++e) acc[e] = 0.f;
#pragma unroll
      for (int x = 0; x < kDecWaves; ++x) {
        const float* src = (const float*)(vst + x * STAGE) + (size_t)row * D;
#pragma unroll
        for (int e = 0; e < SEG; e += 4) {
          const f32x4 y = *(const f32x4*)(src + 4 * (((d0 + e) / 4) ^ (row % OC)));
          acc[e] += y[0];
          acc[e + 1] += y[1];
          acc[e + 2] += y[2];
          acc[e + 3] += y[3];
        }
      }
      const int rg = row / prm.s_q, rt = row - rg * prm.s_q;
      const int rh = hk * prm.group + rg;
      const float lse_row = Ltot > 0.f ? kLn2 * (M + __log2f(Ltot)) : -INFINITY;
      if (prm.n_splits == 1) {
        uint16_t* orow = prm.o + ((size_t)(b * prm.s_q + rt) * prm.heads + rh) * D + d0;
        if constexpr (SEG == 8) {
          u32x4 out;
#pragma unroll
          for (int u = 0; u < 4; ++u) out[u] = TT::pack2(acc[2 * u] * inv, acc[2 * u + 1] * inv);
          *(u32x4*)orow = out;
        } else {
          u32x2 out;
#pragma unroll
          for (int u = 0; u < 2; ++u) out[u] = TT::pack2(acc[2 * u] * inv, acc[2 * u + 1] * inv);
          *(u32x2*)orow = out;
        }
        if ((tid & 15) == 0) prm.lse[((size_t)b * prm.heads + rh) * prm.s_q + rt] = lse_row;
      } else {
        const size_t prow = ((size_t)(b * prm.heads + rh) * prm.s_q + rt) * prm.n_splits + split;
        float* po = prm.part_o + prow * D + d0;
#pragma unroll
        for (int e = 0; e < SEG; e += 4)
          *(f32x4*)(po + e) = f32x4{acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
        if ((tid & 15) == 0) prm.part_lse[prow] = lse_row;
      }
    }
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Combine the chunks of one output row (b, h, t), one wave per row:
// LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s over the chunks
// that hold keys (the others wrote nothing); chunks with LSE_s = -inf carry
// no weight, and a row with none left is O = 0, LSE = -inf. Lane s holds
// chunk s's LSE and weight (at most 64 chunks). Once the sequence length
// gives the number of active chunks, their LSEs and the partial outputs of
// the first 32 of them are loaded together, before any is used (slots past
// the active chunks re-read the last one and get weight 0), so the partial
// results cost one memory round trip.
template <typename TT, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           const int32_t* __restrict__ seqlens,
                                                           uint16_t* __restrict__ o,
                                                           float* __restrict__ lse, int n_rows,
                                                           int n_splits, int chunk, int max_len,
                                                           int heads, int s_q) {
  constexpr int PER = D / 64;
  constexpr int U = 32;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  const int t = row % s_q, bh = row / s_q;
  const int b = bh / heads, h = bh - b * heads;
  const int na = decode_active_chunks(min(max(seqlens[b], 0), max_len), chunk, n_splits);
  const float ls = lane < na ? part_lse[(size_t)row * n_splits + lane] : -INFINITY;
  const float* src = part_o + (size_t)row * n_splits * D + lane * PER;
  float val[U][PER];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < PER; ++e) val[u][e] = src[(size_t)min(u, na - 1) * D + e];
  const float m = wave_max(ls);
  const float wt = (ls == -INFINITY) ? 0.f : __expf(ls - m);
  const float wsum = wave_sum(wt);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < na; s0 += U) {
    if (s0 > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < PER; ++e)
          val[u][e] = src[(size_t)min(s0 + u, na - 1) * D + e];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float ws = s0 + u < na
                           ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                           __builtin_bit_cast(int, wt), s0 + u))
                           : 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = ws != 0.f ? fmaf(ws, val[u][e], acc[e]) : acc[e];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint16_t* dst = o + ((size_t)(b * s_q + t) * heads + h) * D + lane * PER;
  if constexpr (PER == 2) {
    *(uint32_t*)dst = TT::pack2(acc[0] * inv, acc[1] * inv);
  } else {
    *dst = (uint16_t)(TT::pack2(acc[0] * inv, 0.f) & 0xffffu);
  }
  if (lane == 0) lse[row] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

template <typename TT, int D>
hipError_t launch_typed(const DecodeArgs& a, const DecodePlan& plan) {
  DecParams p;
  p.q = (const uint16_t*)a.q;
  p.k = (const uint16_t*)a.k_cache;
  p.v = (const uint16_t*)a.v_cache;
  p.o = (uint16_t*)a.o;
  p.lse = a.lse;
  p.seqlens = a.cache_seqlens;
  p.part_o = plan.n_splits > 1 ? (float*)((char*)a.workspace + plan.part_o_off) : nullptr;
  p.part_lse = plan.n_splits > 1 ? (float*)((char*)a.workspace + plan.part_lse_off) : nullptr;
  p.batch = (int)a.B;
  p.s_q = (int)a.s_q;
  p.cap = (int)a.cap;
  p.max_len = (int)a.max_len;
  p.heads = (int)a.H;
  p.hkv = (int)a.H_kv;
  p.group = (int)(a.H / a.H_kv);
  p.n_splits = plan.n_splits;
  p.chunk = plan.chunk;
  p.c = fabsf(a.scale) * kLog2e;
  p.qsign = a.scale < 0.f ? 0x80008000u : 0u;
  const int64_t grid = a.B * a.H_kv * plan.n_splits;
  if (p.group * p.s_q <= 16)
    hipLaunchKernelGGL((decode16_kernel<TT, D>), dim3((unsigned)grid), dim3(kDecThreads), 0,
                       a.stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<TT, D>), dim3((unsigned)grid), dim3(kDecThreads), 0,
                       a.stream, p);
  if (plan.n_splits > 1) {
    const int n_rows = (int)(a.B * a.H * a.s_q);
    hipLaunchKernelGGL((decode_merge_kernel<TT, D>), dim3((unsigned)((n_rows + 3) / 4)), dim3(256),
                       0, a.stream, p.part_o, p.part_lse, p.seqlens, p.o, p.lse, n_rows,
                       plan.n_splits, p.chunk, p.max_len, p.heads, p.s_q);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan) {
  const bool bf = a.dtype == FA_BF16;
  if (a.D == 128) return bf ? launch_typed<Bf16, 128>(a, plan) : launch_typed<F16, 128>(a, plan);
  return bf ? launch_typed<Bf16, 64>(a, plan) : launch_typed<F16, 64>(a, plan);
}

}  // namespace fa
