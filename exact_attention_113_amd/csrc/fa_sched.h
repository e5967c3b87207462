// Work orders of the kernels' grids: which (sequence, head, tile) each
// workgroup takes, how many workgroups a launch has, and how the decode
// kernel cuts a cache into chunks. Host and device code share these
// functions, so the mapping the kernels run is the one the CPU-side
// coverage check enumerates (every row produced exactly once, every index
// inside its tensor). The orders a wave computes with one sequence per lane
// (`*_wave`) have a host form (`*_host`) that runs the same steps lane by
// lane; the check enumerates that.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Map a linear workgroup id to a logical one so that runs of consecutive
// logical ids land on one XCD. Workgroups are dealt to the 8 XCDs round
// robin by linear id; when the grid is a multiple of 8, logical id
// (x * total/8 + s) is given to the s-th workgroup of XCD x.
__host__ __device__ inline int xcd_logical_id(int lin, int total) {
  if ((total & 7) != 0) return lin;
  return (lin & 7) * (total >> 3) + (lin >> 3);
}

// Rows [s0, s0 + n) of a packed batch are sequence b: its offsets clamped
// into [0, total] and its length to seqlen (the longest sequence the grid
// was sized for), so malformed offsets cannot move an access out of bounds.
__host__ __device__ inline void seq_span(const int32_t* cu, int b, int total, int seqlen, int& s0,
                                         int& n) {
  const int a0 = cu[b], a1 = cu[b + 1];
  s0 = a0 < 0 ? 0 : (a0 > total ? total : a0);
  const int s1 = a1 < s0 ? s0 : (a1 > total ? total : a1);
  n = s1 - s0 < seqlen ? s1 - s0 : seqlen;
}

// ---- forward (bf16 / fp16) -------------------------------------------------

// Workgroup lin of the forward: query tile qt (counted from the last) of
// (sequence, head) pair p. Heavier causal query tiles come first (longest
// job first over the CUs; in packed batches round r takes each sequence's
// r-th tile from its end). The pairs are numbered head-major,
// p = h * batch + b; when they divide evenly over the 8 XCDs, each XCD keeps
// one contiguous range of p: the same heads of every sequence. With
// `pairs` (long dense grids, fwd_shape) each XCD takes its range two pairs
// at a time, all tiles of both (heaviest first, the two alternating), so
// fewer heads' K/V share its L2 and the heavy-light balance comes from the
// dynamic dispatch over the many rounds.
__host__ __device__ inline void fwd_tile_of(int lin, int n_qtiles, int bh_count, bool pairs,
                                            int& qt, int& p) {
  if (pairs && (bh_count & 15) == 0) {
    const int hpx = bh_count >> 3;
    const int xcd = lin & 7, slot = lin >> 3;
    const int j = slot / (2 * n_qtiles), within = slot - j * 2 * n_qtiles;
    qt = n_qtiles - 1 - within / 2;
    p = xcd * hpx + 2 * j + (within & 1);
  } else if ((bh_count & 7) == 0) {
    const int hpx = bh_count >> 3;
    const int xcd = lin & 7, slot = lin >> 3;
    qt = n_qtiles - 1 - slot / hpx;
    p = xcd * hpx + slot % hpx;
  } else {
    qt = n_qtiles - 1 - lin / bh_count;
    p = lin % bh_count;
  }
}

// A packed batch counts a sequence's tiles back from its own last one, so
// that the slots past the end of shorter sequences come last in the
// dispatch order; negative means no tile (the workgroup exits).
__host__ __device__ inline int fwd_seq_tile(int qt, int n_qtiles, int n, int bm, bool packed) {
  return packed ? qt - (n_qtiles - (n + bm - 1) / bm) : qt;
}

// Packed batches: a grid of only the batch's real tiles, heaviest first over
// the whole batch. Tile t of a sequence (rows t * bm ..) orders it: under a
// causal mask it sees t + 1 key tiles whatever its sequence, and with full
// attention only sequences of more than t tiles have a tile t, so the high
// indices belong to the longest sequences either way. Within one index the
// heads vary fastest, then the sequences in order. Workgroup lin takes slot
// s = lin >> 3 of XCD lin & 7, which owns heads (lin & 7) * H/8 .. + H/8 - 1
// of every sequence as in the dense order (a K/V head's query heads share
// its L2); slots past the batch's last tile exit at once. Measured on the
// 16-sequence prefill batch (256..4096 tokens, H32/8, D128): 928-931 ->
// 791-792 us causal and 1658-1663 -> 1414-1418 us with full attention
// against the grid of (sequence, head) x the longest sequence's tiles, whose
// empty workgroups each held a CU. The device form keeps one sequence's tile
// count and one tile index per lane, hence the limits.
constexpr int kLptMaxBatch = 64;
constexpr int kLptMaxTiles = 64;
inline bool fwd_packed_lpt_ok(int64_t batch, int64_t heads, int n_qtiles) {
  return heads % 8 == 0 && batch <= kLptMaxBatch && n_qtiles <= kLptMaxTiles;
}
// Slots for every tile: the tiles number sum_b ceil(n_b / bm), at most
// (total + batch (bm - 1)) / bm and batch * n_qtiles.
inline int64_t fwd_packed_lpt_grid(int64_t batch, int64_t total, int64_t heads, int bm,
                                   int n_qtiles) {
  const int64_t bound = (total + batch * (bm - 1)) / bm;
  const int64_t most = batch * (int64_t)n_qtiles;
  return heads * (bound < most ? bound : most);
}
// Tiles of sequence b: ceil(n_b / bm) with n_b as the kernels see it.
__host__ __device__ inline int packed_tiles(const int32_t* cu, int b, int total, int seqlen,
                                            int bm) {
  int s0, n;
  seq_span(cu, b, total, seqlen, s0, n);
  return (n + bm - 1) / bm;
}
// Slot s of an XCD with g8 heads: sequence b, head hl of the XCD's heads and
// tile t; false past the last tile. This host form runs the device form's
// steps over the 64 lanes one after another (lane j: sequence j's tile count,
// and the count c[j] of the batch's tiles with index >= j).
inline bool fwd_packed_lpt_host(const int32_t* cu, int batch, int total, int seqlen, int bm,
                                int n_qtiles, int g8, int s, int& b, int& hl, int& t) {
  int nt[64], c[64];
  for (int l = 0; l < 64; ++l) nt[l] = l < batch ? packed_tiles(cu, l, total, seqlen, bm) : 0;
  for (int l = 0; l < 64; ++l) {
    c[l] = 0;
    for (int j = 0; j < batch; ++j) c[l] += nt[j] - l > 0 ? nt[j] - l : 0;
  }
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l) m |= (uint64_t)(l < n_qtiles && g8 * c[l] > s) << l;
  if (m == 0) return false;
  t = __builtin_popcountll(m) - 1;
  const int i = s - g8 * (t + 1 < 64 ? c[t + 1] : 0);
  hl = i % g8;
  const int k = i / g8;
  uint64_t m2 = 0;
  for (int l = 0; l < 64; ++l) m2 |= (uint64_t)(l < batch && nt[l] > t) << l;
  uint64_t m3 = 0;
  for (int l = 0; l < 64; ++l) {
    const int rank = __builtin_popcountll(m2 & ((1ull << l) - 1));
    m3 |= (uint64_t)(((m2 >> l) & 1) && rank == k) << l;
  }
  b = m3 ? __builtin_ctzll(m3) : -1;
  return b >= 0;
}
// The same on the device, lane l of the calling wave holding lane l's
// values; every wave of a workgroup gets the same answer.
__device__ inline bool fwd_packed_lpt_wave(const int32_t* cu, int batch, int total, int seqlen,
                                           int bm, int n_qtiles, int g8, int s, int lane, int& b,
                                           int& hl, int& t) {
  const int nt = lane < batch ? packed_tiles(cu, lane, total, seqlen, bm) : 0;
  int c = 0;
  for (int j = 0; j < batch; ++j) {
    const int d = __builtin_amdgcn_readlane(nt, j) - lane;
    c += d > 0 ? d : 0;
  }
  const uint64_t m = __ballot(lane < n_qtiles && g8 * c > s);
  if (m == 0) return false;
  t = __popcll(m) - 1;
  const int i = s - g8 * (t + 1 < 64 ? __builtin_amdgcn_readlane(c, t + 1) : 0);
  hl = i % g8;
  const int k = i / g8;
  const uint64_t m2 = __ballot(lane < batch && nt > t);
  const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m2 >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m2, 0u));
  const uint64_t m3 = __ballot(((m2 >> lane) & 1ull) && rank == k);
  b = m3 ? __ffsll((unsigned long long)m3) - 1 : -1;
  return b >= 0;
}

// Largest grids (in 256-row workgroups) whose forward splits each row
// group's keys between two waves: causal attention up to one round of the
// CUs, full attention up to half of one (see the forward kernel). At head
// dim 64, grids of at most a quarter round split them four ways (64-row
// workgroups; measured B2 H8 N512 full 10.6 -> 9.0 us and B1 H32 N512
// causal 11.4 -> 9.5 us; at head dim 128, whose 128-key tiles double the
// bytes a workgroup loads before its first product, B1 H32 N512 causal
// went 15.4 -> 15.8 us, so it keeps two).
constexpr int64_t kMaxSplitCausal = 256;
constexpr int64_t kMaxSplitFull = 128;
constexpr int64_t kMaxSplit4 = 64;
// Dense grids of at least four workgroups per CU use the pairwise XCD order
// of fwd_tile_of (interleaved runs on two boxes: the B4 H16 N8192 D128
// training forward 1.0-2.0 % faster, B1 H32 N16384 causal 0.5-1.8 %; at two
// workgroups per CU, B1 H32 N4096, it was 1-4 % slower, the heavy-first
// pairing of tiles on a CU being worth more there).
constexpr int64_t kMinPairOrder = 1024;

struct FwdShape {
  int ks;        // 1: whole key ranges per wave; 2 or 4: waves per row group
  int bm;        // query rows per workgroup (256 / ks)
  int n_qtiles;  // query tiles per (sequence, head)
  int64_t grid;  // workgroups
  bool pairs;    // pairwise XCD order (dense batches only)
};

// Grid of the half-precision forward for bh_count (sequence, head) pairs of
// (at most) n rows and head dim d.
inline FwdShape fwd_shape(int64_t bh_count, int64_t n, bool causal, int d) {
  const int64_t tiles = ((n + 255) / 256) * bh_count;
  FwdShape s;
  s.ks = tiles > (causal ? kMaxSplitCausal : kMaxSplitFull) ? 1
         : (d == 64 && tiles <= kMaxSplit4)                 ? 4
                                                            : 2;
  s.bm = 256 / s.ks;
  s.n_qtiles = (int)((n + s.bm - 1) / s.bm);
  s.grid = (int64_t)s.n_qtiles * bh_count;
  s.pairs = s.grid >= kMinPairOrder && (bh_count & 15) == 0;
  return s;
}

// fp32 forward. Unsplit (ks = 1), four waves of 32 query rows each run over
// whole key ranges. Grids of at most kMaxSplitF32 such 128-row tiles split
// each row group's keys over ks waves: ks = 4 (one row group, 32 rows) at
// head dim 64, ks = 2 (two row groups, 64 rows) at 128, which keeps the
// double-buffered K/V tiles of 32 keys per split within the LDS. Every
// workgroup has four waves, one per SIMD: against eight-wave workgroups of
// twice the rows (two waves per SIMD) B1 H2 N256 D64 went 20.3 -> 14.1 us,
// D128 51.8 -> 32.1 us, B1 H8 N2048 causal D64 90.5 -> 74.4 us and D128
// 288 -> 178 us, bitwise the same results: the matrix work of a v_mfma
// f32 32x32x2 wave is not shared with a second wave, and the grid covers
// twice the CUs.
constexpr int64_t kMaxSplitF32 = 256;
__host__ __device__ constexpr int f32_row_groups(int ks) { return 4 / ks; }
__host__ __device__ constexpr int f32_split(int d) { return d == 64 ? 4 : 2; }

struct F32Shape {
  int ks;        // waves per row group
  int bm;        // query rows per workgroup (32 per row group)
  int n_qtiles;  // query tiles per (batch, head)
  int64_t grid;  // workgroups
};

inline F32Shape f32_shape(int64_t bh_count, int64_t n, int d) {
  F32Shape s;
  const int64_t tiles = ((n + 127) / 128) * bh_count;
  s.ks = tiles > kMaxSplitF32 ? 1 : f32_split(d);
  s.bm = 32 * f32_row_groups(s.ks);
  s.n_qtiles = (int)((n + s.bm - 1) / s.bm);
  s.grid = (int64_t)s.n_qtiles * bh_count;
  return s;
}

// fp32 forward: workgroup lin takes query tile qt (heaviest first) of the
// (batch, head) pair bh, each XCD a contiguous range of logical ids.
__host__ __device__ inline void f32_tile_of(int lin, int grid, int n_qtiles, int& qt, int& bh) {
  const int logical = xcd_logical_id(lin, grid);
  bh = logical / n_qtiles;
  qt = n_qtiles - 1 - logical % n_qtiles;
}

// ---- backward ---------------------------------------------------------------

// Workgroup blk of either backward kernel: unit (a (sequence, head) pair,
// numbered head-major, heads pinned to XCDs) and slot. Unit-major (the
// default): each XCD runs one unit's tiles after another, sharing that
// unit's operands in its L2. Round-major (small causal grids): round r takes
// slot r of every unit, which spreads heavy and light tiles evenly over the
// CUs.
__host__ __device__ inline void bwd_unit_slot(int blk, int grid, bool round_major, int units,
                                              int n_tiles, int& unit, int& slot) {
  if (round_major) {
    if ((units & 7) == 0) {
      const int per_xcd = units >> 3;
      const int s = blk >> 3;
      unit = (blk & 7) * per_xcd + s % per_xcd;
      slot = s / per_xcd;
    } else {
      unit = blk % units;
      slot = blk / units;
    }
  } else {
    const int logical = xcd_logical_id(blk, grid);
    unit = logical / n_tiles;
    slot = logical % n_tiles;
  }
}

// dQ: the query tile of a slot, or -1 past the end of a shorter sequence.
// Unit-major counts from the longest sequence's end, round-major from this
// sequence's own end.
__host__ __device__ inline int bwd_dq_tile(int slot, bool round_major, int n_tiles, int n, int bm) {
  const int qt = (round_major ? (n + bm - 1) / bm : n_tiles) - 1 - slot;
  return (qt < 0 || qt * bm >= n) ? -1 : qt;
}

// Packed backward grids in the unit-major order (each XCD works through
// the units of its heads one after another, sequences in order, a unit's
// tiles heaviest first) hold only the batch's real tiles: the workgroups
// that the grid sized by the longest sequence gives each shorter sequence's
// unit past its end, and that exit at once, are left out. The units are
// (sequence, head) with `heads` the K/V heads (dK/dV) or the query heads
// (dQ); XCD x owns heads x * heads/8 .. + heads/8 - 1. Slot s of an XCD
// gives its head j, the sequence b and r, the rank of the tile within the
// unit in the order above (dK/dV: key tile r; dQ: query tile n_b - 1 - r).
// The device form keeps one sequence per lane, hence the limit.
inline bool bwd_packed_compact_ok(int64_t batch, int64_t heads, bool round_major) {
  return !round_major && heads % 8 == 0 && batch <= kLptMaxBatch;
}
inline int64_t bwd_packed_compact_grid(int64_t batch, int64_t total, int64_t heads, int bt,
                                       int n_tiles) {
  const int64_t bound = (total + batch * (bt - 1)) / bt;
  const int64_t most = batch * (int64_t)n_tiles;
  return heads * (bound < most ? bound : most);
}
// Host form, the device form's steps over the lanes one after another
// (lane j: sequence j's tile count and the tiles of the sequences before it).
inline bool bwd_packed_compact_host(const int32_t* cu, int batch, int total, int seqlen, int bt,
                                    int g8, int s, int& j, int& b, int& r) {
  int nt[64], pre[64], sum = 0;
  for (int l = 0; l < 64; ++l) {
    nt[l] = l < batch ? packed_tiles(cu, l, total, seqlen, bt) : 0;
    pre[l] = sum;
    sum += nt[l];
  }
  if (sum == 0) return false;
  j = s / sum;
  if (j >= g8) return false;
  const int rr = s - j * sum;
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l) m |= (uint64_t)(l < batch && pre[l] <= rr && rr < pre[l] + nt[l]) << l;
  if (m == 0) return false;
  b = __builtin_ctzll(m);
  r = rr - pre[b];
  return true;
}
__device__ inline bool bwd_packed_compact_wave(const int32_t* cu, int batch, int total, int seqlen,
                                               int bt, int g8, int s, int lane, int& j, int& b,
                                               int& r) {
  const int nt = lane < batch ? packed_tiles(cu, lane, total, seqlen, bt) : 0;
  int pre = 0, sum = 0;
  for (int l = 0; l < batch; ++l) {
    const int x = __builtin_amdgcn_readlane(nt, l);
    pre += l < lane ? x : 0;
    sum += x;
  }
  if (sum == 0) return false;
  j = s / sum;
  if (j >= g8) return false;
  const int rr = s - j * sum;
  const uint64_t m = __ballot(lane < batch && pre <= rr && rr < pre + nt);
  if (m == 0) return false;
  b = __ffsll((unsigned long long)m) - 1;
  r = rr - __builtin_amdgcn_readlane(pre, b);
  return true;
}

constexpr int kBwdKeyTile = 128;    // keys per dK/dV workgroup
constexpr int kBwdQueryTile = 256;  // query rows per dQ workgroup
// Causal dQ grids of at most two workgroups per CU run round-major
// (measured at B1 H32 N4096 D128, 512 workgroups: backward 569 against
// 626-634 us unit-major; at 2048 workgroups and in the packed GQA batch
// unit-major was 1.5 % and 5 % faster). Full attention's tiles all cost
// the same, so there the order could only change the L2 sharing.
constexpr int64_t kMaxRoundMajorDq = 512;
// Causal dK/dV grids of at most four workgroups per CU run round-major.
constexpr int64_t kMaxRoundMajorDkdv = 1024;

struct BwdShape {
  int n_ktiles, n_qtiles;      // key tiles (dK/dV) and query tiles (dQ) per unit
  int64_t grid_dkdv, grid_dq;  // workgroups
  bool rm_dkdv, rm_dq;         // round-major work orders
};

// Grids of the two backward kernels for `batch` sequences of (at most) n
// rows, h query heads over hkv K/V heads.
inline BwdShape bwd_shape(int64_t batch, int64_t h, int64_t hkv, int64_t n, bool causal) {
  BwdShape s;
  s.n_ktiles = (int)((n + kBwdKeyTile - 1) / kBwdKeyTile);
  s.n_qtiles = (int)((n + kBwdQueryTile - 1) / kBwdQueryTile);
  s.grid_dkdv = (int64_t)s.n_ktiles * batch * hkv;
  s.grid_dq = (int64_t)s.n_qtiles * batch * h;
  s.rm_dkdv = causal && s.grid_dkdv <= kMaxRoundMajorDkdv;
  s.rm_dq = causal && s.grid_dq <= kMaxRoundMajorDq;
  return s;
}

// ---- decode ------------------------------------------------------------------

// Workgroup blk of the decode kernel: sequence b, K/V head hk, chunk split.
// Heads vary fastest: the workgroups dispatched together read the pieces of
// the same cache rows (each row holds every K/V head of one token).
__host__ __device__ inline void decode_unit(int blk, int n_splits, int hkv, int& b, int& hk,
                                            int& split) {
  hk = blk % hkv;
  const int rest = blk / hkv;
  split = rest % n_splits;
  b = rest / n_splits;
}

// Chunks of a sequence with L visible cache keys (L already clamped to
// [0, max_len]) that hold keys: chunks 0 .. result - 1 write a partial
// result; the rest do nothing, and the merge weighs only the first ones. A
// sequence with no key still has chunk 0 (it writes O = 0, LSE = -inf).
__host__ __device__ inline int decode_active_chunks(int L, int chunk, int n_splits) {
  if (L <= 0) return 1;
  const int n = (L + chunk - 1) / chunk;
  return n < n_splits ? n : n_splits;
}

// Batches of at most kDecodeOrderMaxBatch sequences number the chunks that
// hold keys first: workgroup blk takes K/V head blk % H_kv (heads fastest, as
// above) of active chunk c = blk / H_kv, the chunks of sequence 0 first, then
// sequence 1's, and so on; the workgroups past the last active chunk exit
// after all real work has been dispatched instead of holding CUs among it.
// The device form keeps one sequence per lane.
constexpr int kDecodeOrderMaxBatch = 64;
__host__ __device__ inline int decode_active_of(const int32_t* seqlens, int b, int max_len,
                                                int chunk, int n_splits) {
  const int L0 = seqlens[b];
  const int L = L0 < 0 ? 0 : (L0 > max_len ? max_len : L0);
  return decode_active_chunks(L, chunk, n_splits);
}
inline bool decode_active_unit_host(const int32_t* seqlens, int batch, int max_len, int chunk,
                                    int n_splits, int c, int& b, int& split) {
  int pre = 0;
  for (int l = 0; l < batch; ++l) {
    const int na = decode_active_of(seqlens, l, max_len, chunk, n_splits);
    if (c < pre + na) {
      b = l;
      split = c - pre;
      return true;
    }
    pre += na;
  }
  return false;
}
__device__ inline bool decode_active_unit_wave(const int32_t* seqlens, int batch, int max_len,
                                               int chunk, int n_splits, int c, int lane, int& b,
                                               int& split) {
  const int na = lane < batch ? decode_active_of(seqlens, lane, max_len, chunk, n_splits) : 0;
  int pre = 0;
  for (int l = 0; l < batch; ++l) {
    const int x = __builtin_amdgcn_readlane(na, l);
    pre += l < lane ? x : 0;
  }
  const uint64_t m = __ballot(lane < batch && pre <= c && c < pre + na);
  if (m == 0) return false;
  b = __ffsll((unsigned long long)m) - 1;
  split = c - __builtin_amdgcn_readlane(pre, b);
  return true;
}

// Workgroups the chunk plan aims for, and the most chunks per row (one
// lane of the merge kernel's wave each).
#ifndef FA_DECODE_TARGET_WGS
#define FA_DECODE_TARGET_WGS 4096
#endif
constexpr int64_t kDecodeTargetWgs = FA_DECODE_TARGET_WGS;
constexpr int64_t kMaxSplits = 64;

// How the cache is cut into chunks (one workgroup per sequence, K/V head and
// chunk) and where the per-chunk partial results go in the workspace.
struct DecodePlan {
  int n_splits, chunk;
  size_t part_o_off, part_o_bytes;      // fp32 [B, H, s_q, n_splits, D]
  size_t part_lse_off, part_lse_bytes;  // fp32 [B, H, s_q, n_splits]
  size_t total;                         // 0 when the cache is one chunk
};

inline bool decode_plan(int64_t B, int64_t s_q, int64_t H, int64_t H_kv, int64_t max_len,
                        int64_t D, DecodePlan* plan) {
  if (B < 1 || s_q < 1 || H < 1 || H_kv < 1 || max_len < 0 || D < 1) return false;
  // Enough workgroups to fill the chip a few times over, chunks of at least
  // 128 keys (one block per wave), at most kMaxSplits chunks per row.
  const int64_t units = B * H_kv;
  const int64_t want = (kDecodeTargetWgs + units - 1) / units;
  const int64_t most = max_len > 0 ? (max_len + 127) / 128 : 1;
  int64_t n = want < most ? want : most;
  if (n > kMaxSplits) n = kMaxSplits;
  if (n < 1) n = 1;
  int64_t chunk = max_len > 0 ? (max_len + n - 1) / n : 128;
  chunk = (chunk + 127) / 128 * 128;
  n = max_len > 0 ? (max_len + chunk - 1) / chunk : 1;
  plan->n_splits = (int)n;
  plan->chunk = (int)chunk;
  auto pad = [](size_t x) { return (x + 255) / 256 * 256; };
  if (n > 1) {
    const size_t rows = (size_t)B * H * s_q;
    plan->part_o_off = 0;
    plan->part_o_bytes = pad(rows * n * D * 4);
    plan->part_lse_off = plan->part_o_bytes;
    plan->part_lse_bytes = pad(rows * n * 4);
    plan->total = plan->part_o_bytes + plan->part_lse_bytes;
  } else {
    plan->part_o_off = plan->part_o_bytes = plan->part_lse_off = plan->part_lse_bytes = 0;
    plan->total = 0;
  }
  return true;
}

}  // namespace fa
