// CPU check of the kernels' work orders (test infrastructure).
//
// For each launch it enumerates every workgroup of the grid through the same
// host/device functions the kernels and launchers use (fa_sched.h), and
// checks that every query row, key row or cache row of every (sequence, head)
// is produced exactly once, that rows outside every sequence are not touched,
// and that every row index used for Q, K, V, O, the statistics and the
// decode workspace stays inside its tensor. Prints one line per case and
// exits non-zero when any check fails.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "fa_internal.h"

namespace {

int g_fail = 0, g_cases = 0;

#define CHECK(cond, ...)                         \
  do {                                           \
    if (!(cond)) {                               \
      ++g_fail;                                  \
      std::printf("FAIL %s: ", name.c_str());    \
      std::printf(__VA_ARGS__);                  \
      std::printf("\n");                         \
      return;                                    \
    }                                            \
  } while (0)

// A batch of sequences: dense (all of length n, rows [B, H, n]) or packed
// (offsets into [total, H] token-major rows; total may exceed the last
// offset, leaving tokens outside every sequence).
struct Batch {
  bool packed;
  std::vector<int> lens;
  std::vector<int32_t> cu;
  int total;
  int seqlen;  // dense n, or the longest sequence
};

Batch dense(int B, int n) {
  Batch x{false, std::vector<int>(B, n), {}, B * n, n};
  return x;
}

Batch packed(const std::vector<int>& lens, int tail = 0) {
  Batch x{true, lens, {0}, 0, 0};
  for (int n : lens) {
    x.cu.push_back(x.cu.back() + n);
    if (n > x.seqlen) x.seqlen = n;
  }
  x.total = x.cu.back() + tail;
  if (x.seqlen == 0) x.seqlen = 1;
  return x;
}

// Row of (sequence b, head h, position i) in a tensor of `heads` heads, and
// the sequence's first row and length as the kernels see them.
void span(const Batch& x, int b, int& s0, int& n) {
  if (x.packed) {
    fa::seq_span(x.cu.data(), b, x.total, x.seqlen, s0, n);
  } else {
    s0 = 0;
    n = x.seqlen;
  }
}
int64_t row_of(const Batch& x, int heads, int b, int h, int s0, int i) {
  return x.packed ? (int64_t)(s0 + i) * heads + h : ((int64_t)b * heads + h) * x.seqlen + i;
}
int64_t rows_of(const Batch& x, int heads) {
  return x.packed ? (int64_t)x.total * heads : (int64_t)x.lens.size() * heads * x.seqlen;
}
// Statistics (LSE, delta): dense [B, H, N], packed [H, total].
int64_t stat_of(const Batch& x, int heads, int b, int h, int s0, int i) {
  return x.packed ? (int64_t)h * x.total + s0 + i : ((int64_t)b * heads + h) * x.seqlen + i;
}

// Every row that belongs to a sequence was counted once, every other row
// not at all.
bool exactly_once(const Batch& x, int heads, const std::vector<int>& cover, std::string& why) {
  std::vector<char> inside(cover.size(), 0);
  for (int b = 0; b < (int)x.lens.size(); ++b) {
    int s0, n;
    span(x, b, s0, n);
    for (int h = 0; h < heads; ++h)
      for (int i = 0; i < n; ++i) inside[row_of(x, heads, b, h, s0, i)] = 1;
  }
  for (size_t r = 0; r < cover.size(); ++r)
    if (cover[r] != (inside[r] ? 1 : 0)) {
      why = "row " + std::to_string(r) + " written " + std::to_string(cover[r]) + " times" +
            (inside[r] ? "" : " (outside every sequence)");
      return false;
    }
  return true;
}

// Half-precision forward (dense or packed, grouped heads).
void check_forward_d(const std::string& name, const Batch& x, int H, int Hkv, bool causal, int d) {
  ++g_cases;
  const int batch = (int)x.lens.size();
  const int bh_count = batch * H;
  const fa::FwdShape sh = fa::fwd_shape(bh_count, x.seqlen, causal, d);
  CHECK(sh.bm * sh.ks == 256 && sh.n_qtiles * sh.bm >= x.seqlen, "shape");
  CHECK(sh.grid < 0x7fffffff, "grid %lld", (long long)sh.grid);
  const int group = H / Hkv;
  std::vector<int> cover(rows_of(x, H), 0);
  const int64_t n_stat = rows_of(x, H);
  // Packed batches within the limits: only real tiles, heaviest first.
  const bool lpt = x.packed && fa::fwd_packed_lpt_ok(batch, H, sh.n_qtiles);
  const int64_t grid = lpt ? fa::fwd_packed_lpt_grid(batch, x.total, H, sh.bm, sh.n_qtiles)
                           : sh.grid;
  CHECK(grid <= sh.grid, "packed grid %lld above %lld", (long long)grid, (long long)sh.grid);
  std::vector<int> last_t(8, 1 << 30);
  std::vector<char> ended(8, 0);
  for (int lin = 0; lin < (int)grid; ++lin) {
    int qt, h, b;
    if (lpt) {
      const int g8 = H / 8, xcd = lin & 7;
      int hl, t;
      if (!fa::fwd_packed_lpt_host(x.cu.data(), batch, x.total, x.seqlen, sh.bm, sh.n_qtiles, g8,
                                   lin >> 3, b, hl, t)) {
        ended[xcd] = 1;
        continue;
      }
      // Heaviest first: on each XCD the tile index never rises, and no
      // slot after an empty one holds a tile.
      CHECK(!ended[xcd] && t <= last_t[xcd], "lin %d: tile %d after %d", lin, t, last_t[xcd]);
      last_t[xcd] = t;
      CHECK(b >= 0 && b < batch && hl >= 0 && hl < g8 && t >= 0 && t < sh.n_qtiles,
            "lin %d -> b %d hl %d t %d", lin, b, hl, t);
      h = xcd * g8 + hl;
      qt = t;
    } else {
      int p;
      fa::fwd_tile_of(lin, sh.n_qtiles, bh_count, sh.pairs && !x.packed, qt, p);
      CHECK(p >= 0 && p < bh_count && qt >= 0 && qt < sh.n_qtiles, "lin %d -> qt %d p %d", lin,
            qt, p);
      h = p / batch;
      b = p - h * batch;
    }
    const int hk = h / group;
    int s0, n;
    span(x, b, s0, n);
    if (!lpt) {
      qt = fa::fwd_seq_tile(qt, sh.n_qtiles, n, sh.bm, x.packed);
      if (qt < 0) continue;
    }
    const int q0 = qt * sh.bm;
    CHECK(q0 < n, "lin %d: tile %d starts past the sequence (%d rows)", lin, qt, n);
    for (int i = q0; i < q0 + sh.bm && i < n; ++i) {
      const int64_t r = row_of(x, H, b, h, s0, i);
      CHECK(r >= 0 && r < (int64_t)cover.size(), "Q/O row %lld out of bounds", (long long)r);
      const int64_t st = stat_of(x, H, b, h, s0, i);
      CHECK(st >= 0 && st < n_stat, "LSE index %lld out of bounds", (long long)st);
      ++cover[r];
    }
    // K and V rows the workgroup reads: 0 .. min(n, q0 + bm + diag) - 1,
    // each clamped to the sequence's last row.
    const int kv_end = causal ? std::min(n, q0 + sh.bm) : n;
    for (int k : {0, kv_end - 1}) {
      const int64_t r = row_of(x, Hkv, b, hk, s0, std::max(std::min(k, n - 1), 0));
      CHECK(r >= 0 && r < rows_of(x, Hkv), "K/V row %lld out of bounds", (long long)r);
    }
  }
  std::string why;
  CHECK(exactly_once(x, H, cover, why), "%s", why.c_str());
  std::printf("ok %s D%d: %lld workgroups, key split %d%s\n", name.c_str(), d, (long long)grid,
              sh.ks,
              lpt ? ", whole-batch order" : sh.pairs && !x.packed ? ", pairwise order" : "");
}

// Both head dims: their grid rules differ for the shortest grids.
void check_forward(const std::string& name, const Batch& x, int H, int Hkv, bool causal) {
  for (int d : {64, 128}) check_forward_d(name, x, H, Hkv, causal, d);
}

// Malformed offsets (decreasing, or past the end of the packed tensors):
// the results are meaningless, but every index must stay in bounds.
void check_malformed(const std::string& name, const std::vector<int32_t>& cu, int total, int H,
                     int Hkv, bool causal) {
  ++g_cases;
  Batch x{true, std::vector<int>(cu.size() - 1, 0), cu, total, total};
  const int batch = (int)x.lens.size();
  for (int d : {64, 128}) {
  const fa::FwdShape sh = fa::fwd_shape(batch * H, x.seqlen, causal, d);
  const bool lpt = fa::fwd_packed_lpt_ok(batch, H, sh.n_qtiles);
  const int64_t grid =
      lpt ? fa::fwd_packed_lpt_grid(batch, x.total, H, sh.bm, sh.n_qtiles) : sh.grid;
  for (int lin = 0; lin < (int)grid; ++lin) {
    int qt, h, b;
    if (lpt) {
      int hl;
      if (!fa::fwd_packed_lpt_host(x.cu.data(), batch, x.total, x.seqlen, sh.bm, sh.n_qtiles,
                                   H / 8, lin >> 3, b, hl, qt))
        continue;
      CHECK(b >= 0 && b < batch && hl >= 0 && hl < H / 8, "malformed: b %d hl %d", b, hl);
      h = (lin & 7) * (H / 8) + hl;
    } else {
      int p;
      fa::fwd_tile_of(lin, sh.n_qtiles, batch * H, false, qt, p);
      h = p / batch;
      b = p - h * batch;
    }
    int s0, n;
    span(x, b, s0, n);
    if (!lpt) {
      qt = fa::fwd_seq_tile(qt, sh.n_qtiles, n, sh.bm, true);
      if (qt < 0) continue;
    }
    for (int i = qt * sh.bm; i < qt * sh.bm + sh.bm && i < n; ++i) {
      CHECK(row_of(x, H, b, h, s0, i) < rows_of(x, H), "forward row out of bounds");
      CHECK(row_of(x, Hkv, b, h / (H / Hkv), s0, i) < rows_of(x, Hkv), "K/V row out of bounds");
      CHECK(stat_of(x, H, b, h, s0, i) < rows_of(x, H), "LSE out of bounds");
    }
  }
  }
  const fa::BwdShape bs = fa::bwd_shape(batch, H, Hkv, x.seqlen, causal);
  for (int blk = 0; blk < (int)bs.grid_dkdv; ++blk) {
    int unit, kt;
    fa::bwd_unit_slot(blk, (int)bs.grid_dkdv, bs.rm_dkdv, batch * Hkv, bs.n_ktiles, unit, kt);
    const int hk = unit / batch, b = unit - hk * batch;
    int s0, n;
    span(x, b, s0, n);
    for (int k = kt * fa::kBwdKeyTile; k < (kt + 1) * fa::kBwdKeyTile && k < n; ++k)
      CHECK(row_of(x, Hkv, b, hk, s0, k) < rows_of(x, Hkv), "dK/dV row out of bounds");
  }
  for (int blk = 0; blk < (int)bs.grid_dq; ++blk) {
    int unit, slot;
    fa::bwd_unit_slot(blk, (int)bs.grid_dq, bs.rm_dq, batch * H, bs.n_qtiles, unit, slot);
    const int h = unit / batch, b = unit - h * batch;
    int s0, n;
    span(x, b, s0, n);
    const int qt = fa::bwd_dq_tile(slot, bs.rm_dq, bs.n_qtiles, n, fa::kBwdQueryTile);
    if (qt < 0) continue;
    for (int i = qt * fa::kBwdQueryTile; i < (qt + 1) * fa::kBwdQueryTile && i < n; ++i)
      CHECK(row_of(x, H, b, h, s0, i) < rows_of(x, H), "dQ row out of bounds");
  }
  std::printf("ok %s: every index in bounds\n", name.c_str());
}

// fp32 forward (dense only).
void check_forward_f32(const std::string& name, int B, int H, int N, int D) {
  ++g_cases;
  const Batch x = dense(B, N);
  const fa::F32Shape sh = fa::f32_shape((int64_t)B * H, N, D);
  const int BM = sh.bm, n_qtiles = sh.n_qtiles, grid = (int)sh.grid;
  CHECK(BM == 32 * fa::f32_row_groups(sh.ks), "rows per workgroup %d, ks %d", BM, sh.ks);
  std::vector<int> cover(rows_of(x, H), 0);
  for (int lin = 0; lin < grid; ++lin) {
    int qt, bh;
    fa::f32_tile_of(lin, grid, n_qtiles, qt, bh);
    CHECK(bh >= 0 && bh < B * H && qt >= 0 && qt < n_qtiles, "lin %d", lin);
    for (int i = qt * BM; i < qt * BM + BM && i < N; ++i) ++cover[(int64_t)bh * N + i];
  }
  std::string why;
  CHECK(exactly_once(x, H, cover, why), "%s", why.c_str());
  std::printf("ok %s: %d workgroups, ks %d\n", name.c_str(), grid, sh.ks);
}

// Backward: dK/dV over key tiles of each (sequence, K/V head), dQ over query
// tiles of each (sequence, query head).
int units_q_of(int batch, int H) { return batch * H; }

void check_backward(const std::string& name, const Batch& x, int H, int Hkv, bool causal) {
  ++g_cases;
  const int batch = (int)x.lens.size();
  const int group = H / Hkv;
  const fa::BwdShape sh = fa::bwd_shape(batch, H, Hkv, x.seqlen, causal);
  std::vector<int> cover_kv(rows_of(x, Hkv), 0), cover_q(rows_of(x, H), 0);
  const int64_t n_stat = rows_of(x, H);
  const int units_kv = batch * Hkv;
  // Packed grids within the limits hold only real tiles: each XCD's list of
  // (unit, tile) must be the full grid's list with the empty slots left out.
  const bool c1 = x.packed && fa::bwd_packed_compact_ok(batch, Hkv, sh.rm_dkdv);
  const bool c2 = x.packed && fa::bwd_packed_compact_ok(batch, H, sh.rm_dq);
  std::vector<std::vector<std::pair<int, int>>> full_kv(8), compact_kv(8), full_q(8), compact_q(8);
  if (c1)
    for (int blk = 0; blk < (int)sh.grid_dkdv; ++blk) {
      int unit, kt, s0, n;
      fa::bwd_unit_slot(blk, (int)sh.grid_dkdv, false, units_kv, sh.n_ktiles, unit, kt);
      span(x, unit % batch, s0, n);
      if (kt * fa::kBwdKeyTile < n) full_kv[blk & 7].push_back({unit, kt});
    }
  if (c2)
    for (int blk = 0; blk < (int)sh.grid_dq; ++blk) {
      int unit, slot, s0, n;
      fa::bwd_unit_slot(blk, (int)sh.grid_dq, false, units_q_of(batch, H), sh.n_qtiles, unit, slot);
      span(x, unit % batch, s0, n);
      const int qt = fa::bwd_dq_tile(slot, false, sh.n_qtiles, n, fa::kBwdQueryTile);
      if (qt >= 0) full_q[blk & 7].push_back({unit, qt});
    }
  const int64_t grid1 =
      c1 ? fa::bwd_packed_compact_grid(batch, x.total, Hkv, fa::kBwdKeyTile, sh.n_ktiles)
         : sh.grid_dkdv;
  CHECK(grid1 <= sh.grid_dkdv, "compact dK/dV grid above the full one");
  for (int blk = 0; blk < (int)grid1; ++blk) {
    int unit, kt;
    if (c1) {
      const int g8 = Hkv / 8;
      int j, bb;
      if (!fa::bwd_packed_compact_host(x.cu.data(), batch, x.total, x.seqlen, fa::kBwdKeyTile, g8,
                                       blk >> 3, j, bb, kt))
        continue;
      unit = ((blk & 7) * g8 + j) * batch + bb;
      compact_kv[blk & 7].push_back({unit, kt});
    } else {
      fa::bwd_unit_slot(blk, (int)sh.grid_dkdv, sh.rm_dkdv, units_kv, sh.n_ktiles, unit, kt);
    }
    CHECK(unit >= 0 && unit < units_kv && kt >= 0 && kt < sh.n_ktiles, "dK/dV blk %d", blk);
    const int hk = unit / batch, b = unit - hk * batch;
    int s0, n;
    span(x, b, s0, n);
    const int k0 = kt * fa::kBwdKeyTile;
    if (k0 >= n) continue;
    for (int k = k0; k < k0 + fa::kBwdKeyTile && k < n; ++k) {
      const int64_t r = row_of(x, Hkv, b, hk, s0, k);
      CHECK(r >= 0 && r < (int64_t)cover_kv.size(), "K/V row %lld out of bounds", (long long)r);
      ++cover_kv[r];
    }
    // Query rows of every head of the group that the tile iterates over.
    for (int h = hk * group; h < (hk + 1) * group; ++h)
      for (int i : {causal ? k0 : 0, n - 1}) {
        CHECK(row_of(x, H, b, h, s0, i) < rows_of(x, H) && stat_of(x, H, b, h, s0, i) < n_stat,
              "dK/dV: query row out of bounds");
      }
  }
  const int units_q = batch * H;
  const int64_t grid2 =
      c2 ? fa::bwd_packed_compact_grid(batch, x.total, H, fa::kBwdQueryTile, sh.n_qtiles)
         : sh.grid_dq;
  CHECK(grid2 <= sh.grid_dq, "compact dQ grid above the full one");
  for (int blk = 0; blk < (int)grid2; ++blk) {
    int unit, h, b, s0, n, qt;
    if (c2) {
      const int g8 = H / 8;
      int j, r;
      if (!fa::bwd_packed_compact_host(x.cu.data(), batch, x.total, x.seqlen, fa::kBwdQueryTile,
                                       g8, blk >> 3, j, b, r))
        continue;
      unit = ((blk & 7) * g8 + j) * batch + b;
      CHECK(unit >= 0 && unit < units_q, "dQ blk %d", blk);
      h = unit / batch;
      span(x, b, s0, n);
      qt = (n + fa::kBwdQueryTile - 1) / fa::kBwdQueryTile - 1 - r;
      CHECK(qt >= 0, "dQ blk %d: rank %d past the sequence", blk, r);
      compact_q[blk & 7].push_back({unit, qt});
    } else {
      int slot;
      fa::bwd_unit_slot(blk, (int)sh.grid_dq, sh.rm_dq, units_q, sh.n_qtiles, unit, slot);
      CHECK(unit >= 0 && unit < units_q && slot >= 0 && slot < sh.n_qtiles, "dQ blk %d", blk);
      h = unit / batch;
      b = unit - h * batch;
      span(x, b, s0, n);
      qt = fa::bwd_dq_tile(slot, sh.rm_dq, sh.n_qtiles, n, fa::kBwdQueryTile);
    }
    if (qt < 0) continue;
    const int q0 = qt * fa::kBwdQueryTile;
    CHECK(q0 < n, "dQ blk %d: tile %d starts past the sequence (%d rows)", blk, qt, n);
    for (int i = q0; i < q0 + fa::kBwdQueryTile && i < n; ++i) {
      const int64_t r = row_of(x, H, b, h, s0, i);
      CHECK(r >= 0 && r < (int64_t)cover_q.size(), "dQ row %lld out of bounds", (long long)r);
      CHECK(stat_of(x, H, b, h, s0, i) < n_stat, "dQ statistic out of bounds");
      ++cover_q[r];
    }
  }
  for (int xcd = 0; xcd < 8; ++xcd) {
    CHECK(!c1 || compact_kv[xcd] == full_kv[xcd], "dK/dV XCD %d: compact order differs", xcd);
    CHECK(!c2 || compact_q[xcd] == full_q[xcd], "dQ XCD %d: compact order differs", xcd);
  }
  std::string why;
  CHECK(exactly_once(x, Hkv, cover_kv, why), "dK/dV: %s", why.c_str());
  CHECK(exactly_once(x, H, cover_q, why), "dQ: %s", why.c_str());
  std::printf("ok %s: dK/dV %lld workgroups (%s), dQ %lld (%s)\n", name.c_str(),
              (long long)grid1,
              c1 ? "real tiles only" : sh.rm_dkdv ? "round-major" : "unit-major",
              (long long)grid2, c2 ? "real tiles only" : sh.rm_dq ? "round-major" : "unit-major");
}

// Decode: chunks of the cache of each (sequence, K/V head).
void check_decode(const std::string& name, int s_q, int H, int Hkv, int cap, int max_len,
                  const std::vector<int>& lens) {
  ++g_cases;
  const int B = (int)lens.size();
  fa::DecodePlan plan;
  CHECK(fa::decode_plan(B, s_q, H, Hkv, max_len, 128, &plan), "no plan");
  CHECK(plan.n_splits >= 1 && plan.n_splits <= fa::kMaxSplits, "%d chunks", plan.n_splits);
  CHECK(plan.chunk % 128 == 0 && (int64_t)plan.n_splits * plan.chunk >= max_len,
        "chunks %d x %d do not cover %d keys", plan.n_splits, plan.chunk, max_len);
  CHECK(max_len == 0 || (int64_t)(plan.n_splits - 1) * plan.chunk < max_len, "an empty chunk");
  const int grid = B * Hkv * plan.n_splits;
  const int group = H / Hkv;
  std::vector<int> cover((size_t)B * Hkv * cap, 0);
  std::vector<int> written((size_t)B * Hkv * plan.n_splits, 0);
  // Batches within the limit number the active chunks first (heads fastest);
  // no workgroup after the first that exits has work.
  const bool ordered = B <= fa::kDecodeOrderMaxBatch;
  bool exited = false;
  for (int blk = 0; blk < grid; ++blk) {
    int b, hk, split;
    if (ordered) {
      hk = blk % Hkv;
      if (!fa::decode_active_unit_host(lens.data(), B, max_len, plan.chunk, plan.n_splits,
                                       blk / Hkv, b, split)) {
        exited = true;
        continue;
      }
      CHECK(!exited, "blk %d has work after an idle workgroup", blk);
    } else {
      fa::decode_unit(blk, plan.n_splits, Hkv, b, hk, split);
    }
    CHECK(b >= 0 && b < B && hk >= 0 && hk < Hkv && split >= 0 && split < plan.n_splits,
          "blk %d", blk);
    const int L = std::min(std::max(lens[b], 0), max_len);
    const int k_lo = split * plan.chunk, k_hi = std::min(L, k_lo + plan.chunk);
    // Chunks past the active ones return at once; they must hold no key.
    const int na = fa::decode_active_chunks(L, plan.chunk, plan.n_splits);
    CHECK(na >= 1 && na <= plan.n_splits, "%d active chunks", na);
    if (split >= na) {
      CHECK(k_hi <= k_lo, "skipped chunk %d of sequence %d holds keys", split, b);
      continue;
    }
    if (plan.n_splits > 1) ++written[((size_t)b * Hkv + hk) * plan.n_splits + split];
    for (int k = k_lo; k < k_hi; ++k) {
      CHECK(k < cap, "key %d past the capacity %d", k, cap);
      ++cover[((size_t)b * Hkv + hk) * cap + k];
    }
    if (plan.n_splits > 1)
      for (int h = hk * group; h < (hk + 1) * group; ++h)
        for (int t = 0; t < s_q; ++t) {
          const size_t prow = ((size_t)(b * H + h) * s_q + t) * plan.n_splits + split;
          CHECK((prow + 1) * 128 * 4 <= plan.part_o_bytes && (prow + 1) * 4 <= plan.part_lse_bytes,
                "partial row %zu outside the workspace", prow);
        }
  }
  for (int b = 0; b < B; ++b) {
    const int L = std::min(std::max(lens[b], 0), max_len);
    // The merge weighs chunks [0, na) of each row: each is written once.
    const int na = fa::decode_active_chunks(L, plan.chunk, plan.n_splits);
    if (plan.n_splits > 1)
      for (int hk = 0; hk < Hkv; ++hk)
        for (int sp = 0; sp < plan.n_splits; ++sp) {
          const int c = written[((size_t)b * Hkv + hk) * plan.n_splits + sp];
          CHECK(c == (sp < na ? 1 : 0), "sequence %d head %d chunk %d written %d times", b, hk,
                sp, c);
        }
    for (int hk = 0; hk < Hkv; ++hk)
      for (int k = 0; k < cap; ++k) {
        const int c = cover[((size_t)b * Hkv + hk) * cap + k];
        CHECK(c == (k < L ? 1 : 0), "sequence %d head %d key %d read %d times", b, hk, k, c);
      }
  }
  std::printf("ok %s: %d workgroups, %d chunks of %d keys\n", name.c_str(), grid, plan.n_splits,
              plan.chunk);
}

}  // namespace

int main() {
  // Dense forward: the named workloads, ragged lengths, the key-split grid
  // thresholds (causal 256 / full 128 256-row tiles), grids whose (batch,
  // head) count is not a multiple of 8.
  for (bool causal : {true, false}) {
    const std::string c = causal ? " causal" : " full";
    for (int n : {512, 1024, 2048, 4096, 8192, 16384})
      check_forward("fwd B1 H32 N" + std::to_string(n) + c, dense(1, n), 32, 32, causal);
    check_forward("fwd B2 H8 N512" + c, dense(2, 512), 8, 8, causal);
    check_forward("fwd B4 H16 N8192" + c, dense(4, 8192), 16, 16, causal);
    for (int n : {1, 2, 7, 31, 33, 63, 65, 127, 129, 200, 1000})
      check_forward("fwd B2 H3 N" + std::to_string(n) + c, dense(2, n), 3, 3, causal);
    check_forward("fwd B1 H48 N2048" + c, dense(1, 2048), 48, 48, causal);
    check_forward("fwd B1 H33 N2048" + c, dense(1, 2048), 33, 33, causal);
    check_forward("fwd B3 H32 N1024" + c, dense(3, 1024), 32, 32, causal);
    check_forward("fwd B1 H32 N1536" + c, dense(1, 1536), 32, 32, causal);
    check_forward("fwd B8 H16 N1000" + c, dense(8, 1000), 16, 16, causal);
    check_forward("fwd B4096 H32 N128" + c, dense(4096, 128), 32, 32, causal);
    check_forward("fwd B1 H2 N131072" + c, dense(1, 131072), 2, 2, causal);
    check_forward("fwd B2 H32 N4000" + c, dense(2, 4000), 32, 32, causal);  // pairwise, ragged
  }
  // Packed batches: empty, one-token and ragged sequences, grouped heads,
  // tokens after the last sequence, the packed prefill workload's lengths.
  const std::vector<int> edge = {1, 7, 0, 65, 300, 129, 256};
  const std::vector<int> prefill = {3984, 256, 1201, 4096, 2500, 777, 3001, 1024,
                                    2048, 300,  3999, 1500, 640,  2900, 3300, 1111};
  for (bool causal : {true, false})
    for (int hkv : {4, 2, 1}) {
      const std::string c = std::string(causal ? " causal" : " full") + " H4/" + std::to_string(hkv);
      check_forward("fwd packed edge" + c, packed(edge), 4, hkv, causal);
      check_forward("fwd packed edge + tail" + c, packed(edge, 37), 4, hkv, causal);
      check_backward("bwd packed edge" + c, packed(edge), 4, hkv, causal);
      check_backward("bwd packed edge + tail" + c, packed(edge, 37), 4, hkv, causal);
    }
  check_forward("fwd packed prefill H32/8", packed(prefill), 32, 8, true);
  check_backward("bwd packed prefill H32/8", packed(prefill), 32, 8, true);
  check_forward("fwd packed empty first sequence", packed({0, 5}), 4, 4, true);
  check_backward("bwd packed empty first sequence", packed({0, 5}), 4, 4, true);
  check_forward("fwd packed 40 short", packed(std::vector<int>(40, 3)), 8, 2, true);
  // The whole-batch order (heads a multiple of 8, at most 64 sequences and 64
  // tiles): the edge lengths, with tokens after the last sequence, 64 and 65
  // sequences (the second keeps the per-sequence order), a 64-tile sequence.
  for (bool causal : {true, false})
    for (int hkv : {8, 2, 1}) {
      const std::string c = std::string(causal ? " causal" : " full") + " H8/" + std::to_string(hkv);
      check_forward("fwd packed edge" + c, packed(edge), 8, hkv, causal);
      check_forward("fwd packed edge + tail" + c, packed(edge, 37), 8, hkv, causal);
      check_backward("bwd packed edge" + c, packed(edge), 8, hkv, causal);
      check_backward("bwd packed edge + tail" + c, packed(edge, 37), 8, hkv, causal);
    }
  // Backward grids of only real tiles (unit-major grids, K/V or query heads
  // a multiple of 8): the prefill lengths with H16/8 and H8/8, 64 and 65
  // sequences.
  for (bool causal : {true, false}) {
    const std::string c = causal ? " causal" : " full";
    check_backward("bwd packed prefill H16/8" + c, packed(prefill), 16, 8, causal);
    check_backward("bwd packed prefill + tail H8/8" + c, packed(prefill, 300), 8, 8, causal);
    std::vector<int> many;
    for (int i = 0; i < 65; ++i) many.push_back((i * 613) % 900 + (i % 9 == 0 ? 0 : 2));
    check_backward("bwd packed 65 sequences H8/8" + c, packed(many), 8, 8, causal);
    many.pop_back();
    check_backward("bwd packed 64 sequences H8/8" + c, packed(many), 8, 8, causal);
  }
  {
    std::vector<int> many;
    for (int i = 0; i < 65; ++i) many.push_back((i * 977) % 1500 + (i % 7 == 0 ? 0 : 1));
    check_forward("fwd packed 65 sequences H16/4", packed(many), 16, 4, true);
    many.pop_back();
    check_forward("fwd packed 64 sequences H16/4", packed(many), 16, 4, true);
    check_forward("fwd packed 64-tile sequence H8/8", packed({16384, 3, 1000}), 8, 8, true);
    check_forward("fwd packed 65-tile sequence H8/8", packed({16385, 3, 1000}), 8, 8, false);
  }
  // Malformed offsets: decreasing, negative, past the end.
  for (bool causal : {true, false}) {
    check_malformed("malformed offsets A", {0, 5, 3, 100}, 20, 4, 2, causal);
    check_malformed("malformed offsets B", {-7, 300, 250, 999, 1000}, 600, 4, 4, causal);
    check_malformed("malformed offsets C", {10, 2, 2000}, 512, 8, 1, causal);
    check_malformed("malformed offsets D", {0, 900, 100, 100, 5000, 700}, 1000, 16, 4, causal);
  }
  // fp32 forward.
  for (int d : {64, 128}) {
    const std::string dd = " D" + std::to_string(d);
    check_forward_f32("fwd f32 B1 H2 N256" + dd, 1, 2, 256, d);
    check_forward_f32("fwd f32 B2 H3 N1000" + dd, 2, 3, 1000, d);
    check_forward_f32("fwd f32 B2 H4 N77" + dd, 2, 4, 77, d);
    check_forward_f32("fwd f32 B1 H16 N4096" + dd, 1, 16, 4096, d);
    check_forward_f32("fwd f32 B3 H5 N2049" + dd, 3, 5, 2049, d);
  }
  // Dense backward: the training shape, the round-major thresholds (dQ 512,
  // dK/dV 1024 workgroups), unit counts not a multiple of 8, ragged lengths.
  for (bool causal : {true, false}) {
    const std::string c = causal ? " causal" : " full";
    check_backward("bwd B4 H16 N8192" + c, dense(4, 8192), 16, 16, causal);
    check_backward("bwd B1 H32 N4096" + c, dense(1, 4096), 32, 32, causal);
    check_backward("bwd B1 H32 N4352" + c, dense(1, 4352), 32, 32, causal);
    check_backward("bwd B4 H32 N1100" + c, dense(4, 1100), 32, 32, causal);
    check_backward("bwd B1 H2 N1100" + c, dense(1, 1100), 2, 2, causal);
    for (int n : {1, 7, 33, 64, 65, 127, 129, 300})
      check_backward("bwd B2 H2 N" + std::to_string(n) + c, dense(2, n), 2, 2, causal);
    check_backward("bwd B3 H5 N777" + c, dense(3, 777), 5, 5, causal);
  }
  // Decode: the decode batch's cache lengths, edge lengths (empty, one key,
  // beyond the bound, negative), grouped heads and several new tokens.
  const std::vector<int> caches = {1024, 16384, 5000, 9000, 1500, 12000, 7777, 3000,
                                   16000, 2048, 4100, 8191, 10000, 6000, 15000, 2500};
  check_decode("decode batch H32/8", 1, 32, 8, 16384, 16384, caches);
  for (int s_q : {1, 4})
    for (int hkv : {8, 2, 1}) {
      const std::string c = " s_q " + std::to_string(s_q) + " H8/" + std::to_string(hkv);
      check_decode("decode edge" + c, s_q, 8, hkv, 700, 700, {0, 1, 3, 333, 700});
      check_decode("decode clamped" + c, s_q, 8, hkv, 700, 500, {-5, 700, 499, 501, 0});
    }
  check_decode("decode short caches", 1, 64, 32, 100, 100, {1, 50, 100, 7});
  check_decode("decode empty bound", 1, 4, 4, 64, 0, {0, 3});
  {
    // 64 sequences take the active-first order, 65 the plain one.
    std::vector<int> many;
    for (int i = 0; i < 65; ++i) many.push_back((i * 331) % 3000 - (i % 11 == 0 ? 50 : 0));
    check_decode("decode 65 sequences", 1, 8, 2, 3000, 3000, many);
    many.pop_back();
    check_decode("decode 64 sequences", 2, 8, 2, 3000, 2900, many);
  }
  std::printf("%d cases, %d failed\n", g_cases, g_fail);
  return g_fail ? 1 : 0;
}
