// Host check of the planning arithmetic shared by the launcher and the kernels
// (csrc/ha_internal.hpp): chunk queue groups, equal key ranges of split chunk
// segments and the workspace capacity bounds.  Built and run by
// tests/test_host_planning.py; exits non-zero with a message on the first
// violated property.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "ha_internal.hpp"

static int fail(const char* what, long long a, long long b, long long c) {
  std::printf("FAIL %s (%lld, %lld, %lld)\n", what, a, b, c);
  return 1;
}

int main() {
  using namespace ha;
  // queue groups: every (head, pair) item lands in some group; sub-groups only
  // for fp32 with fewer heads than groups, balanced within a head
  for (int h = 1; h <= 70; ++h) {
    if (chunk_group_sub(false, h) != 1) return fail("bf16 sub-groups", h, 0, 0);
    const int g = chunk_group_sub(true, h);
    if (h < kXcdGroups ? g != kXcdGroups / h : g != 1) return fail("fp32 sub-groups", h, g, 0);
    for (int fp32 = 0; fp32 < 2; ++fp32) {
      const int gs = chunk_group_sub(fp32 != 0, h);
      for (int pairs = 0; pairs <= 80; ++pairs) {
        long long total = 0;
        int lo = 1 << 30, hi = -1;
        for (int x = 0; x < kXcdGroups; ++x) {
          const int n = chunk_group_items(h, gs, pairs, x);
          if (n < 0) return fail("negative group size", h, pairs, x);
          total += n;
          if (gs > 1 && x >= h * gs && n != 0) return fail("unused group holds items", h, pairs, x);
          if (gs > 1 && x < h * gs) {
            lo = n < lo ? n : lo;
            hi = n > hi ? n : hi;
          }
        }
        if (total != static_cast<long long>(h) * pairs) return fail("group sizes do not add up", h, pairs, total);
        if (gs > 1 && hi - lo > 1) return fail("sub-groups unbalanced", h, pairs, hi - lo);
      }
    }
  }
  // static first chunk items of a fused launch: in every queue group the ranks
  // of the chunk-first workgroups, then (spare) of the decode-first ones left
  // without a decode item, are distinct and are exactly 0 .. static_chunk_ranks - 1
  for (int grid = 1; grid <= 600; grid += (grid < 40 ? 1 : 13)) {
    const int half = (grid + 1) / 2;
    for (int n_dec = 0; n_dec <= grid; n_dec += (n_dec < 20 ? 1 : 7)) {
      const int ds = n_dec < grid - half ? n_dec : grid - half;
      for (int spare = 0; spare < 2; ++spare) {
        std::vector<std::vector<int>> seen(kXcdGroups, std::vector<int>(grid + 1, 0));
        for (int b = 0; b < grid; ++b) {
          int r = -1;
          if (b < half) r = b / kXcdGroups;
          else if (spare && b >= half + ds) r = spare_chunk_rank(b, half, ds);
          if (r < 0) continue;
          if (r > grid || seen[b % kXcdGroups][r]++) return fail("static chunk rank repeated", grid, n_dec, b);
        }
        for (int x = 0; x < kXcdGroups; ++x) {
          const int n = static_chunk_ranks(half, ds, grid, spare != 0, x);
          for (int r = 0; r <= grid; ++r)
            if (seen[x][r] != (r < n ? 1 : 0)) return fail("static chunk ranks not 0 .. first - 1", grid, n_dec, x);
        }
      }
    }
  }
  // equal key ranges: 64-aligned, cover the segment, the shortest such length
  for (int lk = 1; lk <= 20000; lk += 7) {
    for (int s = 2; s <= 40; ++s) {
      const int ck = chunk_range_keys(lk, s);
      const int need = (lk + s - 1) / s;
      if (ck % 64 != 0 || static_cast<long long>(ck) * s < lk || ck < need || ck - 64 >= need)
        return fail("range length", lk, s, ck);
    }
  }
  // decode full splits and tail pieces tile a segment exactly: full splits of
  // 2^sh keys, then pieces of 2^(sh - kTailLog2), the last one non-empty
  for (long long lk = 1; lk <= 300000; lk += (lk < 5000 ? 1 : 997)) {
    for (int sh = kSplitMinLog2; sh < kSplitMinLog2 + kSplitCandidates; ++sh) {
      long long full, tail;
      decode_pieces(lk, sh, full, tail);
      const long long n = (lk + (1LL << sh) - 1) >> sh;
      if (sh < kTailMinLog2) {
        if (full != n || tail != 0) return fail("no tail below the threshold", lk, sh, tail);
        continue;
      }
      const long long piece = 1LL << (sh - kTailLog2), covered = (full << sh) + tail * piece;
      if (full != n - 1 || tail < 1 || tail > (1LL << kTailLog2) || covered < lk || covered - piece >= lk)
        return fail("tail pieces", lk, sh, tail);
    }
  }
  // workspace bounds on random steps: query tiles of the chunk segments, decode
  // partial slots at the smallest split, 256-byte aligned arrays in order
  std::mt19937 rng(7);
  for (int trial = 0; trial < 20000; ++trial) {
    const int b = 1 + static_cast<int>(rng() % 300);
    std::vector<int> lq(b), lk(b);
    long long total_q = 0, tiles = 0, parts = 0;
    int max_k = 1;
    for (int i = 0; i < b; ++i) {
      const int kind = static_cast<int>(rng() % 3);
      lq[i] = kind == 0 ? 1 : kind == 1 ? 2 + static_cast<int>(rng() % 300) : static_cast<int>(rng() % 3000);
      lk[i] = lq[i] + static_cast<int>(rng() % 20000);
      total_q += lq[i];
      if (lq[i] >= 2) tiles += (lq[i] + kChunkRows - 1) / kChunkRows;
      if (lq[i] == 1) parts += (lk[i] + kSplitMin - 1) / kSplitMin;
      max_k = lk[i] > max_k ? lk[i] : max_k;
    }
    if (total_q == 0) continue;
    if (tiles > tiles_cap_for(b, static_cast<int>(total_q))) return fail("tiles_cap_for", b, total_q, tiles);
    const int pc = parts_cap_for(b, max_k);
    if (parts > pc && pc < kPartsMax) return fail("parts_cap_for", b, max_k, parts);
    const int hq = 1 + static_cast<int>(rng() % 64), d = (rng() & 1) ? 64 : 128;
    const WsLayout l = ws_layout(b, static_cast<int>(total_q), max_k, hq, d);
    const size_t offs[] = {l.tile_prefix, l.dec_prefix, l.part_prefix, l.seqlens, l.tail_prefix, l.partials,
                           l.chunk_partials, l.total};
    for (int i = 0; i < 8; ++i) {
      if (offs[i] % 256 != 0) return fail("workspace array alignment", b, i, static_cast<long long>(offs[i]));
      if (i > 0 && offs[i] < offs[i - 1]) return fail("workspace arrays out of order", b, i, 0);
    }
    if (l.tile_prefix < sizeof(PlanHeader)) return fail("header overlap", b, 0, 0);
    if (l.chunk_slots_cap != 0 && l.chunk_slots_cap < 2) return fail("chunk slots", b, l.chunk_slots_cap, 0);
    // the same step within a bounded scratch buffer: capacities only shrink,
    // arrays stay aligned and in order, and everything fits once the fixed
    // arrays do
    const size_t cap_bytes = static_cast<size_t>(1 + rng() % 64) << 20;
    const WsLayout c = ws_layout_within(b, static_cast<int>(total_q), max_k, hq, d, cap_bytes);
    if (c.partials != l.partials) return fail("capped layout moved the fixed arrays", b, 0, 0);
    if (c.parts_cap > l.parts_cap || c.chunk_slots_cap > l.chunk_slots_cap || c.parts_cap < 0)
      return fail("capped capacities grew", b, c.parts_cap, c.chunk_slots_cap);
    if (c.chunk_slots_cap != 0 && c.chunk_slots_cap < 2) return fail("capped chunk slots", b, c.chunk_slots_cap, 0);
    if (c.chunk_partials % 256 != 0 || c.total % 256 != 0 || c.chunk_partials < c.partials)
      return fail("capped layout alignment", b, 0, 0);
    const size_t part_bytes = sizeof(float) * static_cast<size_t>(hq) * c.part_stride;
    if (c.chunk_partials - c.partials < static_cast<size_t>(c.parts_cap) * part_bytes ||
        c.total - c.chunk_partials < static_cast<size_t>(c.chunk_slots_cap) * part_bytes * kChunkRows)
      return fail("capped arrays overlap", b, c.parts_cap, c.chunk_slots_cap);
    if (l.total <= cap_bytes && c.total != l.total) return fail("layout capped although it fits", b, 0, 0);
    if (l.partials + 512 <= cap_bytes && c.total > cap_bytes)
      return fail("capped layout too big", b, static_cast<long long>(c.total), static_cast<long long>(cap_bytes));
  }
  std::printf("host planning checks passed\n");
  return 0;
}
