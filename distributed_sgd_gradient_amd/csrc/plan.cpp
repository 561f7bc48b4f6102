// plan.cpp - tile table, tree schedule and workspace layout (host only).
#include "plan.h"

#include <algorithm>
#include <cstdio>

namespace adasum {

namespace {

constexpr int64_t kMaxElements = int64_t(1) << 40;  // per buffer; keeps every size in 64-bit range

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace

bool validate_shape(int K, const int64_t* offsets, int nseg, int dtype, std::string* err) {
  char buf[160];
  if (K < 1) {
    snprintf(buf, sizeof buf, "K must be >= 1 (got %d)", K);
    *err = buf;
    return false;
  }
  if (nseg < 0) {
    snprintf(buf, sizeof buf, "nseg must be >= 0 (got %d)", nseg);
    *err = buf;
    return false;
  }
  if (dtype != int(DType::F32) && dtype != int(DType::F16) && dtype != int(DType::BF16)) {
    snprintf(buf, sizeof buf, "unknown dtype %d (0 = f32, 1 = f16, 2 = bf16)", dtype);
    *err = buf;
    return false;
  }
  if (offsets == nullptr) {
    *err = "seg_offsets is NULL";
    return false;
  }
  if (offsets[0] != 0) {
    snprintf(buf, sizeof buf, "seg_offsets[0] must be 0 (got %lld)", (long long)offsets[0]);
    *err = buf;
    return false;
  }
  for (int s = 0; s < nseg; ++s) {
    if (offsets[s + 1] < offsets[s]) {
      snprintf(buf, sizeof buf, "seg_offsets must be non-decreasing (offsets[%d] = %lld > offsets[%d] = %lld)",
               s, (long long)offsets[s], s + 1, (long long)offsets[s + 1]);
      *err = buf;
      return false;
    }
  }
  if (offsets[nseg] > kMaxElements) {
    snprintf(buf, sizeof buf, "N = %lld exceeds the supported maximum 2^40 elements",
             (long long)offsets[nseg]);
    *err = buf;
    return false;
  }
  // tile count must fit int32 (every kernel indexes tiles with 32-bit ints)
  if (offsets[nseg] / kTile + nseg + 1 > int64_t(INT32_MAX)) {
    *err = "too many tiles for this shape";
    return false;
  }
  return true;
}

Plan build_plan(int K, const int64_t* offsets, int nseg, DType dtype) {
  Plan p;
  p.K = K;
  p.dtype = dtype;
  p.nseg = nseg;
  p.offsets.assign(offsets, offsets + nseg + 1);
  p.N = offsets[nseg];

  // ---- tiles
  p.seg_tile.resize(nseg + 1);
  for (int s = 0; s < nseg; ++s) {
    p.seg_tile[s] = (int32_t)p.tiles.size();
    const int64_t lo = offsets[s], hi = offsets[s + 1];
    int64_t a = lo;
    while (a < hi) {
      // the first tile absorbs the unaligned head; later tiles start aligned
      const int64_t body_start = align_up(a, kGroup);
      const int64_t end = std::min(hi, body_start + kTile);
      p.tiles.push_back(Tile{a, (int32_t)(end - a), (int32_t)s});
      a = end;
    }
  }
  p.seg_tile[nseg] = (int32_t)p.tiles.size();

  // ---- tree schedule
  std::vector<Ref> cur(K);
  for (int k = 0; k < K; ++k) cur[k] = Ref{Ref::Input, k};
  int node = 0;
  bool first = true;
  while (cur.size() > 1) {
    Level lv;
    const int npairs = (int)cur.size() / 2;
    const bool odd = cur.size() % 2 == 1;
    lv.final_level = (cur.size() == 2);
    for (int j = 0; j < npairs; ++j) {
      Pair pr;
      pr.left = cur[2 * j];
      pr.right = cur[2 * j + 1];
      pr.node = node++;
      if (lv.final_level) {
        pr.dst = Ref{Ref::Out, 0};
      } else if (first) {
        pr.dst = Ref{Ref::Slot, j};
      } else {
        pr.dst = pr.left;  // in place: each element is read, then written, by one thread
      }
      lv.pairs.push_back(pr);
    }
    std::vector<Ref> next;
    for (const Pair& pr : lv.pairs) next.push_back(pr.dst);
    if (odd) {
      Ref carried = cur.back();
      if (carried.kind == Ref::Input) {
        // an input carried past level 1 is widened once into an fp32 slot so
        // that every operand above level 1 is fp32
        p.carry_slot = npairs;
        carried = Ref{Ref::Slot, npairs};
      }
      next.push_back(carried);
    }
    if (first) {
      p.nslots = lv.final_level ? 0 : npairs + (odd ? 1 : 0);
      for (int j = 0; j < npairs; ++j) lv.dot_pairs.push_back(j);
    }
    // combine jobs: siblings (2m, 2m+1) of this level form pair m of the next
    // level, so the job computing both emits that pair's statistics
    if (lv.final_level) {
      lv.jobs.push_back(Job{{0, -1}, -1});
    } else {
      for (int m = 0; 2 * m + 1 < npairs; ++m) lv.jobs.push_back(Job{{2 * m, 2 * m + 1}, m});
      if (npairs % 2 == 1) lv.jobs.push_back(Job{{npairs - 1, -1}, -1});
    }
    p.max_pairs = std::max(p.max_pairs, npairs);
    p.levels.push_back(lv);
    cur = next;
    first = false;
  }
  // pairs of level l >= 2 whose statistics no sibling job emitted need a
  // triple-dot pass over their stored operands
  for (size_t l = 1; l < p.levels.size(); ++l) {
    std::vector<char> emitted(p.levels[l].pairs.size(), 0);
    for (const Job& jb : p.levels[l - 1].jobs)
      if (jb.emit >= 0) emitted[jb.emit] = 1;
    for (size_t j = 0; j < emitted.size(); ++j)
      if (!emitted[j]) p.levels[l].dot_pairs.push_back((int)j);
  }

  // ---- workspace layout
  size_t off = 0;
  p.ws_slots = off;
  off = align256(off + (size_t)p.nslots * (size_t)p.N * sizeof(float));
  p.ws_partials = off;
  off = align256(off + p.partials_bytes());
  p.ws_coeffs = off;
  off = align256(off + p.table_bytes(2));
  p.ws_stats = off;
  off = align256(off + p.table_bytes(3));
  p.ws_total = off;
  return p;
}

}  // namespace adasum
