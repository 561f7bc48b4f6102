// plan.cpp - tile table, staged tree schedule and workspace layout (host only).
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstdio>

namespace adasum {

namespace {

constexpr int64_t kMaxElements = int64_t(1) << 40;  // per buffer; keeps every size in 64-bit range

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace

bool validate_shape(int K, const int64_t* offsets, int nseg, int dtype, int schedule, std::string* err) {
  char buf[160];
  if (schedule != int(Schedule::Tree) && schedule != int(Schedule::Chain)) {
    snprintf(buf, sizeof buf, "unknown schedule %d (0 = tree, 1 = chain)", schedule);
    *err = buf;
    return false;
  }
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
  // tile count (times the weighted sum's parts per tile) must fit a launch
  // grid and the kernels' 32-bit tile indices
  if ((offsets[nseg] / kMinTile + nseg + 1) * kWsumSplitMax > int64_t(INT32_MAX)) {
    *err = "too many tiles for this shape";
    return false;
  }
  // the tree walk launches one workgroup per (block, segment) of a stage,
  // and a stage has fewer blocks than K
  if ((int64_t)K * nseg > int64_t(INT32_MAX)) {
    snprintf(buf, sizeof buf, "K * nseg = %lld exceeds 2^31 - 1", (long long)K * nseg);
    *err = buf;
    return false;
  }
  return true;
}

namespace {

struct Elem {
  int lo, hi;   // operand range of the stage
  bool merged;  // false: a bare operand carried through the stage
};

// A merge in stage-wide operand positions (a stage can hold any number of
// operands; only block-relative positions fit the 8-bit fields of Merge).
struct StageMerge {
  int llo, lhi, rhi, node;
};

// Merges of one stage of the tree schedule: up to `levels` levels of
// pairing (v0,v1), (v2,v3), ... over `cur`, the odd last element carried.
void tree_stage(std::vector<Elem>& cur, std::vector<StageMerge>& merges, int& node, int levels) {
  for (int level = 0; level < levels && cur.size() > 1; ++level) {
    std::vector<Elem> next;
    for (size_t j = 0; 2 * j + 1 < cur.size(); ++j) {
      const Elem& l = cur[2 * j];
      const Elem& r = cur[2 * j + 1];
      merges.push_back(StageMerge{l.lo, l.hi, r.hi, node++});
      next.push_back(Elem{l.lo, r.hi, true});
    }
    if (cur.size() % 2 == 1) next.push_back(cur.back());
    cur = next;
  }
}

// One stage of the chain schedule: the accumulated vector (first element)
// meets the following operands one at a time, all of them in this stage.
void chain_stage(std::vector<Elem>& cur, std::vector<StageMerge>& merges, int& node) {
  Elem acc = cur[0];
  for (size_t j = 1; j < cur.size(); ++j) {
    merges.push_back(StageMerge{acc.lo, acc.hi, cur[j].hi, node++});
    acc = Elem{acc.lo, cur[j].hi, true};
  }
  cur.assign(1, acc);
}

}  // namespace

Plan build_plan(int K, const int64_t* offsets, int nseg, DType dtype, Schedule schedule) {
  Plan p;
  p.K = K;
  p.dtype = dtype;
  p.schedule = schedule;
  p.nseg = nseg;
  p.offsets.assign(offsets, offsets + nseg + 1);
  p.N = offsets[nseg];

  // ---- tiles: a workload too small to fill the GPU with kTile tiles is cut
  // finer, so that every launch has thousands of workgroups
  p.tile_rows = std::min<int64_t>(kTile, std::max<int64_t>(kMinTile, align_up(p.N / kTargetTiles, 1024)));
  p.seg_tile.resize(nseg + 1);
  for (int s = 0; s < nseg; ++s) {
    p.seg_tile[s] = (int32_t)p.tiles.size();
    const int64_t lo = offsets[s], hi = offsets[s + 1];
    int64_t a = lo;
    while (a < hi) {
      // the first tile absorbs the unaligned head; later tiles start aligned
      const int64_t body_start = align_up(a, kGroup);
      const int64_t end = std::min(hi, body_start + p.tile_rows);
      p.tiles.push_back(Tile{a, (int32_t)(end - a), (int32_t)s, p.seg_tile[s], 0});
      a = end;
    }
    for (size_t t = (size_t)p.seg_tile[s]; t < p.tiles.size(); ++t) p.tiles[t].seg_t1 = (int32_t)p.tiles.size();
  }
  p.seg_tile[nseg] = (int32_t)p.tiles.size();
  const size_t ntiles = p.tiles.size();
  for (int s = 0; s < nseg; ++s)
    if (p.seg_tile[s + 1] - p.seg_tile[s] >= kGroupMinTiles) p.tile_groups = true;

  // ---- blocks, stage by stage.  An operand of a stage above the first is
  // an fp64 slot (the result of a lower block) or an input gradient that the
  // stage reads where it is, in its own dtype.
  std::vector<Ref> operands(K);
  std::vector<char> is_leaf(K, 1);   // per operand of the current stage
  for (int k = 0; k < K; ++k) operands[k] = Ref{Ref::Input, k};
  int node = 0;
  int next_leaf = K;                 // chain: first input not yet in any stage
  if (schedule == Schedule::Chain) {
    next_leaf = std::min(K, first_stage_ops(dtype, K, schedule));
    operands.resize(next_leaf);
    is_leaf.resize(next_leaf);
  }
  bool first = true;
  while (first || operands.size() > 1) {
    Stage st;
    std::vector<Elem> cur;
    for (int i = 0; i < (int)operands.size(); ++i) cur.push_back(Elem{i, i + 1, false});
    std::vector<StageMerge> stage_merges;
    // the first stage reads only inputs; later ones read fp64 slots (and inputs carried up)
    const int ops = first ? first_stage_ops(dtype, K, schedule) : kMaxOps32;
    if (schedule == Schedule::Tree)
      tree_stage(cur, stage_merges, node, ops == 64 ? 6 : ops == 32 ? 5 : 4);
    else
      chain_stage(cur, stage_merges, node);
    const bool last = cur.size() == 1 && next_leaf == K;
    std::vector<Ref> next_operands;
    std::vector<char> next_is_leaf;
    for (const Elem& e : cur) {
      if (!e.merged && !(last && operands.size() == 1)) {
        next_operands.push_back(operands[e.lo]);  // carried up unchanged
        next_is_leaf.push_back(is_leaf[e.lo]);
        continue;
      }
      // a block: the operands under e (K = 1: the single input, no merge)
      Block b;
      b.operands.assign(operands.begin() + e.lo, operands.begin() + e.hi);
      b.dst = last ? Ref{Ref::Out, 0} : Ref{Ref::Slot, p.nslots++};
      BlockDesc d{};
      d.nb = e.hi - e.lo;
      d.nbt = d.nb <= 2 ? 2 : d.nb <= 4 ? 4 : d.nb <= 8 ? 8 : d.nb <= 16 ? 16 : d.nb <= 32 ? 32 : 64;
      d.merge0 = (int)p.merges.size();
      for (const StageMerge& m : stage_merges) {
        if (m.llo >= e.lo && m.rhi <= e.hi) {
          p.merges.push_back(Merge{(int8_t)(m.llo - e.lo), (int8_t)(m.lhi - e.lo), (int8_t)(m.rhi - e.lo), 0, m.node});
        }
      }
      d.nmerges = (int)p.merges.size() - d.merge0;
      d.wrow = p.nblocks++;
      for (int k = e.lo; k < e.hi; ++k)
        if (is_leaf[k]) d.leafmask |= uint64_t(1) << (k - e.lo);
      d.root = last ? 1 : 0;
      // fp64 sums on the fp64 matrix cores (fp32 inputs; stages that read
      // fp64 slots, any inputs among them widened exactly): a bound on the
      // rounding of a lane's running sum and of the reductions behind it.
      // 16-bit inputs of the first stage: each 32-row chunk rounded to fp32
      // once by the matrix cores, with a margin for the fp64 accumulation.
      bool reads_slot = false;
      for (int k = e.lo; k < e.hi; ++k) reads_slot |= operands[k].kind == Ref::Slot;
      d.gram_err = (dtype == DType::F32 || reads_slot) ? std::ldexp(1.0, -44)
                                                        : std::ldexp(1.0, -24) * (1.0 + std::ldexp(1.0, -10));
      b.desc = (int)p.descs.size();
      p.descs.push_back(d);
      st.blocks.push_back(b);
      next_operands.push_back(b.dst);
      next_is_leaf.push_back(0);
    }
    // chain: the next stage is the accumulated vector plus up to 15 more inputs
    if (schedule == Schedule::Chain && !last) {
      const int take = std::min(K - next_leaf, kMaxOps32 - 1);
      for (int k = next_leaf; k < next_leaf + take; ++k) {
        next_operands.push_back(Ref{Ref::Input, k});
        next_is_leaf.push_back(1);
      }
      next_leaf += take;
    }
    // Gram partials of this stage: one region per block, reused by later stages
    size_t off = 0;
    for (const Block& b : st.blocks) {
      p.descs[b.desc].poff = (int64_t)off;
      off += (size_t)gram_entries(p.descs[b.desc].nbt) * ntiles;
    }
    p.partial_doubles = std::max(p.partial_doubles, off);
    p.stages.push_back(st);
    operands = next_operands;
    is_leaf = next_is_leaf;
    first = false;
    if (last) break;
  }

  // ---- small one-stage combines: walk and weighted sum in one launch
  if (p.stages.size() == 1 && p.stages[0].blocks.size() == 1 && p.descs[0].nbt <= kArgOps && p.N <= kFusedMaxRows &&
      !p.tiles.empty()) {
    p.fused = true;
    const int64_t ne = gram_entries(p.descs[0].nbt);
    for (int s = 0; s < nseg; ++s) {
      const int64_t nt = p.seg_tile[s + 1] - p.seg_tile[s];
      if (nt < 1 || nt * ne > kFusedMaxReads) p.fused = false;
    }
  }

  // ---- workspace layout
  size_t off = 0;
  p.ws_slots = off;
  off = align256(off + (size_t)p.nslots * (size_t)p.N * sizeof(double));
  p.ws_partials = off;
  off = align256(off + p.partial_doubles * sizeof(double));
  p.ws_weights = off;
  off = align256(off + (size_t)p.nblocks * nseg * kMaxOps * sizeof(double));
  p.ws_weights_lo = off;
  off = align256(off + (size_t)p.nblocks * nseg * kMaxOps * sizeof(double));
  p.ws_leafnorm = off;
  off = align256(off + (size_t)p.nblocks * nseg * sizeof(double));
  p.ws_coeffs = off;
  off = align256(off + p.table_bytes(2));
  p.ws_stats = off;
  off = align256(off + p.table_bytes(3));
  p.ws_flags = off;
  off = align256(off + (size_t)p.nblocks * nseg * sizeof(uint32_t));
  p.ws_plo = off;  // low parts of exactly recomputed Gram partials (double-double), laid out as the partials
  off = align256(off + p.partial_doubles * sizeof(double));
  p.ws_total = off;
  return p;
}

}  // namespace adasum
