// Prints execution plans as JSON lines for tests/test_plan_host.py: with no
// argument, K = 1..70 and a few larger K, both schedules, fp32, fp16 and bf16
// inputs, over two fixed segments; with --stdin, one plan per input line
// "K dtype schedule nseg off_1 .. off_nseg".  Built with g++ on the host together
// with the library's plan.cpp (pure C++, no HIP).
#include <cstdio>
#include <string>
#include <vector>

#include "plan.h"

using namespace adasum;

// One plan as a JSON line.
static void dump(const Plan& p, int dt, int sched, int K) {
  printf("{\"dtype\": %d, \"schedule\": %d, \"K\": %d, \"nslots\": %d, \"tile_rows\": %lld, \"stages\": [", dt,
         sched, K, p.nslots, (long long)p.tile_rows);
  for (size_t s = 0; s < p.stages.size(); ++s) {
    const Stage& st = p.stages[s];
    printf("%s{\"blocks\": [", s ? "," : "");
    for (size_t b = 0; b < st.blocks.size(); ++b) {
      const Block& bk = st.blocks[b];
      const BlockDesc& d = p.descs[bk.desc];
      printf("%s{\"ops\": [", b ? "," : "");
      for (size_t k = 0; k < bk.operands.size(); ++k)
        printf("%s[%d,%d]", k ? "," : "", (int)bk.operands[k].kind, bk.operands[k].idx);
      printf("], \"dst\": [%d,%d], \"desc\": %d, \"nb\": %d, \"nbt\": %d, \"leafmask\": %llu, \"root\": %d, "
             "\"poff\": %lld, \"merges\": [", (int)bk.dst.kind, bk.dst.idx, bk.desc, d.nb, d.nbt,
             (unsigned long long)d.leafmask, (int)d.root, (long long)d.poff);
      for (int m = 0; m < d.nmerges; ++m) {
        const Merge& mg = p.merges[d.merge0 + m];
        printf("%s[%d,%d,%d,%d]", m ? "," : "", mg.llo, mg.lhi, mg.rhi, mg.node);
      }
      printf("]}");
    }
    printf("]}");
  }
  printf("], \"tiles\": [");
  for (size_t t = 0; t < p.tiles.size(); ++t)
    printf("%s[%lld,%d,%d,%d,%d]", t ? "," : "", (long long)p.tiles[t].start, p.tiles[t].len, p.tiles[t].seg,
           p.tiles[t].seg_t0, p.tiles[t].seg_t1);
  printf("], \"seg_tile\": [");
  for (size_t s = 0; s < p.seg_tile.size(); ++s) printf("%s%d", s ? "," : "", p.seg_tile[s]);
  printf("], \"gram_err\": [");
  for (size_t b = 0; b < p.descs.size(); ++b) printf("%s%.17g", b ? "," : "", p.descs[b].gram_err);
  printf("], \"fused\": %d, \"tile_groups\": %d, \"partial_doubles\": %zu, \"ws\": [%zu,%zu,%zu,%zu,%zu,%zu,%zu,%zu,%zu,%zu], \"nblocks\": %d}\n",
         (int)p.fused, (int)p.tile_groups,
         p.partial_doubles, p.ws_slots, p.ws_partials, p.ws_weights, p.ws_weights_lo, p.ws_leafnorm, p.ws_coeffs,
         p.ws_stats, p.ws_flags, p.ws_plo, p.ws_total, p.nblocks);
}

int main(int argc, char** argv) {
  if (argc > 1 && std::string(argv[1]) == "--stdin") {
    // lines: K dtype schedule nseg off_1 .. off_nseg   (off_0 = 0)
    int K, dt, sched, nseg;
    while (scanf("%d %d %d %d", &K, &dt, &sched, &nseg) == 4) {
      std::vector<int64_t> off(nseg + 1, 0);
      for (int s = 1; s <= nseg; ++s)
        if (scanf("%lld", reinterpret_cast<long long*>(&off[s])) != 1) return 1;
      std::string err;
      if (!validate_shape(K, off.data(), nseg, dt, sched, &err)) {
        printf("{\"error\": \"%s\"}\n", err.c_str());
        continue;
      }
      dump(build_plan(K, off.data(), nseg, static_cast<DType>(dt), static_cast<Schedule>(sched)), dt, sched, K);
    }
    return 0;
  }
  const int64_t off[3] = {0, 13, 40};
  std::vector<int> Ks;
  for (int K = 1; K <= 70; ++K) Ks.push_back(K);
  for (int K : {96, 127, 128, 129, 200, 255, 256, 257, 300}) Ks.push_back(K);
  for (int dt = 0; dt < 3; ++dt)
    for (int sched = 0; sched < 2; ++sched)
      for (int K : Ks)
        dump(build_plan(K, off, 2, static_cast<DType>(dt), static_cast<Schedule>(sched)), dt, sched, K);
  return 0;
}
