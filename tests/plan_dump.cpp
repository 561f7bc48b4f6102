// Prints the execution plan of K = 1..70 and a few larger K, both schedules,
// fp32 and fp16 inputs, as JSON lines, for tests/test_plan_host.py.  Built with g++ on the host together
// with the library's plan.cpp (pure C++, no HIP).
#include <cstdio>
#include <vector>

#include "plan.h"

using namespace adasum;

int main() {
  const int64_t off[3] = {0, 13, 40};
  std::vector<int> Ks;
  for (int K = 1; K <= 70; ++K) Ks.push_back(K);
  for (int K : {96, 127, 128, 129, 200, 255, 256, 257, 300}) Ks.push_back(K);
  for (int dt = 0; dt < 2; ++dt)
  for (int sched = 0; sched < 2; ++sched) {
    for (int K : Ks) {
      const DType dtype = dt ? DType::F16 : DType::F32;
      const Plan p = build_plan(K, off, 2, dtype, static_cast<Schedule>(sched));
      printf("{\"dtype\": %d, \"schedule\": %d, \"K\": %d, \"nslots\": %d, \"stages\": [", dt, sched, K, p.nslots);
      for (size_t s = 0; s < p.stages.size(); ++s) {
        const Stage& st = p.stages[s];
        printf("%s{\"widen\": [", s ? "," : "");
        for (size_t i = 0; i < st.widen.size(); ++i)
          printf("%s[%d,%d]", i ? "," : "", st.widen[i].first, st.widen[i].second);
        printf("], \"blocks\": [");
        for (size_t b = 0; b < st.blocks.size(); ++b) {
          const Block& bk = st.blocks[b];
          const BlockDesc& d = p.descs[bk.desc];
          printf("%s{\"ops\": [", b ? "," : "");
          for (size_t k = 0; k < bk.operands.size(); ++k)
            printf("%s[%d,%d]", k ? "," : "", (int)bk.operands[k].kind, bk.operands[k].idx);
          printf("], \"dst\": [%d,%d], \"nb\": %d, \"nbt\": %d, \"leafmask\": %u, \"root\": %d, \"merges\": [",
                 (int)bk.dst.kind, bk.dst.idx, d.nb, d.nbt, d.leafmask, (int)d.root);
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
        printf("%s[%lld,%d,%d]", t ? "," : "", (long long)p.tiles[t].start, p.tiles[t].len, p.tiles[t].seg);
      printf("], \"ws_total\": %zu}\n", p.ws_total);
    }
  }
  return 0;
}
