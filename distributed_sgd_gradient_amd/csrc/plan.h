// plan.h - host-side execution plan of one Adasum combine shape.
//
// A plan depends only on (K, dtype, segment offsets).  It holds
//   * the tile table: every segment cut into tiles of at most kTile elements,
//     the first tile starting at the segment start and every later tile at a
//     multiple of kGroup elements, so that vector loads inside a tile are
//     16-byte aligned whatever the segment boundaries are;
//   * the tree schedule: level by level, pairs (v0,v1), (v2,v3), ... of the
//     current vectors with the odd last one carried (the recursive
//     application of the pairwise operator), and for every level the combine
//     jobs, each of which computes one node or two sibling nodes and, for
//     siblings, emits the statistics of the pair they form one level up;
//   * the workspace layout: fp32 slots for intermediate levels, the fp64
//     per-tile partial statistics, and the coefficient / statistic tables.
//
// Pure C++: it is built into the HIP library and into nothing else, and it
// makes no HIP call, so it can be exercised on a machine without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

namespace adasum {

constexpr int kGroup = 8;       // elements per thread per vector step (16 B of 16-bit, 32 B of fp32)
constexpr int kTile = 8192;     // elements per tile (a multiple of kGroup)
constexpr int kBlock = 256;     // threads per workgroup (4 wave64)
constexpr int kMaxJobs = 16;    // combine jobs per launch (kernel-argument budget)
constexpr int kMaxDotPairs = 32;  // triple-dot pairs per launch

enum class DType : int { F32 = 0, F16 = 1, BF16 = 2 };

inline size_t dtype_size(DType t) { return t == DType::F32 ? 4 : 2; }

struct Tile {      // 16 bytes, read by every kernel from device memory
  int64_t start;   // first element (global index into the N-element buffers)
  int32_t len;     // number of elements, 1..kTile
  int32_t seg;     // owning segment
};

// Where an operand or result of a tree node lives.
struct Ref {
  enum Kind : int8_t { Input = 0, Slot = 1, Out = 2 } kind;
  int32_t idx;     // worker index for Input, slot index for Slot
};

struct Pair {      // one tree node: node = Adasum(left, right) -> dst
  Ref left, right, dst;
  int node;        // global node id, level-major
};

struct Job {       // one combine job: one node, or two siblings + emitted stats
  int pair[2];     // indices into Level::pairs; pair[1] < 0 for a single node
  int emit;        // index of the next-level pair whose stats this job emits, or -1
};

struct Level {
  std::vector<Pair> pairs;
  std::vector<Job> jobs;
  std::vector<int> dot_pairs;  // pairs whose stats need a triple-dot pass first
  bool final_level = false;
};

struct Plan {
  int K = 0;
  DType dtype = DType::F32;
  int nseg = 0;
  int64_t N = 0;
  std::vector<int64_t> offsets;      // nseg + 1
  std::vector<Tile> tiles;
  std::vector<int32_t> seg_tile;     // nseg + 1: tiles of segment s are [seg_tile[s], seg_tile[s+1])
  std::vector<Level> levels;
  int nslots = 0;                    // fp32 intermediate vectors of N elements
  int carry_slot = -1;               // slot receiving the carried input when K is odd (K >= 3)
  int max_pairs = 0;                 // largest pair count of any level (partials rows)

  // workspace layout, byte offsets (each 256-aligned)
  size_t ws_slots = 0, ws_partials = 0, ws_coeffs = 0, ws_stats = 0, ws_total = 0;
  size_t partials_bytes() const { return (size_t)max_pairs * tiles.size() * 3 * sizeof(double); }
  size_t table_bytes(int per_node) const { return (size_t)(K > 1 ? K - 1 : 0) * nseg * per_node * sizeof(double); }
};

// Validate (K, offsets, nseg, dtype); on failure return false with a message.
bool validate_shape(int K, const int64_t* offsets, int nseg, int dtype, std::string* err);

// Build the plan of a validated shape.
Plan build_plan(int K, const int64_t* offsets, int nseg, DType dtype);

}  // namespace adasum
