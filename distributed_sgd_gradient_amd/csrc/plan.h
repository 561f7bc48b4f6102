// plan.h - host-side execution plan of one Adasum combine shape.
//
// A plan depends only on (K, dtype, segment offsets).  It holds
//   * the tile table: every segment cut into tiles of at most kTile
//     elements, the first tile starting at the segment start and every later
//     tile at a multiple of kGroup elements, so that vector loads inside a
//     tile are 16-byte aligned whatever the segment boundaries are;
//   * the tree, cut into stages.  Within a stage, every maximal subtree is a
//     block of up to four levels (16 operands); with at most 64 16-bit
//     inputs, whose Gram pass runs on the matrix cores, the single stage
//     takes five levels (32 operands) or six (64 operands).  Every
//     statistic a node of the block needs (a.b, |a|^2, |b|^2 of its two
//     children) is a quadratic form in the Gram matrix of the block's
//     operands, because every node is a linear combination of them; so a
//     block needs one Gram pass over its operands, a small per-segment walk
//     of its merges, and one weighted-sum pass that writes its result;
//   * the workspace layout: fp64 slots for block results that feed a later
//     stage, fp64 per-tile Gram partials and the low parts of their
//     double-double recomputation, leaf weights, the coefficient and
//     statistic tables, and per-(block, segment) flags of pairs whose Gram
//     matrix is recomputed exactly.  An input that a later stage reads (an
//     odd vector carried up the tree, or the chain's next inputs) is read
//     where it is, in its own dtype, next to the fp64 slots.
//
// Pure C++: it makes no HIP call, so it can be exercised without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

namespace adasum {

constexpr int kGroup = 8;        // elements per thread per vector step (16 B of 16-bit, 32 B of fp32)
constexpr int kTile = 32768;     // largest tile, elements (a multiple of kGroup)
constexpr int kMinTile = 2048;   // smallest tile a large segment is cut into
constexpr int kTargetTiles = 4096;  // tiles a workload is cut into when it is small
constexpr int kBlock = 256;      // threads per workgroup (4 wave64)
constexpr int kMaxOps = 64;      // operands per block over 16-bit inputs: up to six tree levels
constexpr int kMaxOps32 = 16;    // operands per block over fp32 operands: four tree levels
constexpr int kMaxJobs = 8;      // blocks per launch (kernel-argument budget)
// Operand pointers of a launch sit in one table, job j's operand k at
// j * op_stride(nbt) + k: 32 per job, or 64 for a launch of 64-operand
// blocks (then at most kArgOps * kMaxJobs / 64 jobs).
constexpr int kArgOps = 32;
constexpr int op_stride(int nbt) { return nbt > kArgOps ? 64 : kArgOps; }
constexpr int max_jobs(int nbt) { return kArgOps * kMaxJobs / op_stride(nbt); }
// The walk of a (block, segment) pair, one workgroup, sums the pair's Gram
// entries over the segment's tiles.  Where that is long (64-operand blocks,
// with 2080 entries; or a segment of at least kGroupMinTiles tiles) a
// separate launch first adds up groups of kTileGroup consecutive tiles over
// many workgroups, in place into each group's first tile, so that the walk
// reads one partial per group.
constexpr int kTileGroup = 16;
constexpr int kGroupMinTiles = 128;
// A one-stage plan of one block of at most 32 operands, with at most
// kFusedMaxRows elements and no empty segment, runs its walk and weighted
// sum in one launch after the Gram pass: every weighted-sum workgroup walks
// its own segment, so the small, launch-bound combines take two launches
// instead of five.  Each workgroup then reads all its segment's tile
// partials, so every segment must have at most kFusedMaxReads of them
// ((tiles of s) x (Gram entries)).
constexpr int64_t kFusedMaxRows = int64_t(1) << 22;
constexpr int64_t kFusedMaxReads = int64_t(1) << 13;
// Workgroups per tile of that launch.  Its tiles have at most kMinTile rows
// (see Plan::tile_rows), which one workgroup covers in one vector step.
constexpr int kFusedSplit = 1;
// Tiles of at most kExactRows rows of 16-bit inputs are short: their Gram
// matrices are summed exactly (double-double) instead of on the matrix cores,
// since short segments are where merges nearly cancel by chance.
constexpr int kExactRows = 256;
// The weighted sum cuts every tile into aligned parts, one workgroup each,
// so that a workgroup's range holds 16 KB of every operand of a full tile:
// 8 parts for fp32 inputs, 4 for 16-bit ones.  It streams best with shorter
// per-workgroup ranges than the Gram pass, whose per-tile reduction favours
// long tiles.
constexpr int wsum_split(int elem_bytes) { return elem_bytes == 4 ? 8 : 4; }
constexpr int kWsumSplitMax = 8;

// F64 is internal: the type of the slots that carry block results between
// stages (never a dtype of the C ABI).
enum class DType : int { F32 = 0, F16 = 1, BF16 = 2, F64 = 3 };

// Order in which the pairwise operator is applied to the K gradients.
//   Tree:  level by level, pairs (v0,v1), (v2,v3), ..., odd last carried;
//   Chain: left to right, acc = Adasum(acc, g_{i+1}).
enum class Schedule : int { Tree = 0, Chain = 1 };

inline size_t dtype_size(DType t) { return t == DType::F64 ? 8 : t == DType::F32 ? 4 : 2; }

// Largest block of the first stage.  Blocks of 32 or 64 operands (16-bit
// inputs only) pay off only where they finish the whole combine in one stage,
// without the fp64 intermediates of a second: above 64 inputs the tree needs
// a second stage anyway, and 16-operand blocks stream faster.  A chain takes
// 16 whatever the dtype.  Inside a block the walk carries each node's
// squared norm from merge to merge: |P'|^2 = ca (ca A + cb d) + cb (ca d +
// cb B).  Where the next operand is nearly parallel to the running result,
// that update cancels most of its terms, and an error already in A grows
// by the square of the merge's cancellation: about 4x per merge where the
// operand is much smaller, more near an opposite one.  The coefficients do
// not correct it (the node is what they define; the walk's record of its
// norm drifts).  Over the 31 or 63 merges of a 32- or 64-operand chain,
// segments of one to four random values reached coefficient errors of 1e-4
// to 4e-2; over 15 the largest in about 400,000 such chains was 7e-8.  The
// tree's five or six levels stay far below.
inline int first_stage_ops(DType t, int K, Schedule sc) {
  if (t == DType::F32 || K > kMaxOps || sc == Schedule::Chain) return kMaxOps32;
  return K <= 32 ? 32 : kMaxOps;
}

// Number of distinct entries of the symmetric n x n Gram matrix.
constexpr int gram_entries(int n) { return n * (n + 1) / 2; }

// Position of entry (i, j), i <= j, in the packed upper triangle (row-major).
constexpr int gram_index(int n, int i, int j) { return i * n - i * (i - 1) / 2 + (j - i); }

struct Tile {      // 24 bytes, read by every kernel from device memory
  int64_t start;   // first element (global index into the N-element buffers)
  int32_t len;     // number of elements
  int32_t seg;     // owning segment
  // the owning segment's tiles [seg_t0, seg_t1), so that a kernel that sums
  // them needs no second dependent load (seg_tile[seg])
  int32_t seg_t0, seg_t1;
};

// One tree node inside a block: node = Adasum(left, right), where left is
// the block operands [llo, lhi) and right the operands [lhi, rhi), each
// already combined into one vector by earlier merges of the block.
struct Merge {
  int8_t llo, lhi, rhi, pad;
  int32_t node;    // global node id, level-major over the whole tree
};

struct BlockDesc {  // device-visible description of one block
  int32_t nb;       // operands (1..64; 1 only for K = 1)
  int32_t nbt;      // Gram size the kernels use: 2, 4, 8, 16, 32 or 64 (operands >= nb are zero)
  int32_t merge0;   // first merge in the merge table
  int32_t nmerges;  // merges of this block, children before parents
  int64_t poff;     // Gram partials of tile t start at partials + poff + t * gram_entries(nbt)
  int32_t wrow;     // row of this block in the leaf-weight table
  int32_t root;     // 1 for the block whose result is the output
  uint64_t leafmask;  // bit k: operand k is one of the K input gradients
  // Relative rounding error of this block's Gram entries, against the sum of
  // |x_i x_j| that each entry adds up: the fp64 sums of the fp64 matrix cores
  // (fp32 inputs, fp64 slots) or the fp32 rounding of the 16-bit matrix
  // cores' 32-row chunks.  The tree walk flags the merges whose coefficients
  // such errors could move beyond tolerance.
  double gram_err;
};

// Where an operand or result lives.
struct Ref {
  enum Kind : int8_t { Input = 0, Slot = 1, Out = 2 } kind;
  int32_t idx;     // worker index for Input, slot index for Slot
};

struct Block {
  std::vector<Ref> operands;  // nb refs; all Input in stage 0; Slot, or Input carried up, later
  Ref dst;                    // Slot, or Out for the root block
  int desc;                   // index into Plan::descs
};

struct Stage {
  std::vector<Block> blocks;
};

struct Plan {
  int K = 0;
  DType dtype = DType::F32;
  Schedule schedule = Schedule::Tree;
  int nseg = 0;
  int64_t N = 0;
  int64_t tile_rows = kTile;      // tile length: about N / kTargetTiles, in [kMinTile, kTile]
  std::vector<int64_t> offsets;   // nseg + 1
  std::vector<Tile> tiles;
  std::vector<int32_t> seg_tile;  // nseg + 1: tiles of segment s are [seg_tile[s], seg_tile[s+1])
  std::vector<Stage> stages;
  std::vector<BlockDesc> descs;
  std::vector<Merge> merges;
  bool fused = false;             // see kFusedMaxRows
  bool tile_groups = false;       // some segment has kGroupMinTiles tiles or more
  int nslots = 0;                 // fp64 vectors of N elements
  int nblocks = 0;                // rows of the leaf-weight table
  size_t partial_doubles = 0;     // largest per-stage Gram partials footprint

  // workspace layout, byte offsets (each 256-aligned)
  size_t ws_slots = 0, ws_partials = 0, ws_weights = 0, ws_weights_lo = 0, ws_leafnorm = 0, ws_coeffs = 0, ws_stats = 0,
         ws_flags = 0, ws_plo = 0, ws_total = 0;
  size_t table_bytes(int per_node) const { return (size_t)(K > 1 ? K - 1 : 0) * nseg * per_node * sizeof(double); }
};

// Validate (K, offsets, nseg, dtype, schedule); on failure return false with a message.
bool validate_shape(int K, const int64_t* offsets, int nseg, int dtype, int schedule, std::string* err);

// Build the plan of a validated shape.
Plan build_plan(int K, const int64_t* offsets, int nseg, DType dtype, Schedule schedule);

}  // namespace adasum
