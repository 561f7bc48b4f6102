// kernels.h - launch interface of the gfx950 Adasum kernels (library-internal).
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace adasum {

// Gram pass: per (block, tile), the packed upper triangle of the fp64 Gram
// matrix of the block's operands over the tile.  Operand k of job j is
// x[j * op_stride(nbt) + k]; those at or beyond the block's operand count are
// NULL and read as zero.  In a launch
// over fp64 slots (a stage above the first), bit k of narrow[j] marks operand
// k of job j as an input gradient, read in the inputs' dtype and widened
// exactly.
struct GramArgs {
  const void* x[kMaxJobs * kArgOps];
  uint32_t narrow[kMaxJobs];
  int64_t poff[kMaxJobs];  // partials of tile t: partials + poff + t * gram_entries(nbt)
  const Tile* tiles;
  double* partials;
  // low parts of double-double entries at the same index as in partials:
  // written by the exact sums of short 16-bit tiles and by the exact
  // recomputation of flagged pairs
  double* partials_lo;
  // exact recomputation only: the tiles of (block, segment) pairs whose
  // flags[wrow[j]][segment] is set
  const uint32_t* flags;
  int32_t wrow[kMaxJobs];
  int nseg;
  int short_tiles;  // every tile has at most kMinTile rows
};
static_assert(sizeof(GramArgs) <= 4096, "kernel arguments fit 4 KB");

// Tree walk: per (block, segment), sum the tile Gram partials in tile order,
// then evaluate the block's merges on the Gram matrix: statistics,
// coefficients and the final weight of every operand.
struct TreeArgs {
  const BlockDesc* descs;
  const Merge* merges;
  const int32_t* seg_tile;  // nseg + 1
  const double* partials;
  // a segment of one short tile (tiles[t].len <= kExactRows) of a block over
  // 16-bit inputs (lo_inputs) takes its Gram entries as partials +
  // partials_lo (double-double); the refining walk takes every entry so
  const double* partials_lo;
  const Tile* tiles;
  int lo_inputs;
  int desc0;                // first block of this launch (consecutive descs)
  int nblocks;
  int nblocks_total;        // blocks of the whole plan (rows of weights / leafnorm)
  int nseg;
  double* weights;          // [nblocks total][nseg][kMaxOps]: operand weights, rounded to fp64
  double* weights_lo;       // the same layout: their double-double low parts
  double* leafnorm;         // [nblocks total][nseg]: sum of |g_k|^2 over the block's input operands
  double* coeffs;           // [K-1][nseg][2]
  double* stats;            // [K-1][nseg][3]
  double* ortho;            // [nseg] or NULL: |result|^2 / sum_k |g_k|^2, written by the root block
  // refine = 0: every pair is walked, and flags[wrow][segment] is written
  // (flags NULL: no flags): bit 0 where the Gram entries' rounding
  // (BlockDesc::gram_err) could move a coefficient by more than kRefineTol
  // (kRefineTol16 over 16-bit inputs)
  // of it, bit 1 there too and where the block's result is at most
  // kSumCancel of its weighted parts in squared norm.  refine = 1: only pairs
  // with bit 0 are walked again, on the recomputed double-double entries.
  // The weighted sum adds up pairs with bit 1 in double-double.
  uint32_t* flags;          // [nblocks total][nseg]
  int refine;
  int wide;                 // some block of the launch has 64 operands (nbt = 64)
  int grouped;              // launch_tile_groups ran on this launch's partials
};

// Relative coefficient error bound above which a pair's Gram matrix is
// recomputed exactly (the coefficient gate is 1e-6): blocks whose entries are
// fp64 sums (fp32 inputs, fp64 slots).  A coefficient's error moves every
// node built on it, and a chain that cancels again later can amplify it a
// thousandfold by its end, so the bound sits well below the gate wherever
// that costs nothing on ordinary data (an entry errs by about 2^-44 of its
// terms there; the bound flags a merge only where its parts cancel to
// below about 1/40 of their norm).  Blocks over 16-bit inputs, whose
// entries carry the matrix cores' fp32 rounding (2^-24), would flag every
// merge at that bound and keep kRefineTol16.
constexpr double kRefineTol = 1e-10;
constexpr double kRefineTol16 = 2.5e-7;

// A block result whose squared norm is at most this fraction of
// sum_k w_k^2 |x_k|^2 is summed in double-double: in fp64 its rounding would
// be about 2^-53 sqrt(NB / kSumCancel) of the result.
constexpr double kSumCancel = 1e-2;

// Weighted sum: per (block, tile), y = sum_k w_k x_k in fp64, rounded once
// to the result's type (an fp64 slot keeps the sum as it is); narrow as for
// the Gram pass.
struct WsumArgs {
  const void* x[kMaxJobs * kArgOps];  // laid out as in GramArgs
  uint32_t narrow[kMaxJobs];
  void* y[kMaxJobs];
  int wrow[kMaxJobs];
  const Tile* tiles;
  int nseg;
  const double* weights;
  const double* weights_lo;  // low parts of the double-double weights
  const uint32_t* flags;     // the walk's flags: bit 1 selects the double-double sum
};
static_assert(sizeof(WsumArgs) <= 4096, "kernel arguments fit 4 KB");

// The same arguments for a launch of one job of at most kArgOps operands
// (the small combines of Plan::fused).  The host's cost of a launch grows
// with the size of its arguments, and these launches are bound by it.
struct GramArgs1 {
  const void* x[kArgOps];
  uint32_t narrow[1];
  int64_t poff[1];
  const Tile* tiles;
  double* partials;
  double* partials_lo;
  const uint32_t* flags;
  int32_t wrow[1];
  int nseg;
  int short_tiles;
};
struct WsumArgs1 {
  const void* x[kArgOps];
  uint32_t narrow[1];
  void* y[1];
  int wrow[1];
  const Tile* tiles;
  int nseg;
  const double* weights;
  const double* weights_lo;
  const uint32_t* flags;
};

// Plain sum of up to kSumOps operands, element by element in fp64, in
// operand order: acc = (acc_in ? acc_in : 0) + x0 + x1 + ...; the result goes
// to acc_out (fp64) or, rounded once, to out.
constexpr int kSumOps = 64;
struct SumArgs {
  const void* x[kSumOps];
  int nx;
  const double* acc_in;
  double* acc_out;
  void* out;
  int64_t n;
};

// nbt: Gram size of every block in the launch (2 .. 32).  operand: the
// operands' type (F64: fp64 slots of a later stage); narrow_t: with F64, the
// dtype of the input operands the narrow masks mark.
hipError_t launch_gram(DType operand, DType narrow_t, int nbt, const GramArgs& a, int ntiles, int njobs,
                       hipStream_t st);
hipError_t launch_tree(const TreeArgs& a, hipStream_t st);
// For the blocks of a launch (descs desc0 .. desc0 + nblocks - 1): the Gram
// partials of each group of kTileGroup consecutive tiles of a segment with
// more than one tile, added in tile order in fp64 into the group's first
// tile.  A tree launch on those partials then sets `grouped`.
hipError_t launch_tile_groups(const TreeArgs& a, int ntiles, hipStream_t st);
// The Gram partials of every tile of a flagged (block, segment) pair,
// recomputed exactly: double-double sums of exact products in row order,
// high parts to partials, low parts to partials_lo.  Other tiles return at once.
hipError_t launch_gram_exact(DType operand, DType narrow_t, int nbt, const GramArgs& a, int ntiles, int njobs,
                             hipStream_t st);
// out_t: F64 for a slot that feeds a later stage, else the output dtype.
hipError_t launch_wsum(DType in_t, DType narrow_t, int nbt, DType out_t, const WsumArgs& a, int ntiles, int njobs,
                       hipStream_t st);
hipError_t launch_sum(DType t, const SumArgs& a, hipStream_t st);
// A one-stage plan of one block of at most 32 operands whose segments have
// few tiles (Plan::fused): after its Gram pass, the walk, any exact
// recomputation and the weighted sum in one launch over the weighted sum's
// grid (t as for launch_tree, w as for launch_wsum of that block).
hipError_t launch_fused(DType in_t, int nbt, const TreeArgs& t, const WsumArgs1& w, int ntiles, hipStream_t st);
// The Gram pass of that plan's one block (inputs of type operand).
hipError_t launch_gram1(DType operand, int nbt, const GramArgs1& a, int ntiles, hipStream_t st);

}  // namespace adasum
