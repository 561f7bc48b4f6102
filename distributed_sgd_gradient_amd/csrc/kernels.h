// kernels.h - launch interface of the gfx950 Adasum kernels (library-internal).
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace adasum {

// Gram pass: per (block, tile), the packed upper triangle of the fp64 Gram
// matrix of the block's operands over the tile.  Operands x[j][k] with k at
// or beyond the block's operand count are NULL and read as zero.  In an fp32
// launch, bit k of narrow[j] marks operand k of job j as an input gradient
// stored in the launch's 16-bit type (read and widened exactly on load).
struct GramArgs {
  const void* x[kMaxJobs][kMaxOps];
  uint32_t narrow[kMaxJobs];
  int64_t poff[kMaxJobs];  // partials of tile t: partials + poff + t * gram_entries(nbt)
  const Tile* tiles;
  double* partials;
  // short tiles (at most kExactRows rows) of 16-bit launches and of blocks
  // that read a slot sum their entries exactly in double-double and write
  // the low parts here, at the same index as in partials (NULL: not kept)
  double* partials_lo;
  // exact recomputation only: the tiles of (block, segment) pairs whose
  // flags[wrow[j]][segment] is set
  const uint32_t* flags;
  int32_t wrow[kMaxJobs];
  int nseg;
  // fp32 operands only: operand k of job j is the fp32 slot side_slot[j][k]
  // (-1: not a slot); a short tile (short_off[t] >= 0) whose job reads a slot
  // takes that slot's rows from its fp64 side buffer, side + slot *
  // short_rows + short_off[t], and sums its Gram matrix exactly.  short_off
  // NULL: no side buffers.
  const double* side;
  const int64_t* short_off;
  int64_t short_rows;
  int32_t side_slot[kMaxJobs][kMaxOps];
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
  // a segment of one short tile (tiles[t].len <= kExactRows) takes its Gram
  // entries as partials + partials_lo (double-double) when its block reads a
  // slot, or when lo_inputs is set (16-bit inputs); NULL: fp64 entries only
  const double* partials_lo;
  const Tile* tiles;
  int lo_inputs;
  int desc0;                // first block of this launch (consecutive descs)
  int nblocks;
  int nblocks_total;        // blocks of the whole plan (rows of weights / leafnorm)
  int nseg;
  double* weights;          // [nblocks total][nseg][kMaxOps]
  double* leafnorm;         // [nblocks total][nseg]: sum of |g_k|^2 over the block's input operands
  double* coeffs;           // [K-1][nseg][2]
  double* stats;            // [K-1][nseg][3]
  double* ortho;            // [nseg] or NULL: |result|^2 / sum_k |g_k|^2, written by the root block
  // Every chunk sum behind a Gram entry carries a relative rounding error of
  // at most gram_err (0: the entries are exact up to fp64 rounding).  With
  // gram_err > 0 the walk sets flags[wrow][segment] to 1 where those errors
  // could move a coefficient by more than kRefineTol of it, else to 0.
  // refine = 1: only flagged pairs are walked (again).
  double gram_err;
  uint32_t* flags;          // [nblocks total][nseg]
  int refine;
};

// Relative coefficient error bound above which a pair's Gram matrix is
// recomputed exactly (the coefficient gate is 1e-6).
constexpr double kRefineTol = 2.5e-7;

// Weighted sum: per (block, tile), y = sum_k w_k x_k, rounded once; narrow
// as for the Gram pass.
struct WsumArgs {
  const void* x[kMaxJobs][kMaxOps];
  uint32_t narrow[kMaxJobs];
  void* y[kMaxJobs];
  int wrow[kMaxJobs];
  const Tile* tiles;
  int nseg;
  const double* weights;
  // a job whose result is an fp32 slot also writes the fp64 sums of short
  // tiles to its side buffer, side[j][short_off[t] + row - tile start]
  // (side[j] NULL: not a slot, or no short tiles)
  double* side[kMaxJobs];
  const int64_t* short_off;
  // operand k of job j is the fp32 slot side_slot[j][k] when bit k of
  // side_mask[j] is set; in a short tile that operand is read from the
  // slot's fp64 side buffer, side_in + slot * short_rows + short_off[t], so
  // a result carried through several stages is rounded only at the root
  const double* side_in;
  int64_t short_rows;
  uint32_t side_mask[kMaxJobs];
  int32_t side_slot[kMaxJobs][kMaxOps];
};
static_assert(sizeof(WsumArgs) <= 4096, "kernel arguments fit 4 KB");

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
// operands' dtype; with operand F32, narrow_t is the 16-bit dtype of the
// operands the narrow masks mark (F32 when there are none).
hipError_t launch_gram(DType operand, DType narrow_t, int nbt, const GramArgs& a, int ntiles, int njobs,
                       hipStream_t st);
hipError_t launch_tree(const TreeArgs& a, hipStream_t st);
// 16-bit operands: the Gram partials of every tile of a flagged (block,
// segment) pair, recomputed exactly (double-double sums of exact products, row order).
hipError_t launch_gram_exact(DType operand, int nbt, const GramArgs& a, int ntiles, int njobs, hipStream_t st);
hipError_t launch_wsum(DType in_t, DType narrow_t, int nbt, DType out_t, const WsumArgs& a, int ntiles, int njobs,
                       hipStream_t st);
hipError_t launch_sum(DType t, const SumArgs& a, hipStream_t st);

}  // namespace adasum
