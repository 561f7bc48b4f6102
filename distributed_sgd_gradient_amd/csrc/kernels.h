// kernels.h - launch interface of the gfx950 Adasum kernels (library-internal).
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace adasum {

// Per-tile partial statistics (a.b, |a|^2, |b|^2) of up to kMaxDotPairs pairs.
// Partials of pair j, tile t go to partials[(row[j] * ntiles + t) * 3 + {0,1,2}].
struct DotArgs {
  const void* a[kMaxDotPairs];
  const void* b[kMaxDotPairs];
  int row[kMaxDotPairs];
  const Tile* tiles;
  int ntiles;
  double* partials;
};

// Per (pair, segment): sum the tile partials in tile order, derive the
// coefficients, write the coefficient and statistic tables.
struct FinalizeArgs {
  const double* partials;   // rows 0..npairs-1, ntiles each
  const int32_t* seg_tile;  // nseg + 1
  int ntiles;
  int nseg;
  int npairs;
  int first_node;           // global node id of pair 0 of this level
  double* coeffs;           // [K-1][nseg][2]
  double* stats;            // [K-1][nseg][3]
};

// One launch of combine jobs: each job computes one node c = ca*x0 + cb*x1,
// or two sibling nodes and the per-tile statistics of the pair they form.
struct CombineArgs {
  const void* x[kMaxJobs][4];
  void* y[kMaxJobs][2];
  int node[kMaxJobs][2];
  int emit[kMaxJobs];       // partials row for the emitted statistics (sibling jobs)
  const Tile* tiles;
  int ntiles;
  int nseg;
  const double* coeffs;
  double* partials;
};

// Widen one input to fp32 over every tile.
struct WidenArgs {
  const void* src;
  float* dst;
  const Tile* tiles;
};

// Operand element type of a launch: the input dtype, or fp32 for slots.
hipError_t launch_triple_dot(DType operand, const DotArgs& a, int npairs, hipStream_t st);
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t st);
// in_t: type of x operands; out_t: type of y results; siblings: two-node jobs
hipError_t launch_combine(DType in_t, DType out_t, bool siblings, const CombineArgs& a, int njobs,
                          hipStream_t st);
hipError_t launch_widen(DType src_t, const WidenArgs& a, int ntiles, hipStream_t st);

}  // namespace adasum
