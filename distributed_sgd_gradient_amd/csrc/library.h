// library.h - internal interface between the library's host sources: the
// plan cache, argument validation and the stage scheduler (adasum.hip), used
// by the entry point that works in a fixed scratch array (noalloc.hip).
// Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <map>
#include <memory>
#include <mutex>
#include <string>

#include "plan.h"

namespace adasum {

// Device copies of a plan's tables.
struct DeviceTables {
  Tile* tiles = nullptr;
  int32_t* seg_tile = nullptr;
  BlockDesc* descs = nullptr;
  Merge* merges = nullptr;
};

struct CachedPlan {
  Plan plan;
  std::map<int, DeviceTables> per_device;
  // A call of this shape was made while its stream was being captured into
  // a HIP graph: the graph holds pointers to the device tables, so the shape
  // is never evicted and its tables are never freed.
  bool pinned = false;
};

// The buffers of one combine call (device pointers; grads is a host array).
struct CallBuffers {
  const void* const* grads;
  void* out;
  char* ws;
  double* coeffs;
  double* stats;
  double* ortho;
};

extern std::mutex g_mu;  // guards the plan cache, the library workspaces and the profiler

// Record msg as the calling thread's last error and return code.
int fail(int code, const std::string& msg);
int fail_hip(hipError_t e, const char* what);

// The cached plan of a validated shape (built on a miss).  Caller holds g_mu.
// may_free = false: a shape evicted to make room keeps its device tables
// until a later call that may free them.
std::shared_ptr<CachedPlan> find_plan(int K, const int64_t* off, int nseg, DType dt, Schedule sc,
                                      bool may_free = true);

// Host-side checks of a call's pointers (NULLs, alignment, overlaps; a
// workspace of ws_needed bytes when ws_needed > 0).
int validate_buffers(const void* const* grads, int K, int64_t N, size_t esz, int nseg, const void* out,
                     const void* ws, size_t ws_bytes, size_t ws_needed, const double* coeffs, const double* stats,
                     const double* ortho);

// Every buffer of a call is device memory of `device`, long enough where the
// runtime knows its extent.
int check_devices(const void* const* grads, int K, size_t vec_bytes, const void* out, const void* ws,
                  size_t ws_needed, const double* coeffs, const double* stats, const double* ortho, size_t nodes,
                  int nseg, int device);

// Whether work enqueued on st now is being captured into a graph.
bool capturing(hipStream_t st);

// Enqueue every stage of a plan on st.
int enqueue(const Plan& p, const DeviceTables& dt, const CallBuffers& b, hipStream_t st);

}  // namespace adasum
