// noalloc.hip - the combine for callers that cannot allocate device memory.
//
// adasum_combine_noalloc runs the same kernels as adasum_combine_ex, with the
// workspace and the plan tables of the call in a fixed array of device memory
// (`scratch`, below) instead of memory the caller or the library allocates.
// It calls no hipMalloc or hipFree: the tables are copied into the array on
// the call's stream, and a plan evicted from the library's cache to make room
// for this call's shape keeps its device tables until a later call that may
// free them.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <map>
#include <memory>
#include <mutex>
#include <string>

#include "../../include/adasum.h"
#include "library.h"
#include "plan.h"

// Every GPU the library runs on holds its own copy of this array until the
// process ends.  In host code `scratch` is a host-side stand-in for the
// symbol, not a device address: only the address hipGetSymbolAddress returns
// for the current device is passed to kernels and copies.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace adasum {
namespace {

std::map<int, char*> g_scratch;  // device -> address of its copy of scratch; guarded by g_mu

// Caller holds g_mu, with `device` current.  The address is taken once per
// device, at that device's first call.
int scratch_of(int device, char** out) {
  auto it = g_scratch.find(device);
  if (it != g_scratch.end()) {
    *out = it->second;
    return ADASUM_OK;
  }
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress of the scratch array");
  if (ptr == nullptr) return fail(ADASUM_EHIP, "hipGetSymbolAddress returned NULL for the scratch array");
  g_scratch[device] = static_cast<char*>(ptr);
  *out = static_cast<char*>(ptr);
  return ADASUM_OK;
}

// Where a call's plan tables go in the array: behind its workspace, each
// table 256-byte aligned.
struct ScratchLayout {
  size_t tiles, seg_tile, descs, merges, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

ScratchLayout scratch_layout(const Plan& p) {
  ScratchLayout L;
  size_t off = align256(p.ws_total);
  L.tiles = off;
  off = align256(off + sizeof(Tile) * p.tiles.size());
  L.seg_tile = off;
  off = align256(off + sizeof(int32_t) * p.seg_tile.size());
  L.descs = off;
  off = align256(off + sizeof(BlockDesc) * p.descs.size());
  L.merges = off;
  off = align256(off + sizeof(Merge) * p.merges.size());
  L.total = off;
  return L;
}

int combine_noalloc(const void* const* grads, int K, const int64_t* seg_offsets, int nseg, int dtype, int schedule,
                    void* out, double* coeffs, double* stats, double* ortho, void* stream) {
  std::string err;
  if (!validate_shape(K, seg_offsets, nseg, dtype, schedule, &err)) return fail(ADASUM_EINVAL, err);
  const DType dt = static_cast<DType>(dtype);
  const Schedule sc = static_cast<Schedule>(schedule);
  const int64_t N = seg_offsets[nseg];
  std::lock_guard<std::mutex> lock(g_mu);
  std::shared_ptr<CachedPlan> cp = find_plan(K, seg_offsets, nseg, dt, sc, /*may_free=*/false);
  const Plan& p = cp->plan;
  const ScratchLayout L = scratch_layout(p);
  if (L.total > kScratchBytes) {
    char buf[240];
    snprintf(buf, sizeof buf,
             "this shape needs %zu bytes of scratch, more than the %zu that adasum_combine_noalloc holds; use "
             "adasum_combine_ex with a workspace of adasum_workspace_bytes()", L.total, kScratchBytes);
    return fail(ADASUM_EINVAL, buf);
  }
  int rc = validate_buffers(grads, K, N, dtype_size(dt), nseg, out, nullptr, 0, 0, coeffs, stats, ortho);
  if (rc != ADASUM_OK) return rc;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  rc = check_devices(grads, K, (size_t)N * dtype_size(dt), out, nullptr, 0, coeffs, stats, ortho,
                     K > 1 ? (size_t)(K - 1) : 0, nseg, device);
  if (rc != ADASUM_OK) return rc;
  char* base = nullptr;
  rc = scratch_of(device, &base);
  if (rc != ADASUM_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (capturing(st))
    return fail(ADASUM_EINVAL, "adasum_combine_noalloc copies its tables from host memory on every call and cannot "
                               "be captured into a graph; capture adasum_combine_ex with a workspace allocated "
                               "before the capture");
  // The tables are copied from the host plan on the call's stream; a copy
  // from pageable host memory has consumed its source when it returns.
  // Nothing in the workspace needs to start at zero: every kernel writes the
  // regions it reads before reading them (Gram partials and their low parts,
  // weights, flags, the lower stages' slots).
  const struct {
    size_t at;
    const void* src;
    size_t bytes;
  } copies[] = {
      {L.tiles, p.tiles.data(), sizeof(Tile) * p.tiles.size()},
      {L.seg_tile, p.seg_tile.data(), sizeof(int32_t) * p.seg_tile.size()},
      {L.descs, p.descs.data(), sizeof(BlockDesc) * p.descs.size()},
      {L.merges, p.merges.data(), sizeof(Merge) * p.merges.size()},
  };
  for (const auto& c : copies) {
    if (c.bytes == 0) continue;
    e = hipMemcpyAsync(base + c.at, c.src, c.bytes, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return fail_hip(e, "copying the plan tables into the scratch array");
  }
  DeviceTables tables;
  tables.tiles = reinterpret_cast<Tile*>(base + L.tiles);
  tables.seg_tile = reinterpret_cast<int32_t*>(base + L.seg_tile);
  tables.descs = reinterpret_cast<BlockDesc*>(base + L.descs);
  tables.merges = reinterpret_cast<Merge*>(base + L.merges);
  CallBuffers b;
  b.grads = grads;
  b.out = out;
  b.ws = base;
  b.coeffs = coeffs ? coeffs : reinterpret_cast<double*>(base + p.ws_coeffs);
  b.stats = stats ? stats : reinterpret_cast<double*>(base + p.ws_stats);
  b.ortho = ortho;
  return enqueue(p, tables, b, st);
}

}  // namespace
}  // namespace adasum

extern "C" int adasum_combine_noalloc(const void* const* grads, int K, const int64_t* seg_offsets, int nseg,
                                      int dtype, int schedule, void* out, double* coeffs, double* stats,
                                      double* ortho, void* stream) {
  return adasum::combine_noalloc(grads, K, seg_offsets, nseg, dtype, schedule, out, coeffs, stats, ortho, stream);
}
