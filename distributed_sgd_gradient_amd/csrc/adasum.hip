// adasum.hip - C ABI, argument validation, plan cache and stage scheduler.
//
// The tree is cut into stages of at most four levels (five when at most 32
// 16-bit inputs make it one stage); each stage is a set of blocks (subtrees
// of at most 16 operands, or that one 32-operand block).  A block above the
// first stage reads fp64 slots (lower blocks' results) and, where an input is
// carried up, that input in its own dtype.  One call enqueues, stage by stage:
//   1. gram: one launch per (block size, operand type) over every block and
//      every tile: the Gram partials of each block's operands, in fp64;
//   2. tree: one launch over every (block, segment): tile partials summed in
//      tile order, every merge of the block evaluated on the Gram matrix
//      (statistics, coefficients), the final operand weights written, and a
//      flag on every pair whose coefficients the rounding of its Gram
//      entries could move beyond tolerance (a merge under deep
//      cancellation); one launch per Gram launch recomputes the flagged
//      pairs' tiles exactly (the others return at once) and a second walk
//      redoes only them;
//   3. wsum: one launch per (block size, types) over every block and tile:
//      the block's result, sum_k w_k x_k (in double-double for flagged
//      pairs), into an fp64 slot or into out.
// So a combine of K <= 16 gradients (K <= 32 for 16-bit ones) is five
// launches and two passes over the inputs, whatever the number of segments.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iterator>
#include <list>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/adasum.h"
#include "kernels.h"
#include "library.h"
#include "plan.h"

namespace adasum {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

// ADASUM_LOG=1 in the environment: one line on stderr per new plan and per
// launch (kind, grid, algorithmic bytes), for tracing a call's schedule.
bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("ADASUM_LOG");
    return v != nullptr && v[0] != '\0' && v[0] != '0';
  }();
  return on;
}

void log_launch(const char* kind, int stage, int ntiles, int njobs, int nbt, double bytes) {
  if (!log_enabled()) return;
  std::fprintf(stderr, "[adasum] stage %d %-5s grid %d x %d  Gram size %d  %.0f bytes\n", stage, kind, ntiles, njobs,
               nbt, bytes);
}

int fail_hip(hipError_t e, const char* what) {
  char buf[256];
  snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(e));
  g_last_error = buf;
  return ADASUM_EHIP;
}

// ---------------------------------------------------------------- plan cache

constexpr size_t kMaxCachedPlans = 64;

std::mutex g_mu;  // guards every library-wide table below
std::list<std::shared_ptr<CachedPlan>> g_plans;    // most recently used first
std::vector<std::shared_ptr<CachedPlan>> g_retired;  // evicted by a call that may not free; freed later

bool same_shape(const Plan& p, int K, const int64_t* off, int nseg, DType dt, Schedule sc) {
  return p.K == K && p.nseg == nseg && p.dtype == dt && p.schedule == sc &&
         std::memcmp(p.offsets.data(), off, sizeof(int64_t) * (size_t)(nseg + 1)) == 0;
}

void release_tables(CachedPlan& cp) {
  if (cp.per_device.empty()) return;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return;
  for (auto& kv : cp.per_device) {
    if (hipSetDevice(kv.first) != hipSuccess) continue;
    (void)hipDeviceSynchronize();  // kernels of earlier calls may still read the tables
    (void)hipFree(kv.second.tiles);
    (void)hipFree(kv.second.seg_tile);
    (void)hipFree(kv.second.descs);
    (void)hipFree(kv.second.merges);
  }
  cp.per_device.clear();
  (void)hipSetDevice(cur);
}

// may_free = false: for the no-allocation entry point, which calls no hipFree.
std::shared_ptr<CachedPlan> find_plan(int K, const int64_t* off, int nseg, DType dt, Schedule sc, bool may_free) {
  if (may_free) {
    for (auto& r : g_retired) release_tables(*r);
    g_retired.clear();
  }
  for (auto it = g_plans.begin(); it != g_plans.end(); ++it) {
    if (same_shape((*it)->plan, K, off, nseg, dt, sc)) {
      auto hit = *it;
      g_plans.erase(it);
      g_plans.push_front(hit);
      return hit;
    }
  }
  auto cp = std::make_shared<CachedPlan>();
  cp->plan = build_plan(K, off, nseg, dt, sc);
  if (log_enabled()) {
    const Plan& p = cp->plan;
    std::fprintf(stderr, "[adasum] plan K=%d nseg=%d N=%lld dtype=%d schedule=%s: %zu tiles of <= %lld, %zu stages, "
                 "%d blocks, %d slots, workspace %zu bytes\n", K, nseg, (long long)p.N, (int)dt,
                 sc == Schedule::Tree ? "tree" : "chain", p.tiles.size(), (long long)p.tile_rows, p.stages.size(),
                 p.nblocks, p.nslots, p.ws_total);
  }
  g_plans.push_front(cp);
  // evict the least recently used shape that no captured graph refers to
  size_t unpinned = 0;
  for (auto& q : g_plans) unpinned += q->pinned ? 0 : 1;
  if (unpinned > kMaxCachedPlans) {
    for (auto it = std::prev(g_plans.end());; --it) {
      if (!(*it)->pinned && *it != cp) {
        if (may_free)
          release_tables(**it);
        else
          g_retired.push_back(*it);
        g_plans.erase(it);
        break;
      }
      if (it == g_plans.begin()) break;
    }
  }
  return cp;
}

// Whether work enqueued on st now is being captured into a graph.
bool capturing(hipStream_t st) {
  hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &status) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return status != hipStreamCaptureStatusNone;
}

// Caller holds g_mu.  Uploads the plan tables to `device` once.
int device_tables(CachedPlan& cp, int device, DeviceTables* out) {
  auto it = cp.per_device.find(device);
  if (it != cp.per_device.end()) {
    *out = it->second;
    return ADASUM_OK;
  }
  const Plan& p = cp.plan;
  DeviceTables t;
  struct Upload {
    void** dst;
    const void* src;
    size_t bytes;
  } ups[] = {
      {reinterpret_cast<void**>(&t.tiles), p.tiles.data(), sizeof(Tile) * p.tiles.size()},
      {reinterpret_cast<void**>(&t.seg_tile), p.seg_tile.data(), sizeof(int32_t) * p.seg_tile.size()},
      {reinterpret_cast<void**>(&t.descs), p.descs.data(), sizeof(BlockDesc) * p.descs.size()},
      {reinterpret_cast<void**>(&t.merges), p.merges.data(), sizeof(Merge) * p.merges.size()},
  };
  int rc = ADASUM_OK;
  for (Upload& u : ups) {
    if (hipMalloc(u.dst, u.bytes > 0 ? u.bytes : 16) != hipSuccess) {
      *u.dst = nullptr;
      rc = fail(ADASUM_ENOMEM, "hipMalloc of a plan table failed");
      break;
    }
    if (u.bytes > 0) {
      hipError_t e = hipMemcpy(*u.dst, u.src, u.bytes, hipMemcpyHostToDevice);
      if (e != hipSuccess) {
        rc = fail_hip(e, "uploading the plan tables");
        break;
      }
    }
  }
  if (rc != ADASUM_OK) {
    for (Upload& u : ups)
      if (*u.dst) (void)hipFree(*u.dst);
    return rc;
  }
  cp.per_device[device] = t;
  *out = t;
  return ADASUM_OK;
}

// ---------------------------------------------------------------- library workspace

struct OwnedWorkspace {
  void* ptr = nullptr;
  size_t bytes = 0;
  bool captured = false;  // used under graph capture: never freed (a graph may still refer to it)
};
std::map<std::pair<int, void*>, OwnedWorkspace> g_ws;  // (device, stream) -> buffer; guarded by g_mu

// ---------------------------------------------------------------- launch timing

enum KernelKind { kGram = 0, kTree, kWsum, kSum, kExact, kNumKinds };
const char* const kKindNames[kNumKinds] = {"gram", "tree", "wsum", "sum", "exact"};

struct ProfRecord {
  int kind;
  double bytes;
  hipEvent_t start, stop;
};

bool g_prof_on = false;                                 // guarded by g_mu
std::vector<ProfRecord> g_prof;                         // guarded by g_mu
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_ev_pool;  // guarded by g_mu

// Records the start event of a launch; returns the record index or -1.
int prof_start(int kind, double bytes, hipStream_t st) {
  if (!g_prof_on) return -1;
  std::pair<hipEvent_t, hipEvent_t> ev{nullptr, nullptr};
  if (!g_ev_pool.empty()) {
    ev = g_ev_pool.back();
    g_ev_pool.pop_back();
  } else if (hipEventCreate(&ev.first) != hipSuccess || hipEventCreate(&ev.second) != hipSuccess) {
    return -1;
  }
  if (hipEventRecord(ev.first, st) != hipSuccess) {
    g_ev_pool.push_back(ev);
    return -1;
  }
  g_prof.push_back(ProfRecord{kind, bytes, ev.first, ev.second});
  return (int)g_prof.size() - 1;
}

void prof_stop(int idx, hipStream_t st) {
  if (idx >= 0) (void)hipEventRecord(g_prof[idx].stop, st);
}

// ---------------------------------------------------------------- validation helpers

struct Range {
  uintptr_t lo, hi;
  const char* name;
};

bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// Checks every pointer argument of a combine call against the shape.
int validate_buffers(const void* const* grads, int K, int64_t N, size_t esz, int nseg, const void* out,
                     const void* ws, size_t ws_bytes, size_t ws_needed, const double* coeffs,
                     const double* stats, const double* ortho) {
  char buf[200];
  if (grads == nullptr) return fail(ADASUM_EINVAL, "grads is NULL");
  const size_t vec_bytes = (size_t)N * esz;
  if (N > 0) {
    if (out == nullptr) return fail(ADASUM_EINVAL, "out is NULL");
    if (!aligned16(out)) return fail(ADASUM_EINVAL, "out must be 16-byte aligned");
    for (int k = 0; k < K; ++k) {
      if (grads[k] == nullptr) {
        snprintf(buf, sizeof buf, "grads[%d] is NULL", k);
        return fail(ADASUM_EINVAL, buf);
      }
      if (!aligned16(grads[k])) {
        snprintf(buf, sizeof buf, "grads[%d] must be 16-byte aligned", k);
        return fail(ADASUM_EINVAL, buf);
      }
    }
  }
  if (ws_needed > 0) {
    if (ws == nullptr) return fail(ADASUM_EINVAL, "workspace is NULL but this shape needs one");
    if (ws_bytes < ws_needed) {
      snprintf(buf, sizeof buf, "workspace too small: %zu bytes given, %zu needed", ws_bytes, ws_needed);
      return fail(ADASUM_EINVAL, buf);
    }
    if (!aligned16(ws)) return fail(ADASUM_EINVAL, "workspace must be 16-byte aligned");
  }
  if (!aligned8(coeffs) || !aligned8(stats) || !aligned8(ortho))
    return fail(ADASUM_EINVAL, "coeffs, stats and ortho must be 8-byte aligned");
  const size_t nodes = K > 1 ? (size_t)(K - 1) : 0;
  auto rng = [](const void* p, size_t bytes, const char* name) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes, name};
  };
  std::vector<Range> written;
  if (vec_bytes > 0) written.push_back(rng(out, vec_bytes, "out"));
  if (ws_needed > 0) written.push_back(rng(ws, ws_needed, "workspace"));
  if (coeffs && nodes * nseg > 0) written.push_back(rng(coeffs, nodes * nseg * 2 * sizeof(double), "coeffs"));
  if (stats && nodes * nseg > 0) written.push_back(rng(stats, nodes * nseg * 3 * sizeof(double), "stats"));
  if (ortho && nseg > 0) written.push_back(rng(ortho, (size_t)nseg * sizeof(double), "ortho"));
  for (size_t i = 0; i < written.size(); ++i) {
    for (size_t j = i + 1; j < written.size(); ++j) {
      if (overlaps(written[i], written[j])) {
        snprintf(buf, sizeof buf, "%s overlaps %s", written[i].name, written[j].name);
        return fail(ADASUM_EINVAL, buf);
      }
    }
    if (vec_bytes == 0) continue;
    for (int k = 0; k < K; ++k) {
      if (overlaps(written[i], rng(grads[k], vec_bytes, "input"))) {
        snprintf(buf, sizeof buf, "%s overlaps input grads[%d]", written[i].name, k);
        return fail(ADASUM_EINVAL, buf);
      }
    }
  }
  return ADASUM_OK;
}

// Checks that p is device memory of `device` and, where the runtime can
// tell the allocation's extent, that [p, p + bytes) lies inside it (a host
// pointer, or a buffer on another GPU, would otherwise fault inside a
// kernel).  Failed queries are cleared so that they cannot surface later as
// the error of a launch.
int check_device_range(const void* p, size_t bytes, const char* name, int device) {
  char buf[200];
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    snprintf(buf, sizeof buf, "%s is not device memory known to the HIP runtime", name);
    return fail(ADASUM_EINVAL, buf);
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) {
    snprintf(buf, sizeof buf, "%s is not device memory (memory type %d)", name, (int)attr.type);
    return fail(ADASUM_EINVAL, buf);
  }
  if (attr.type == hipMemoryTypeDevice && attr.device != device) {
    snprintf(buf, sizeof buf, "%s is on device %d but the call runs on device %d", name, attr.device, device);
    return fail(ADASUM_EINVAL, buf);
  }
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();  // extent unknown (e.g. virtually mapped memory): nothing more to check
    return ADASUM_OK;
  }
  const uintptr_t lo = reinterpret_cast<uintptr_t>(base), end = lo + size;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (a < lo || a + bytes > end) {
    snprintf(buf, sizeof buf, "%s: %zu bytes from this address run past the end of its allocation", name, bytes);
    return fail(ADASUM_EINVAL, buf);
  }
  return ADASUM_OK;
}

// Every caller buffer of a combine or sum call, on the current device.
int check_devices(const void* const* grads, int K, size_t vec_bytes, const void* out, const void* ws,
                  size_t ws_needed, const double* coeffs, const double* stats, const double* ortho, size_t nodes,
                  int nseg, int device) {
  char name[32];
  int rc = ADASUM_OK;
  if (vec_bytes > 0) {
    for (int k = 0; k < K && rc == ADASUM_OK; ++k) {
      snprintf(name, sizeof name, "grads[%d]", k);
      rc = check_device_range(grads[k], vec_bytes, name, device);
    }
    if (rc == ADASUM_OK) rc = check_device_range(out, vec_bytes, "out", device);
  }
  if (rc == ADASUM_OK && ws != nullptr && ws_needed > 0) rc = check_device_range(ws, ws_needed, "workspace", device);
  if (rc == ADASUM_OK && coeffs && nodes * nseg > 0)
    rc = check_device_range(coeffs, nodes * nseg * 2 * sizeof(double), "coeffs", device);
  if (rc == ADASUM_OK && stats && nodes * nseg > 0)
    rc = check_device_range(stats, nodes * nseg * 3 * sizeof(double), "stats", device);
  if (rc == ADASUM_OK && ortho && nseg > 0) rc = check_device_range(ortho, (size_t)nseg * sizeof(double), "ortho", device);
  return rc;
}

// ---------------------------------------------------------------- scheduler

void* ref_ptr(const Plan& p, const CallBuffers& b, Ref r) {
  switch (r.kind) {
    case Ref::Input: return const_cast<void*>(b.grads[r.idx]);
    case Ref::Slot: return b.ws + p.ws_slots + (size_t)r.idx * (size_t)p.N * sizeof(double);
    case Ref::Out: return b.out;
  }
  return nullptr;
}

DType ref_type(const Plan& p, Ref r) { return r.kind == Ref::Slot ? DType::F64 : p.dtype; }

// The kernels a block needs: its operands' type (the inputs' dtype in the
// first stage, F64 once it reads a slot) and, for a block over slots, which
// operands are inputs carried up (read in the inputs' dtype).
struct BlockKind {
  DType in_t;
  uint32_t narrow;  // bit k: operand k is an input (only with in_t == F64)
};

BlockKind block_kind(const Plan& p, const Block& b) {
  bool any_slot = false;
  for (const Ref& r : b.operands) any_slot |= r.kind == Ref::Slot;
  if (!any_slot) return {p.dtype, 0u};
  BlockKind k{DType::F64, 0u};
  for (size_t i = 0; i < b.operands.size(); ++i)
    if (b.operands[i].kind == Ref::Input) k.narrow |= 1u << i;
  return k;
}

// A small combine (Plan::fused: one stage of one block, at most kArgOps
// operands): the Gram pass, then the walk and weighted sum in one launch,
// both with one-job arguments.  Such combines are bound by the host's cost
// of their launches.
int enqueue_fused(const Plan& p, const DeviceTables& dt, const CallBuffers& b, hipStream_t st) {
  const int ntiles = (int)p.tiles.size();
  const Block& bk = p.stages[0].blocks[0];
  const BlockDesc& d = p.descs[bk.desc];
  const int nbt = d.nbt;
  double* partials = reinterpret_cast<double*>(b.ws + p.ws_partials);
  double* partials_lo = reinterpret_cast<double*>(b.ws + p.ws_plo);
  uint32_t* flags = reinterpret_cast<uint32_t*>(b.ws + p.ws_flags);
  GramArgs1 g{};
  WsumArgs1 w{};
  for (size_t k = 0; k < bk.operands.size(); ++k) g.x[k] = w.x[k] = ref_ptr(p, b, bk.operands[k]);
  const double in_bytes = (double)p.N * dtype_size(p.dtype) * bk.operands.size();
  g.poff[0] = d.poff;
  g.tiles = dt.tiles;
  g.partials = partials;
  g.partials_lo = partials_lo;
  g.flags = flags;
  g.wrow[0] = d.wrow;
  g.nseg = p.nseg;
  g.short_tiles = p.tile_rows <= kMinTile;
  const double gbytes = in_bytes + 8.0 * gram_entries(nbt) * ntiles;
  log_launch("gram", 1, ntiles, 1, nbt, gbytes);
  const int pg = prof_start(kGram, gbytes, st);
  hipError_t e = launch_gram1(p.dtype, nbt, g, ntiles, st);
  prof_stop(pg, st);
  if (e != hipSuccess) return fail_hip(e, "launching gram");

  TreeArgs t{};
  t.descs = dt.descs;
  t.merges = dt.merges;
  t.seg_tile = dt.seg_tile;
  t.partials = partials;
  t.partials_lo = partials_lo;
  t.tiles = dt.tiles;
  t.lo_inputs = p.dtype != DType::F32;
  t.desc0 = bk.desc;
  t.nblocks = 1;
  t.nseg = p.nseg;
  t.weights = reinterpret_cast<double*>(b.ws + p.ws_weights);
  t.weights_lo = reinterpret_cast<double*>(b.ws + p.ws_weights_lo);
  t.coeffs = b.coeffs;
  t.stats = b.stats;
  t.ortho = b.ortho;
  t.leafnorm = reinterpret_cast<double*>(b.ws + p.ws_leafnorm);
  t.nblocks_total = p.nblocks;
  t.flags = flags;
  w.y[0] = ref_ptr(p, b, bk.dst);
  w.wrow[0] = d.wrow;
  w.tiles = dt.tiles;
  w.nseg = p.nseg;
  w.weights = t.weights;
  w.weights_lo = t.weights_lo;
  w.flags = flags;
  const double wbytes = in_bytes + (double)p.N * dtype_size(p.dtype);
  log_launch("walk+wsum", 1, ntiles, 1, nbt, wbytes);
  const int pw = prof_start(kWsum, wbytes, st);
  e = launch_fused(p.dtype, nbt, t, w, ntiles, st);
  prof_stop(pw, st);
  if (e != hipSuccess) return fail_hip(e, "launching the fused walk and weighted sum");
  return ADASUM_OK;
}

int enqueue(const Plan& p, const DeviceTables& dt, const CallBuffers& b, hipStream_t st) {
  if (p.fused) return enqueue_fused(p, dt, b, st);
  const int ntiles = (int)p.tiles.size();
  hipError_t e;
  double* partials = reinterpret_cast<double*>(b.ws + p.ws_partials);
  double* partials_lo = reinterpret_cast<double*>(b.ws + p.ws_plo);
  double* weights = reinterpret_cast<double*>(b.ws + p.ws_weights);
  double* weights_lo = reinterpret_cast<double*>(b.ws + p.ws_weights_lo);
  uint32_t* flags = reinterpret_cast<uint32_t*>(b.ws + p.ws_flags);
  int stage_no = 0;
  for (const Stage& sg : p.stages) {
    ++stage_no;
    TreeArgs t{};
    t.descs = dt.descs;
    t.merges = dt.merges;
    t.seg_tile = dt.seg_tile;
    t.partials = partials;
    t.partials_lo = partials_lo;
    t.tiles = dt.tiles;
    t.lo_inputs = p.dtype != DType::F32;
    t.desc0 = sg.blocks.front().desc;
    t.nblocks = (int)sg.blocks.size();
    t.nseg = p.nseg;
    t.weights = weights;
    t.weights_lo = weights_lo;
    t.coeffs = b.coeffs;
    t.stats = b.stats;
    t.ortho = b.ortho;
    t.leafnorm = reinterpret_cast<double*>(b.ws + p.ws_leafnorm);
    t.nblocks_total = p.nblocks;
    for (const Block& bk : sg.blocks) t.wide |= p.descs[bk.desc].nbt > kArgOps ? 1 : 0;
    if (ntiles == 0) {  // every segment empty: coefficients 1, statistics 0
      if (p.nseg > 0) {
        e = launch_tree(t, st);
        if (e != hipSuccess) return fail_hip(e, "launching tree");
      }
      continue;
    }
    // The Gram launches of this stage, kept for the exact recomputation of
    // flagged (block, segment) pairs
    struct GramLaunch {
      GramArgs args;
      DType in_t;
      int nbt, njobs;
    };
    std::vector<GramLaunch> grams;
    // 1. Gram partials, blocks grouped by (operand type, Gram size)
    // 3. weighted sums, grouped by (operand type, Gram size, result type)
    for (int pass = 0; pass < 2; ++pass) {
      std::vector<char> done(sg.blocks.size(), 0);
      for (size_t i = 0; i < sg.blocks.size(); ++i) {
        if (done[i]) continue;
        const Block& b0 = sg.blocks[i];
        const DType in_t = block_kind(p, b0).in_t;
        const DType out_t = ref_type(p, b0.dst);
        const int nbt = p.descs[b0.desc].nbt;
        std::vector<const Block*> group;
        for (size_t k = i; k < sg.blocks.size(); ++k) {
          const Block& bk = sg.blocks[k];
          if (done[k] || p.descs[bk.desc].nbt != nbt || block_kind(p, bk).in_t != in_t) continue;
          if (pass == 1 && ref_type(p, bk.dst) != out_t) continue;
          done[k] = 1;
          group.push_back(&bk);
        }
        const int per_launch = max_jobs(nbt);
        for (size_t c = 0; c < group.size(); c += per_launch) {
          const int n = (int)std::min<size_t>(per_launch, group.size() - c);
          double in_bytes = 0, out_bytes = 0;
          if (pass == 0) {
            GramArgs a{};
            for (int j = 0; j < n; ++j) {
              const Block& bk = *group[c + j];
              for (size_t k = 0; k < bk.operands.size(); ++k) {
                a.x[j * op_stride(nbt) + k] = ref_ptr(p, b, bk.operands[k]);
                in_bytes += (double)p.N * dtype_size(ref_type(p, bk.operands[k]));
              }
              a.narrow[j] = block_kind(p, bk).narrow;
              a.poff[j] = p.descs[bk.desc].poff;
              a.wrow[j] = p.descs[bk.desc].wrow;
              out_bytes += 8.0 * gram_entries(nbt) * ntiles;
            }
            a.tiles = dt.tiles;
            a.partials = partials;
            a.partials_lo = partials_lo;
            a.flags = flags;
            a.nseg = p.nseg;
            a.short_tiles = p.tile_rows <= kMinTile;
            log_launch("gram", stage_no, ntiles, n, nbt, in_bytes + out_bytes);
            const int pr = prof_start(kGram, in_bytes + out_bytes, st);
            e = launch_gram(in_t, p.dtype, nbt, a, ntiles, n, st);
            prof_stop(pr, st);
            if (e != hipSuccess) return fail_hip(e, "launching gram");
            grams.push_back(GramLaunch{a, in_t, nbt, n});
          } else {
            WsumArgs a{};
            for (int j = 0; j < n; ++j) {
              const Block& bk = *group[c + j];
              for (size_t k = 0; k < bk.operands.size(); ++k) {
                a.x[j * op_stride(nbt) + k] = ref_ptr(p, b, bk.operands[k]);
                in_bytes += (double)p.N * dtype_size(ref_type(p, bk.operands[k]));
              }
              a.narrow[j] = block_kind(p, bk).narrow;
              a.y[j] = ref_ptr(p, b, bk.dst);
              a.wrow[j] = p.descs[bk.desc].wrow;
              out_bytes += (double)p.N * dtype_size(out_t);
            }
            a.tiles = dt.tiles;
            a.nseg = p.nseg;
            a.weights = weights;
            a.weights_lo = weights_lo;
            a.flags = flags;
            log_launch("wsum", stage_no, ntiles, n, nbt, in_bytes + out_bytes);
            const int pr = prof_start(kWsum, in_bytes + out_bytes, st);
            e = launch_wsum(in_t, p.dtype, nbt, out_t, a, ntiles, n, st);
            prof_stop(pr, st);
            if (e != hipSuccess) return fail_hip(e, "launching wsum");
          }
        }
      }
      if (pass == 0 && p.nseg > 0) {
        // 2. per (block, segment): statistics, coefficients, operand weights,
        // and a flag on every pair whose coefficients the rounding of its
        // Gram entries could move beyond tolerance (a merge under deep
        // cancellation); those pairs' tiles are then recomputed exactly and
        // walked again
        t.flags = flags;
        t.grouped = p.descs[sg.blocks.front().desc].nbt > kArgOps || p.tile_groups;
        if (t.grouped) {
          // 64-operand blocks (a stage of their own), or segments of many
          // tiles: the walk reads tile-group sums, formed over many workgroups
          double gbytes = 0;
          for (const Block& bk : sg.blocks) gbytes += 8.0 * gram_entries(p.descs[bk.desc].nbt) * ntiles;
          log_launch("groups", stage_no, ntiles, t.nblocks, 0, gbytes);
          const int pg = prof_start(kTree, gbytes, st);
          e = launch_tile_groups(t, ntiles, st);
          prof_stop(pg, st);
          if (e != hipSuccess) return fail_hip(e, "launching tile groups");
        }
        double bytes = 0;
        for (const Block& bk : sg.blocks) bytes += 8.0 * gram_entries(p.descs[bk.desc].nbt) * ntiles;
        log_launch("tree", stage_no, t.nblocks * p.nseg, 1, 0, bytes);
        const int pr = prof_start(kTree, bytes, st);
        e = launch_tree(t, st);
        prof_stop(pr, st);
        if (e != hipSuccess) return fail_hip(e, "launching tree");
        for (const GramLaunch& g : grams) {
          // algorithmic bytes: the flag of every tile (flagged tiles, none in
          // the usual case, also re-read their operands)
          const double fbytes = 4.0 * ntiles * g.njobs;
          log_launch("exact", stage_no, ntiles, g.njobs, g.nbt, fbytes);
          const int pe = prof_start(kExact, fbytes, st);
          e = launch_gram_exact(g.in_t, p.dtype, g.nbt, g.args, ntiles, g.njobs, st);
          prof_stop(pe, st);
          if (e != hipSuccess) return fail_hip(e, "launching exact gram");
        }
        TreeArgs r = t;
        r.refine = 1;
        const double rbytes = 4.0 * t.nblocks * p.nseg;  // the flags
        log_launch("tree", stage_no, t.nblocks * p.nseg, 1, 0, rbytes);
        const int pt = prof_start(kTree, rbytes, st);
        e = launch_tree(r, st);
        prof_stop(pt, st);
        if (e != hipSuccess) return fail_hip(e, "launching tree");
      }
    }
  }
  return ADASUM_OK;
}

int combine_impl(const void* const* grads, int K, const int64_t* seg_offsets, int nseg, int dtype, int schedule,
                 void* out, void* workspace, size_t workspace_bytes, double* coeffs, double* stats,
                 double* ortho, void* stream, bool owned_workspace) {
  std::string err;
  if (!validate_shape(K, seg_offsets, nseg, dtype, schedule, &err)) return fail(ADASUM_EINVAL, err);
  const DType dt = static_cast<DType>(dtype);
  const Schedule sc = static_cast<Schedule>(schedule);
  const int64_t N = seg_offsets[nseg];

  std::lock_guard<std::mutex> lock(g_mu);
  std::shared_ptr<CachedPlan> cp = find_plan(K, seg_offsets, nseg, dt, sc);
  const Plan& p = cp->plan;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int device = 0;

  if (owned_workspace) {
    int rc = validate_buffers(grads, K, N, dtype_size(dt), nseg, out, nullptr, 0, 0, nullptr, nullptr, nullptr);
    if (rc != ADASUM_OK) return rc;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    rc = check_devices(grads, K, (size_t)N * dtype_size(dt), out, nullptr, 0, nullptr, nullptr, nullptr, 0, nseg,
                       device);
    if (rc != ADASUM_OK) return rc;
    OwnedWorkspace& ow = g_ws[{device, stream}];
    const bool cap = capturing(st);
    if (ow.bytes < p.ws_total) {
      if (cap)
        return fail(ADASUM_EINVAL, "adasum_combine would allocate its workspace while the stream is being captured "
                                   "into a graph; make one call of this shape on this stream before capturing");
      if (ow.ptr) {
        e = hipStreamSynchronize(st);  // earlier calls on this stream may still use the old buffer
        if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize before growing the workspace");
        if (!ow.captured) (void)hipFree(ow.ptr);  // else a captured graph may still use it: kept
        ow.ptr = nullptr;
        ow.bytes = 0;
        ow.captured = false;
      }
      e = hipMalloc(&ow.ptr, p.ws_total);
      if (e != hipSuccess) {
        ow.ptr = nullptr;
        return fail(ADASUM_ENOMEM, "hipMalloc of the library workspace failed");
      }
      ow.bytes = p.ws_total;
    }
    if (cap) ow.captured = true;
    workspace = ow.ptr;
    workspace_bytes = ow.bytes;
    // inputs and out were checked above; the library buffer cannot alias them
  } else {
    int rc = validate_buffers(grads, K, N, dtype_size(dt), nseg, out, workspace, workspace_bytes, p.ws_total,
                              coeffs, stats, ortho);
    if (rc != ADASUM_OK) return rc;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    rc = check_devices(grads, K, (size_t)N * dtype_size(dt), out, workspace, p.ws_total, coeffs, stats, ortho,
                       K > 1 ? (size_t)(K - 1) : 0, nseg, device);
    if (rc != ADASUM_OK) return rc;
  }

  DeviceTables tables;
  if (capturing(st)) {
    if (cp->per_device.find(device) == cp->per_device.end())
      return fail(ADASUM_EINVAL, "the first call of a shape uploads its tables and may not be captured into a "
                                 "graph; make one call of this shape before capturing");
    cp->pinned = true;  // the graph refers to this shape's tables from now on
  }
  int rc = device_tables(*cp, device, &tables);
  if (rc != ADASUM_OK) return rc;
  char* ws = static_cast<char*>(workspace);
  CallBuffers b;
  b.grads = grads;
  b.out = out;
  b.ws = ws;
  b.coeffs = coeffs ? coeffs : reinterpret_cast<double*>(ws + p.ws_coeffs);
  b.stats = stats ? stats : reinterpret_cast<double*>(ws + p.ws_stats);
  b.ortho = ortho;
  return enqueue(p, tables, b, st);
}

}  // namespace adasum

extern "C" {

int adasum_combine(const void* const* grads, int K, const int64_t* seg_offsets, int nseg, int dtype, void* out,
                   void* stream) {
  return adasum::combine_impl(grads, K, seg_offsets, nseg, dtype, int(adasum::Schedule::Tree), out, nullptr, 0,
                              nullptr, nullptr, nullptr, stream, true);
}

int64_t adasum_workspace_bytes(int K, const int64_t* seg_offsets, int nseg, int dtype, int schedule) {
  std::string err;
  if (!adasum::validate_shape(K, seg_offsets, nseg, dtype, schedule, &err))
    return adasum::fail(ADASUM_EINVAL, err);
  std::lock_guard<std::mutex> lock(adasum::g_mu);
  return (int64_t)adasum::find_plan(K, seg_offsets, nseg, static_cast<adasum::DType>(dtype),
                                    static_cast<adasum::Schedule>(schedule))
      ->plan.ws_total;
}

int adasum_combine_ex(const void* const* grads, int K, const int64_t* seg_offsets, int nseg, int dtype,
                      int schedule, void* out, void* workspace, size_t workspace_bytes, double* coeffs,
                      double* stats, double* ortho, void* stream) {
  return adasum::combine_impl(grads, K, seg_offsets, nseg, dtype, schedule, out, workspace, workspace_bytes, coeffs,
                              stats, ortho, stream, false);
}

int64_t adasum_sum_workspace_bytes(int K, int64_t N, int dtype) {
  using namespace adasum;
  if (K < 1 || N < 0 || (dtype != int(DType::F32) && dtype != int(DType::F16) && dtype != int(DType::BF16)))
    return fail(ADASUM_EINVAL, "adasum_sum_workspace_bytes: K >= 1, N >= 0 and a known dtype are required");
  // more operands than one launch holds: an fp64 running sum between launches
  return K <= kSumOps ? 0 : N * (int64_t)sizeof(double);
}

int adasum_sum(const void* const* grads, int K, int64_t N, int dtype, void* out, void* workspace,
               size_t workspace_bytes, void* stream) {
  using namespace adasum;
  const int64_t need = adasum_sum_workspace_bytes(K, N, dtype);
  if (need < 0) return (int)need;
  const int64_t off[2] = {0, N};
  std::string err;
  if (!validate_shape(K, off, 1, dtype, 0, &err)) return fail(ADASUM_EINVAL, err);
  const DType dt = static_cast<DType>(dtype);
  int rc = validate_buffers(grads, K, N, dtype_size(dt), 0, out, workspace, workspace_bytes, (size_t)need,
                            nullptr, nullptr, nullptr);
  if (rc != ADASUM_OK) return rc;
  if (N == 0) return ADASUM_OK;
  int device = 0;
  hipError_t de = hipGetDevice(&device);
  if (de != hipSuccess) return fail_hip(de, "hipGetDevice");
  rc = check_devices(grads, K, (size_t)N * dtype_size(dt), out, workspace, (size_t)need, nullptr, nullptr, nullptr, 0,
                     0, device);
  if (rc != ADASUM_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_mu);
  double* acc = static_cast<double*>(workspace);
  for (int k0 = 0; k0 < K; k0 += kSumOps) {
    SumArgs a{};
    a.nx = std::min(kSumOps, K - k0);
    for (int i = 0; i < a.nx; ++i) a.x[i] = grads[k0 + i];
    a.acc_in = k0 > 0 ? acc : nullptr;
    const bool final_launch = k0 + kSumOps >= K;
    a.acc_out = final_launch ? nullptr : acc;
    a.out = out;
    a.n = N;
    const double bytes = (double)N * (a.nx * dtype_size(dt) + (a.acc_in ? 8.0 : 0.0) +
                                      (final_launch ? dtype_size(dt) : 8.0));
    const int pr = prof_start(kSum, bytes, st);
    hipError_t e = launch_sum(dt, a, st);
    prof_stop(pr, st);
    if (e != hipSuccess) return fail_hip(e, "launching sum");
  }
  return ADASUM_OK;
}

int adasum_profile_begin(void) {
  std::lock_guard<std::mutex> lock(adasum::g_mu);
  for (auto& r : adasum::g_prof) adasum::g_ev_pool.push_back({r.start, r.stop});
  adasum::g_prof.clear();
  adasum::g_prof_on = true;
  return ADASUM_OK;
}

int adasum_profile_end(adasum_kernel_time_t* rows, int max_rows) {
  using namespace adasum;
  std::lock_guard<std::mutex> lock(g_mu);
  g_prof_on = false;
  if (max_rows < 0 || (max_rows > 0 && rows == nullptr))
    return fail(ADASUM_EINVAL, "rows must hold max_rows >= 0 entries");
  int launches[kNumKinds] = {0};
  double ms[kNumKinds] = {0}, bytes[kNumKinds] = {0};
  int rc = ADASUM_OK;
  for (auto& r : g_prof) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess) rc = fail_hip(e, "reading profile events");
    launches[r.kind] += 1;
    ms[r.kind] += t;
    bytes[r.kind] += r.bytes;
    g_ev_pool.push_back({r.start, r.stop});
  }
  g_prof.clear();
  if (rc != ADASUM_OK) return rc;
  int n = 0;
  for (int k = 0; k < kNumKinds; ++k) {
    if (launches[k] == 0) continue;
    if (n < max_rows) {
      std::memset(&rows[n], 0, sizeof(rows[n]));
      std::strncpy(rows[n].kernel, kKindNames[k], sizeof(rows[n].kernel) - 1);
      rows[n].launches = launches[k];
      rows[n].milliseconds = ms[k];
      rows[n].bytes = bytes[k];
    }
    ++n;
  }
  return n < max_rows ? n : max_rows;
}

const char* adasum_strerror(int code) {
  switch (code) {
    case ADASUM_OK: return "success";
    case ADASUM_EINVAL: return "invalid argument";
    case ADASUM_ENOMEM: return "out of memory";
    case ADASUM_EHIP: return "HIP runtime error";
  }
  return "unknown error code";
}

const char* adasum_last_error(void) { return adasum::g_last_error.c_str(); }

int adasum_version(void) { return 100; }

}  // extern "C"
