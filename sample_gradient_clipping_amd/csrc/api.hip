// C ABI of libdpfused: argument checks, path choice, workspace, launches.
//
// Every entry point validates all of its arguments before queueing anything:
// a failed check launches nothing and writes nothing.  Workspace (per-sample
// norm partials, clip factors, mask row-activity bits, the projected
// activations) comes from a per-device cache of blocks, each ordered after
// its previous use by an event, backed by a per-device memory pool; the
// staged per-sample gradient tiles have a per-device buffer of their own.
#include <hip/hip_runtime.h>

#include <atomic>
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "dpfused.h"
#include "kernels.hpp"

// Static scratch of dpfused_linear_clip_accumulate_noalloc, for callers that
// cannot allocate (graph capture, tight serving loops): 80 MiB, which holds
// a Llama-13B-sized linear's workspace without split tiles (the Gram
// kernel's parked blocks, 64 MiB on 256 compute units, plus norm partials,
// clip factors and mask bits).  Each device holds its own copy, at its own
// address, until the process ends.
constexpr size_t kScratchBytes = (size_t)80 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;
std::atomic<int> g_norm_path{0};   // 0 auto, 1 gram, 2 direct, 3 staged
std::atomic<int> g_timing{0};
std::atomic<int> g_trace{0};        // roctx range around every entry point
std::atomic<int> g_debug{0};        // synchronise after every launch, report errors
std::atomic<int64_t> g_ws_limit{0};   // workspace requests above this fail (0: no limit)
std::atomic<int> g_onepass_spin{1 << 20};   // single pass: tries of a blocking wait
std::atomic<int> g_onepass_never{0};        // single pass: testing, every wait gives up

// Defaults from the environment, read once when the library is loaded:
// DPFUSED_NORM_PATH (auto, gram, direct, staged, onepass or 0-4), DPFUSED_TRACE,
// DPFUSED_DEBUG (0/1), DPFUSED_WS_LIMIT (bytes).
bool read_env() {
  if (const char* v = std::getenv("DPFUSED_NORM_PATH")) {
    const std::string t(v);
    const int path = t == "gram" ? 1 : t == "direct" ? 2 : t == "staged" ? 3
                   : t == "onepass" ? 4
                   : (t.size() == 1 && t[0] >= '0' && t[0] <= '4') ? t[0] - '0' : 0;
    g_norm_path.store(path);
  }
  if (const char* v = std::getenv("DPFUSED_TRACE")) g_trace.store(std::atoi(v) != 0);
  if (const char* v = std::getenv("DPFUSED_DEBUG")) g_debug.store(std::atoi(v) != 0);
  if (const char* v = std::getenv("DPFUSED_WS_LIMIT")) {
    const long long n = std::atoll(v);
    g_ws_limit.store(n > 0 ? (int64_t)n : 0);
  }
  return true;
}
const bool g_env_read = read_env();

bool over_limit(size_t bytes) {
  const int64_t lim = g_ws_limit.load();
  return lim > 0 && (int64_t)bytes > lim;
}

// A roctx range named after the entry point, when the trace option is on.
struct TraceRange {
  bool on;
  explicit TraceRange(const char* name) : on(g_trace.load() != 0) {
    if (on) roctxRangePushA(name);
  }
  ~TraceRange() {
    if (on) roctxRangePop();
  }
};

dpf_status fail(dpf_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

dpf_status ok() {
  g_last_error.clear();
  return DPF_OK;
}

size_t elem_size(int dtype) { return dtype == DPF_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// Timing registry
// ---------------------------------------------------------------------------
struct Pending {
  std::string name;
  hipEvent_t start = nullptr, stop = nullptr;
};
struct Total {
  std::string name;
  double ms = 0.0;
  int64_t n = 0;
};
std::mutex g_tmu;
std::vector<Pending> g_pending;
std::vector<Total> g_totals;

// ---------------------------------------------------------------------------
// Argument checks
// ---------------------------------------------------------------------------
constexpr int64_t kMaxDim = (int64_t)1 << 30;

dpf_status check_act(const dpf_act* a, const char* name) {
  if (a == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, std::string(name) + " is NULL");
  if (a->data == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, std::string(name) + ".data is NULL");
  if (a->dtype != DPF_F32 && a->dtype != DPF_BF16)
    return fail(DPF_ERR_UNSUPPORTED, std::string(name) + ".dtype is not DPF_F32 or DPF_BF16");
  if (a->reserved != 0) return fail(DPF_ERR_UNSUPPORTED, std::string(name) + ".reserved must be 0");
  if (a->B < 1 || a->T < 1 || a->D < 1)
    return fail(DPF_ERR_INVALID_ARGUMENT, std::string(name) + ": B, T and D must be >= 1");
  if (a->B > kMaxDim || a->T > kMaxDim || a->D > kMaxDim || a->B * a->T > ((int64_t)1 << 40))
    return fail(DPF_ERR_UNSUPPORTED, std::string(name) + ": dimension too large");
  if (a->stride_t < a->D)
    return fail(DPF_ERR_INVALID_ARGUMENT, std::string(name) + ".stride_t < D (rows overlap)");
  if (a->stride_b < (a->T - 1) * a->stride_t + a->D)
    return fail(DPF_ERR_INVALID_ARGUMENT, std::string(name) + ".stride_b too small (samples overlap)");
  if (!aligned16(a->data))
    return fail(DPF_ERR_UNSUPPORTED, std::string(name) + ".data is not 16-byte aligned");
  return DPF_OK;
}

dpf_status check_pair(const dpf_act* X, const dpf_act* G) {
  dpf_status s = check_act(X, "X");
  if (s != DPF_OK) return s;
  s = check_act(G, "G");
  if (s != DPF_OK) return s;
  if (X->dtype != G->dtype) return fail(DPF_ERR_UNSUPPORTED, "X and G have different dtypes");
  if (X->B != G->B || X->T != G->T)
    return fail(DPF_ERR_INVALID_ARGUMENT, "X and G disagree on B or T");
  return DPF_OK;
}

bool vec_ok(const dpf_act* a) {
  const size_t es = elem_size(a->dtype);
  return aligned16(a->data) && (a->D * es) % 16 == 0 && (a->stride_t * es) % 16 == 0 &&
         (a->stride_b * es) % 16 == 0;
}

dpf::Act to_act(const dpf_act* a) { return dpf::Act{a->data, a->stride_b, a->stride_t}; }

// Largest staged workspace (B per-sample gradient tiles, fp32) a call may use.
constexpr double kStagedMaxBytes = 16.0 * (1ull << 30);

// The norm path of one call.  The automatic choice is always one of the two
// forms that never store a per-sample gradient: the Gram identity or the
// direct form (each g_i tile computed and dropped).  The staged form, which
// keeps every g_i tile in device memory between the norm and accumulate
// phases, runs only when the "norm_path" option asks for it.
//
// allow_staged: the caller can keep the per-sample tiles from the norm phase
// to the accumulate phase (the single-layer calls, and group clipping, which
// holds every linear's tiles until the group's clip factors exist).
// The single-pass kernel runs one workgroup per 128 x 128 output tile, all
// resident at once (a cooperative launch), on the large-tile layout.
bool onepass_ok(const dpf::LayerArgs& a, bool vec) {
  if (!dpf::big_path(a, vec) || a.B > 65535) return false;
  const int nt = dpf::onepass_tiles(a.din, a.dout);
  return nt <= 256 && nt <= dpf::onepass_resident_limit();
}

dpf::NormPath choose_path(const dpf::LayerArgs& a, bool vec, bool allow_staged,
                          bool allow_onepass = false) {
  const bool big = dpf::big_path(a, vec);
  const int forced = g_norm_path.load();
  if (forced == 4 && allow_onepass && onepass_ok(a, vec)) return dpf::NormPath::kOnePass;
  if (forced == 1) return dpf::NormPath::kGram;
  if (forced == 2) return dpf::NormPath::kDirect;
  if (forced == 3) {
    const bool staged_ok = allow_staged && big &&
                           (double)dpf::staged_big_workspace_bytes(a) <= kStagedMaxBytes &&
                           (double)a.B * dpf::big_tiles(a.din, a.dout) < 2147483647.0;
    return staged_ok ? dpf::NormPath::kStaged : dpf::NormPath::kDirect;
  }
  const double T = a.T, din = a.din, dout = a.dout;
  const double direct = 2.0 * T * din * dout;   // flops per sample
  if (big) {
    // The large-tile Gram kernel works on 256 x 256 token blocks (padded),
    // with a fixed cost per block (two pipeline fills, a parked X Gram):
    // measured on MI355X it beats the direct kernel once it needs at most
    // half the direct kernel's flops.
    const double gram = 2.0 * dpf::gram_big_items_per_sample(a.T) * 65536.0 * (din + dout);
    return 2.0 * gram <= direct ? dpf::NormPath::kGram : dpf::NormPath::kDirect;
  }
  // Gram costs T^2 (din + dout) per sample, the direct form 2 T din dout.
  return T * T * (din + dout) <= direct ? dpf::NormPath::kGram : dpf::NormPath::kDirect;
}

// Per-device stream-ordered memory pool for workspace (everything but the
// staged tiles, which are taken apart from it below).  It keeps up to
// g_keep_bytes reserved across synchronisations (the default pool returns
// freed memory at every synchronisation), so workspace is not mapped afresh
// on every step.  The default, 512 MiB, is about twice the workspace of the
// largest Llama-13B-layer call (a 5120 x 5120 linear at B = 8, T = 2048:
// split-tile partials of the accumulate and Gram kernels plus the norm
// partials), so the calls of one layer step reuse blocks.
std::atomic<int64_t> g_keep_bytes{(int64_t)512 << 20};
// Bytes of staged per-sample tiles kept for the next call; 0 (the default):
// the tiles are given back at the end of every call.
std::atomic<int64_t> g_staged_keep{0};
// Device memory one call takes beyond its inputs and outputs (workspace plus
// staged tiles): the last call on this thread, and the most since reset.
thread_local int64_t t_call_bytes = 0;
std::atomic<int64_t> g_call_high{0};
void note_call_bytes(size_t bytes) {
  t_call_bytes += (int64_t)bytes;
  int64_t h = g_call_high.load();
  while (t_call_bytes > h && !g_call_high.compare_exchange_weak(h, t_call_bytes)) {
  }
}

// Starts the per-call memory count, and the roctx range of the entry point
// when the trace option is on.
struct CallScope {
  TraceRange range;
  explicit CallScope(const char* name) : range(name) { t_call_bytes = 0; }
};
std::mutex g_pool_mu;
constexpr int kMaxDevices = 64;
hipMemPool_t g_pools[kMaxDevices] = {};
bool g_pool_tried[kMaxDevices] = {};

int stream_device(hipStream_t s) {
  int dev = -1;
  if (s != nullptr) {
    hipDevice_t d;
    if (hipStreamGetDevice(s, &d) == hipSuccess) dev = (int)d;
  }
  if (dev < 0 && hipGetDevice(&dev) != hipSuccess) dev = -1;
  return dev;
}

bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return true;   // state unknown: take the path that is safe under capture
  }
  return cs != hipStreamCaptureStatusNone;
}

hipMemPool_t workspace_pool(hipStream_t s) {
  const int dev = stream_device(s);
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_pool_mu);
  if (!g_pool_tried[dev]) {
    g_pool_tried[dev] = true;
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &props) == hipSuccess) {
      uint64_t keep = (uint64_t)g_keep_bytes.load();
      (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
      g_pools[dev] = pool;
    } else {
      (void)hipGetLastError();   // fall back to hipMallocAsync's default pool
    }
  }
  return g_pools[dev];
}

// The staged per-sample tiles (up to gigabytes, staged path only) are taken
// for one call and given back at its end: stream-ordered hipMallocAsync /
// hipFreeAsync on the call's stream.  With the "staged_keep_bytes" option
// above 0 a buffer of up to that size is kept per device for the next call
// instead (pool allocations of that size, freed and made again by calls on
// several streams, were measured to stall for tens of milliseconds on
// MI355X).  Calls on any stream take a kept buffer in turn: each one's
// stream first waits (on the GPU) for the event recorded after the previous
// holder's last use, and records its own after its last launch.  A stream
// being captured into a graph never uses the kept buffer (its events are
// recorded outside the capture): it takes capture-local memory.
struct StagedBuffer {
  std::mutex mu;
  void* ptr = nullptr;
  size_t size = 0;
  hipEvent_t last = nullptr;
  bool recorded = false;
};
StagedBuffer g_staged[kMaxDevices];

class StagedLease {
 public:
  ~StagedLease() { release(); }
  // Holds at least `bytes` of staged tiles for work queued on `s` until
  // release(); false if they cannot be had.
  bool acquire(hipStream_t s, size_t bytes) {
    if (over_limit(bytes)) return false;
    s_ = s;
    const int dev = stream_device(s);
    if (g_staged_keep.load() <= 0 || (int64_t)bytes > g_staged_keep.load() || dev < 0 ||
        dev >= kMaxDevices || stream_capturing(s)) {
      if (hipMallocAsync(&local_, bytes, s) != hipSuccess || local_ == nullptr) {
        (void)hipGetLastError();
        local_ = nullptr;
        return false;
      }
      held_ = true;
      note_call_bytes(bytes);
      return true;
    }
    buf_ = &g_staged[dev];
    lk_ = std::unique_lock<std::mutex>(buf_->mu);
    if (buf_->last == nullptr &&
        hipEventCreateWithFlags(&buf_->last, hipEventDisableTiming) != hipSuccess) {
      buf_->last = nullptr;
      return fail_acquire();
    }
    if (buf_->recorded && hipStreamWaitEvent(s, buf_->last, 0) != hipSuccess) return fail_acquire();
    if (buf_->size < bytes) {
      if (buf_->ptr != nullptr) (void)hipFreeAsync(buf_->ptr, s);
      buf_->ptr = nullptr;
      buf_->size = 0;
      if (hipMallocAsync(&buf_->ptr, bytes, s) != hipSuccess || buf_->ptr == nullptr) {
        buf_->ptr = nullptr;
        return fail_acquire();
      }
      buf_->size = bytes;
    }
    held_ = true;
    note_call_bytes(bytes);
    return true;
  }
  void* ptr() const { return !held_ ? nullptr : local_ != nullptr ? local_ : buf_->ptr; }
  void release() {
    if (!held_) return;
    held_ = false;
    if (local_ != nullptr) {
      (void)hipFreeAsync(local_, s_);
      local_ = nullptr;
      return;
    }
    if (hipEventRecord(buf_->last, s_) == hipSuccess) buf_->recorded = true;
    if ((int64_t)buf_->size > g_staged_keep.load()) {
      (void)hipFreeAsync(buf_->ptr, s_);
      buf_->ptr = nullptr;
      buf_->size = 0;
    }
    lk_.unlock();
  }

 private:
  bool fail_acquire() {
    (void)hipGetLastError();
    lk_.unlock();
    return false;
  }
  StagedBuffer* buf_ = nullptr;
  void* local_ = nullptr;
  std::unique_lock<std::mutex> lk_;
  hipStream_t s_ = nullptr;
  bool held_ = false;
};

// Freed workspace blocks are kept for later calls: a pool allocation and its
// free cost more host time than a small call's kernel launches.  A kept block
// carries an event recorded on the stream of its last use; the next user's
// stream waits for that event on the GPU, so a block may move between streams.
// Each device keeps at most g_keep_bytes of blocks (oldest freed first).
struct CachedBlock {
  void* ptr;
  size_t size;
  hipEvent_t ev;
};
struct BlockCache {
  std::mutex mu;
  std::vector<CachedBlock> blocks;   // oldest first
  size_t bytes = 0;
  std::vector<hipEvent_t> spare;     // events of blocks given back to the pool
};
BlockCache g_cache[kMaxDevices];

// Frees cached blocks until at most `keep` bytes remain, on stream `s` after
// each block's last use (s == nullptr: wait for it on the host first).
void trim_cache(BlockCache& c, size_t keep, hipStream_t s) {
  while (c.bytes > keep && !c.blocks.empty()) {
    CachedBlock b = c.blocks.front();
    c.blocks.erase(c.blocks.begin());
    c.bytes -= b.size;
    if (s != nullptr) (void)hipStreamWaitEvent(s, b.ev, 0);
    else (void)hipEventSynchronize(b.ev);
    (void)hipFreeAsync(b.ptr, s);
    c.spare.push_back(b.ev);
  }
}

void set_keep_bytes(int64_t keep) {
  g_keep_bytes.store(keep);
  for (int d = 0; d < kMaxDevices; ++d) {
    std::lock_guard<std::mutex> lk(g_cache[d].mu);
    trim_cache(g_cache[d], (size_t)keep, nullptr);
  }
  {
    std::lock_guard<std::mutex> lk(g_pool_mu);
    for (int d = 0; d < kMaxDevices; ++d) {
      if (g_pools[d] == nullptr) continue;
      uint64_t k = (uint64_t)keep;
      (void)hipMemPoolSetAttribute(g_pools[d], hipMemPoolAttrReleaseThreshold, &k);
      (void)hipMemPoolTrimTo(g_pools[d], (size_t)keep);
    }
  }
}

void set_staged_keep(int64_t keep) {
  g_staged_keep.store(keep);
  for (int d = 0; d < kMaxDevices; ++d) {
    StagedBuffer& b = g_staged[d];
    std::lock_guard<std::mutex> lk(b.mu);
    if (b.ptr == nullptr || (int64_t)b.size <= keep) continue;
    if (b.recorded) (void)hipEventSynchronize(b.last);   // its last user is done with it
    (void)hipFreeAsync(b.ptr, nullptr);
    b.ptr = nullptr;
    b.size = 0;
  }
}

// Stream-ordered workspace carved into 256-byte aligned pieces: a kept block
// of at least the size (and at most about twice it), else a new one from the
// pool.  Given back to the cache when the call's launches are queued.
struct Workspace {
  hipStream_t s;
  void* base = nullptr;
  size_t size = 0, cap = 0;
  hipEvent_t ev = nullptr;
  int dev = -1;   // -1: not from (and not returned to) the cache
  bool external = false;   // memory the workspace does not own (the static scratch)
  explicit Workspace(hipStream_t st) : s(st) {}
  ~Workspace() {
    if (base == nullptr || external) return;
    if (dev < 0 || dev >= kMaxDevices) {
      (void)hipFreeAsync(base, s);
      return;
    }
    BlockCache& c = g_cache[dev];
    std::lock_guard<std::mutex> lk(c.mu);
    if (ev == nullptr && !c.spare.empty()) {
      ev = c.spare.back();
      c.spare.pop_back();
    }
    if (ev == nullptr && hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) ev = nullptr;
    if (ev == nullptr || hipEventRecord(ev, s) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipFreeAsync(base, s);
      if (ev != nullptr) c.spare.push_back(ev);
      return;
    }
    c.blocks.push_back(CachedBlock{base, cap, ev});
    c.bytes += cap;
    trim_cache(c, (size_t)g_keep_bytes.load(), s);
  }
  size_t reserve(size_t bytes) {
    const size_t at = (size + 255) & ~(size_t)255;
    size = at + bytes;
    return at;
  }
  bool allocate() {
    if (size == 0) return true;
    if (over_limit(size)) return false;
    note_call_bytes(size);
    // A stream being captured into a graph (or one whose state cannot be
    // read) gets plain stream-ordered memory, which the capture records as
    // the graph's own allocation and free: kept blocks are ordered by events
    // recorded outside any capture, and the pool is not the graph's.
    if (stream_capturing(s)) {
      dev = -1;
      if (hipMallocAsync(&base, size, s) != hipSuccess || base == nullptr) {
        (void)hipGetLastError();
        base = nullptr;
        return false;
      }
      cap = size;
      return true;
    }
    dev = stream_device(s);
    if (dev >= 0 && dev < kMaxDevices) {
      BlockCache& c = g_cache[dev];
      std::lock_guard<std::mutex> lk(c.mu);
      int best = -1;
      for (int i = 0; i < (int)c.blocks.size(); ++i) {
        const size_t b = c.blocks[(size_t)i].size;
        if (b >= size && b <= 2 * size + ((size_t)1 << 20) &&
            (best < 0 || b < c.blocks[(size_t)best].size))
          best = i;
      }
      if (best >= 0) {
        const CachedBlock b = c.blocks[(size_t)best];
        c.blocks.erase(c.blocks.begin() + best);
        c.bytes -= b.size;
        if (hipStreamWaitEvent(s, b.ev, 0) == hipSuccess) {
          base = b.ptr;
          cap = b.size;
          ev = b.ev;
          return true;
        }
        (void)hipGetLastError();   // cannot order after its last use: give it back
        (void)hipEventSynchronize(b.ev);
        (void)hipFreeAsync(b.ptr, s);
        c.spare.push_back(b.ev);
      }
    }
    hipMemPool_t pool = workspace_pool(s);
    const hipError_t e = pool != nullptr ? hipMallocFromPoolAsync(&base, size, pool, s)
                                         : hipMallocAsync(&base, size, s);
    if (e != hipSuccess || base == nullptr) {
      base = nullptr;
      return false;
    }
    cap = size;
    return true;
  }
  // Carve the pieces from memory the caller holds instead of allocating.
  bool use_external(void* p, size_t bytes) {
    if (size > bytes) return false;
    base = p;
    cap = bytes;
    external = true;
    return true;
  }
  template <class T>
  T* at(size_t off) const { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }
};

dpf_status hip_fail(hipError_t e, const char* where) {
  return fail(DPF_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

// Shared body of the dense and projected calls once X (or Y) is final.
struct LayerPlan {
  dpf::LayerArgs args{};
  dpf::NormPath path = dpf::NormPath::kGram;
  bool vec = false;
  int np = 0;
};

LayerPlan plan_layer(const dpf_act* X, const dpf_act* G, const uint8_t* mask,
                     bool allow_staged = false, bool allow_onepass = false) {
  LayerPlan L;
  L.args.X = to_act(X);
  L.args.G = to_act(G);
  L.args.dtype = X->dtype;
  L.args.B = (int)X->B;
  L.args.T = (int)X->T;
  L.args.din = (int)X->D;
  L.args.dout = (int)G->D;
  L.args.mask = mask;
  L.args.nwords = (int)((X->T + dpf::kBitsTokens - 1) / dpf::kBitsTokens);
  L.args.denom = (float)X->B;
  L.args.beta = 0;
  L.vec = vec_ok(X) && vec_ok(G);
  L.path = choose_path(L.args, L.vec, allow_staged, allow_onepass);
  L.np = dpf::norm_partials_per_sample(L.args, L.path, L.vec);
  return L;
}

// Workspace pieces of one or more layer calls (offsets into a Workspace).
struct LayerWs {
  size_t bits = 0, steps = 0, part = 0, c = 0, sk = 0;
  bool has_bits = false, has_steps = false, has_part = false, has_sk = false;
  size_t staged = 0;   // staged path (one layer): bytes of per-sample tiles (a StagedLease)
};

// Reserve, in one workspace, what the layers need when their launches
// follow one another on one stream: row bits and the active-step list when
// masked (the layers share B, T and the mask), norm partials, clip factors,
// and the split-tile partials that the norm and accumulate kernels of a
// layer use one after the other.  Pieces that no two launches use at the
// same time are shared between the layers at the size of the largest.
LayerWs reserve_layers(const LayerPlan* const* Ls, int n, Workspace& ws, bool norm, bool clip,
                       bool accum) {
  LayerWs o;
  const dpf::LayerArgs& a0 = Ls[0]->args;
  bool any_big = false;
  size_t part = 0, sk = 0;
  for (int l = 0; l < n; ++l) {
    const LayerPlan& L = *Ls[l];
    const dpf::LayerArgs& a = L.args;
    if (dpf::big_path(a, L.vec)) any_big = true;
    if (norm) part = std::max(part, (size_t)a.B * L.np * sizeof(double));
    // no split partials: staged tiles, or the single pass (no separate phases)
    if (L.path == dpf::NormPath::kStaged || L.path == dpf::NormPath::kOnePass) continue;
    if (norm) sk = std::max(sk, dpf::norm_workspace_bytes(a, L.path, L.vec));
    if (accum) sk = std::max(sk, dpf::accumulate_workspace_bytes(a, L.vec));
  }
  if (a0.mask != nullptr) {
    o.has_bits = true;
    o.bits = ws.reserve((size_t)a0.B * a0.nwords * sizeof(uint32_t));
    if (any_big) {
      o.has_steps = true;
      o.steps = ws.reserve(dpf::step_list_words(a0.B, a0.nwords) * sizeof(uint32_t));
    }
  }
  if (norm) {
    o.has_part = true;
    o.part = ws.reserve(part);
  }
  if (clip) o.c = ws.reserve((size_t)a0.B * sizeof(float));
  if (sk != 0) {
    o.has_sk = true;
    o.sk = ws.reserve(sk);
  }
  if (n == 1 && Ls[0]->path == dpf::NormPath::kStaged)
    o.staged = dpf::norm_workspace_bytes(a0, dpf::NormPath::kStaged, Ls[0]->vec);
  return o;
}

LayerWs reserve_layer(const LayerPlan& L, Workspace& ws, bool norm, bool clip, bool accum) {
  const LayerPlan* one = &L;
  return reserve_layers(&one, 1, ws, norm, clip, accum);
}

// Once the workspace is allocated: queue the row bits and the active-step
// list of a masked call (once for all the layers that share them).
hipError_t prepare_mask(const dpf::LayerArgs& a, const Workspace& ws, const LayerWs& o,
                        hipStream_t s) {
  if (a.mask == nullptr) return hipSuccess;
  uint32_t* bits = ws.at<uint32_t>(o.bits);
  hipError_t e = dpf::launch_row_bits(a.mask, a.B, a.T, bits, a.nwords, s);
  if (e == hipSuccess && o.has_steps)
    e = dpf::launch_step_list(bits, a.B, a.nwords, ws.at<uint32_t>(o.steps), s);
  return e;
}

// Point a layer at its workspace pieces.
void point_layer(LayerPlan& L, const Workspace& ws, const LayerWs& o) {
  dpf::LayerArgs& a = L.args;
  a.rowbits = o.has_bits ? ws.at<uint32_t>(o.bits) : nullptr;
  a.steps = o.has_steps && dpf::big_path(a, L.vec) ? ws.at<uint32_t>(o.steps) : nullptr;
  a.skws = o.has_sk ? ws.at<float>(o.sk) : nullptr;
  a.partials = o.has_part ? ws.at<double>(o.part) : nullptr;
}

hipError_t bind_layer(LayerPlan& L, const Workspace& ws, const LayerWs& o, hipStream_t s) {
  point_layer(L, ws, o);
  return prepare_mask(L.args, ws, o, s);
}

// Accumulate phase of a layer: the staged path combines the tiles its norm
// phase stored; the others run the scaled contraction.
hipError_t accumulate_phase(const LayerPlan& L, hipStream_t s) {
  if (L.path == dpf::NormPath::kStaged) return dpf::launch_staged_combine(L.args, s);
  return dpf::launch_accumulate(L.args, L.vec, s);
}

// Norm phase of a bound layer: partials, then their ordered sum into sq
// (added when accumulate != 0) or, with c != nullptr, the clip factors.
hipError_t norm_phase(const LayerPlan& L, double* sq, int accumulate, float C, float* c,
                      float* norms_out, hipStream_t s) {
  hipError_t e = dpf::launch_norm(L.args, L.path, L.vec, s);
  if (e != hipSuccess) return e;
  return dpf::launch_finalize(L.args.partials, L.args.B, L.np, sq, accumulate, C, c, norms_out, s);
}

dpf_status fused_layer(const dpf_act* X, const dpf_act* G, const uint8_t* mask, float C,
                       float sigma, uint64_t seed, uint64_t offset, float denom, int beta,
                       float* grad_out, float* norms_out, hipStream_t s, Workspace& ws) {
  // The single pass needs a cooperative launch, which a graph capture does
  // not take: captured calls keep the two-phase paths.
  LayerPlan L = plan_layer(X, G, mask, true, !stream_capturing(s));
  L.args.denom = denom;
  L.args.beta = beta;
  L.args.noise_std = sigma * C;
  L.args.seed = seed;
  L.args.offset = offset;
  L.args.out = grad_out;
  // A tiny layer runs the whole step in one workgroup (unless a norm path is
  // forced): one launch, no workspace.
  if (g_norm_path.load() == 0 && dpf::tiny_eligible(L.args)) {
    const hipError_t e = dpf::launch_tiny_layer(L.args, C, norms_out, s);
    if (e != hipSuccess) return hip_fail(e, "tiny layer launch");
    return ok();
  }
  const LayerWs o = reserve_layer(L, ws, true, true, true);
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  StagedLease lease;   // the staged path's per-sample tiles, until the combine is queued
  if (L.path == dpf::NormPath::kStaged && !lease.acquire(s, o.staged))
    return fail(DPF_ERR_OUT_OF_MEMORY, "staged workspace allocation failed");
  hipError_t e = bind_layer(L, ws, o, s);
  if (e != hipSuccess) return hip_fail(e, "mask preparation launch");
  if (L.path == dpf::NormPath::kOnePass) {
    e = dpf::launch_onepass(L.args, C, norms_out, s);
    if (e != hipSuccess) return hip_fail(e, "single-pass launch");
    return ok();
  }
  if (L.path == dpf::NormPath::kStaged) L.args.skws = static_cast<float*>(lease.ptr());
  float* c = ws.at<float>(o.c);
  e = norm_phase(L, nullptr, 0, C, c, norms_out, s);
  if (e != hipSuccess) return hip_fail(e, "norm phase launch");
  L.args.c = c;
  e = accumulate_phase(L, s);
  if (e != hipSuccess) return hip_fail(e, "accumulate launch");
  return ok();
}

dpf_status check_clip(float C, float sigma) {
  if (!std::isfinite(C) || !(C > 0.0f)) return fail(DPF_ERR_INVALID_ARGUMENT, "C must be finite and > 0");
  if (!std::isfinite(sigma) || sigma < 0.0f)
    return fail(DPF_ERR_INVALID_ARGUMENT, "sigma must be finite and >= 0");
  if (!std::isfinite(sigma * C)) return fail(DPF_ERR_INVALID_ARGUMENT, "sigma * C overflows");
  return DPF_OK;
}

// Philox block ranges [o1, o1 + n1) and [o2, o2 + n2) of one key share a
// block (the block index wraps modulo 2^64).
bool blocks_overlap(uint64_t o1, uint64_t n1, uint64_t o2, uint64_t n2) {
  if (n1 == 0 || n2 == 0) return false;
  return (uint64_t)(o2 - o1) < n1 || (uint64_t)(o1 - o2) < n2;
}

uint64_t noise_blocks_of(int64_t n) { return n <= 0 ? 0 : ((uint64_t)n + 3) / 4; }

// Default scale of a seeded projection: entries N(0, 1/r).
float projection_scale(float p_scale, int64_t r) {
  return (std::isnan(p_scale) || p_scale <= 0.0f) ? (float)(1.0 / std::sqrt((double)r)) : p_scale;
}

// Shared body of the projected calls: P read from memory (gen == 0) or
// regenerated from (p_seed, p_offset, p_scale) inside the projection.  Split
// into the workspace plan (reserve_projected) and the launches
// (queue_projected), so that several calls can share one workspace.
// The r-space sum G~^T Y of a projected call is a [dout, r] output of a few
// tiles over B*T tokens: with "rspace_tiles" 1 (the default) its
// accumulation runs on 128 x 128 tiles whose samples are cut into pieces
// over the compute units, 2 adds the direct norm on those tiles, 0 keeps the
// large tiles.  Measured on MI355X (RoBERTa-large, r = 256, B = 32, T = 128).
std::atomic<int> g_rspace_tiles{1};

LayerPlan plan_rspace(const dpf_act* Y, const dpf_act* G, const uint8_t* mask, int small) {
  LayerPlan L = plan_layer(Y, G, mask, true);
  L.args.small_tiles = small;
  L.np = dpf::norm_partials_per_sample(L.args, L.path, L.vec);
  return L;
}

struct ProjectedCall {
  dpf::ProjArgs pa{};
  int small = 0;   // rspace_tiles when the call was planned
  bool pvec = false;
  size_t off_y = 0, off_part = 0, pbytes = 0;
  dpf_act Y{};
  LayerPlan L;
  LayerWs o{};
};

void reserve_projected(ProjectedCall& pc, const dpf_act* X, const dpf_act* G, const uint8_t* mask,
                       const void* P, int gen, uint64_t p_seed, uint64_t p_offset, float p_scale,
                       int64_t r, Workspace& ws) {
  const size_t es = elem_size(X->dtype);
  pc.off_y = ws.reserve((size_t)X->B * X->T * r * es);
  dpf::ProjArgs& pa = pc.pa;
  pa.X = to_act(X);
  pa.P = P;
  pa.dtype = X->dtype;
  pa.B = (int)X->B;
  pa.T = (int)X->T;
  pa.din = (int)X->D;
  pa.r = (int)r;
  pa.mask = mask;
  pa.gen = gen;
  pa.p_seed = p_seed;
  pa.p_offset = p_offset;
  pa.p_scale = p_scale;
  pc.pvec = vec_ok(X) && ((size_t)r * es) % 16 == 0;
  pa.splits = dpf::project_splits(pa, pc.pvec);
  pc.pbytes = dpf::project_workspace_bytes(pa, pc.pvec);
  pc.off_part = pc.pbytes != 0 ? ws.reserve(pc.pbytes) : 0;
  // The layer workspace in the same allocation.
  pc.Y = dpf_act{nullptr, X->dtype, 0, X->B, X->T, r, X->T * r, r};
  pc.small = g_rspace_tiles.load();
  pc.L = plan_rspace(&pc.Y, G, mask, pc.small);
  pc.o = reserve_layer(pc.L, ws, true, true, true);
}

// The launches of a planned call on stream s (ws allocated; for the staged
// path, staged holds the per-sample tiles).
dpf_status queue_projected(ProjectedCall& pc, const dpf_act* G, const uint8_t* mask,
                           const Workspace& ws, void* staged, float C, float sigma, uint64_t seed,
                           uint64_t offset, float* grad_out, float* norms_out, hipStream_t s) {
  pc.Y.data = ws.at<void>(pc.off_y);
  pc.pa.Y = const_cast<void*>(pc.Y.data);
  pc.pa.part = pc.pbytes != 0 ? ws.at<float>(pc.off_part) : nullptr;
  hipError_t e = dpf::launch_project(pc.pa, pc.pvec, s);
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  LayerPlan L = plan_rspace(&pc.Y, G, mask, pc.small);
  e = bind_layer(L, ws, pc.o, s);
  if (e != hipSuccess) return hip_fail(e, "mask preparation launch");
  if (L.path == dpf::NormPath::kStaged) L.args.skws = static_cast<float*>(staged);
  float* c = ws.at<float>(pc.o.c);
  e = norm_phase(L, nullptr, 0, C, c, norms_out, s);
  if (e != hipSuccess) return hip_fail(e, "norm phase launch");
  L.args.c = c;
  L.args.noise_std = sigma * C;
  L.args.seed = seed;
  L.args.offset = offset;
  L.args.out = grad_out;
  e = accumulate_phase(L, s);
  if (e != hipSuccess) return hip_fail(e, "accumulate launch");
  return ok();
}

dpf_status projected_layer(const dpf_act* X, const dpf_act* G, const uint8_t* mask, const void* P,
                           int gen, uint64_t p_seed, uint64_t p_offset, float p_scale, int64_t r,
                           float C, float sigma, uint64_t seed, uint64_t offset, float* grad_out,
                           float* norms_out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace ws(s);
  ProjectedCall pc;
  reserve_projected(pc, X, G, mask, P, gen, p_seed, p_offset, p_scale, r, ws);
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  StagedLease lease;   // the staged path's per-sample tiles, until the combine is queued
  if (pc.L.path == dpf::NormPath::kStaged && !lease.acquire(s, pc.o.staged))
    return fail(DPF_ERR_OUT_OF_MEMORY, "staged workspace allocation failed");
  return queue_projected(pc, G, mask, ws, lease.ptr(), C, sigma, seed, offset, grad_out,
                         norms_out, s);
}

// Norm phase of one linear into sq[B] (added when accumulate != 0).
dpf_status sqnorms_into(const dpf_act* X, const dpf_act* G, const uint8_t* mask, double* sq,
                        int accumulate, hipStream_t s) {
  Workspace ws(s);
  LayerPlan L = plan_layer(X, G, mask);
  const LayerWs o = reserve_layer(L, ws, true, false, false);
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  hipError_t e = bind_layer(L, ws, o, s);
  if (e != hipSuccess) return hip_fail(e, "mask preparation launch");
  e = norm_phase(L, sq, accumulate ? 1 : 0, 1.0f, nullptr, nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "norm phase launch");
  return ok();
}

// ---------------------------------------------------------------------------
// Static scratch of dpfused_linear_clip_accumulate_noalloc
// ---------------------------------------------------------------------------
// The call's workspace lives in the file-scope array `scratch` (top of this
// file) instead of the pool.  Host code never passes the array's name to a
// kernel (in host code it only stands for the symbol): it takes the device
// address once per device with hipGetSymbolAddress and uses that.
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of device dev's copy of `scratch`, taken on its first
// use with dev current; nullptr (and the reason) if it cannot be had.
void* scratch_ptr(int dev, std::string* why) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] != nullptr) return g_scratch_ptr[dev];
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
  void* p = nullptr;
  if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    *why = std::string("no address for the static scratch: ") + hipGetErrorString(e);
    return nullptr;
  }
  g_scratch_ptr[dev] = p;
  return p;
}

// Workspace bytes a dense call on plan L takes (nothing is allocated).
size_t layer_ws_bytes(const LayerPlan& L, hipStream_t s) {
  Workspace dry(s);
  (void)reserve_layer(L, dry, true, true, true);
  return dry.size;
}

// Accumulate phase of one linear with given clip factors c[B].
dpf_status accumulate_with(const dpf_act* X, const dpf_act* G, const uint8_t* mask, const float* c,
                           float noise_std, uint64_t seed, uint64_t offset, float* grad_out,
                           hipStream_t s) {
  Workspace ws(s);
  LayerPlan L = plan_layer(X, G, mask);
  const LayerWs o = reserve_layer(L, ws, false, false, true);
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  hipError_t e = bind_layer(L, ws, o, s);
  if (e != hipSuccess) return hip_fail(e, "mask preparation launch");
  L.args.c = c;
  L.args.noise_std = noise_std;
  L.args.seed = seed;
  L.args.offset = offset;
  L.args.out = grad_out;
  e = accumulate_phase(L, s);
  if (e != hipSuccess) return hip_fail(e, "accumulate launch");
  return ok();
}

}  // namespace

// ===========================================================================
// Timing hooks used by the launchers
// ===========================================================================
namespace dpf {
void timing_begin(const char* name, hipStream_t s) {
  if (!g_timing.load()) return;
  Pending p;
  p.name = name;
  if (hipEventCreate(&p.start) != hipSuccess) return;
  (void)hipEventRecord(p.start, s);
  std::lock_guard<std::mutex> lk(g_tmu);
  g_pending.push_back(p);
}
void timing_end(const char* name, hipStream_t s) {
  if (g_debug.load()) {
    // debugging: wait for the kernel and report a failure by its name
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) std::fprintf(stderr, "dpfused: kernel %s failed: %s\n", name, hipGetErrorString(e));
  }
  if (!g_timing.load()) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto it = g_pending.rbegin(); it != g_pending.rend(); ++it) {
    if (it->stop == nullptr && it->name == name) {
      if (hipEventCreate(&it->stop) == hipSuccess) (void)hipEventRecord(it->stop, s);
      return;
    }
  }
}
}  // namespace dpf

// ===========================================================================
// C entry points
// ===========================================================================
extern "C" {

dpf_status dpfused_linear_clip_accumulate(const dpf_act* X, const dpf_act* G, const uint8_t* mask,
                                          float C, float sigma, uint64_t seed, uint64_t offset,
                                          float* grad_out, float* norms_out, void* stream) {
  CallScope call_("dpfused_linear_clip_accumulate");
  dpf_status st = check_pair(X, G);
  if (st != DPF_OK) return st;
  if ((st = check_clip(C, sigma)) != DPF_OK) return st;
  if (grad_out == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "grad_out is NULL");
  if (!aligned16(grad_out)) return fail(DPF_ERR_UNSUPPORTED, "grad_out is not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace ws(s);
  return fused_layer(X, G, mask, C, sigma, seed, offset, (float)X->B, 0, grad_out, norms_out, s,
                     ws);
}

dpf_status dpfused_linear_clip_accumulate_ex(const dpf_act* X, const dpf_act* G,
                                             const uint8_t* mask, float C, float sigma,
                                             uint64_t seed, uint64_t offset, float denom,
                                             int32_t accumulate, float* grad_out,
                                             float* norms_out, void* stream) {
  CallScope call_("dpfused_linear_clip_accumulate_ex");
  dpf_status st = check_pair(X, G);
  if (st != DPF_OK) return st;
  if ((st = check_clip(C, sigma)) != DPF_OK) return st;
  if (!std::isfinite(denom) || !(denom > 0.0f))
    return fail(DPF_ERR_INVALID_ARGUMENT, "denom must be finite and > 0");
  if (accumulate != 0 && accumulate != 1)
    return fail(DPF_ERR_INVALID_ARGUMENT, "accumulate must be 0 or 1");
  if (grad_out == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "grad_out is NULL");
  if (!aligned16(grad_out)) return fail(DPF_ERR_UNSUPPORTED, "grad_out is not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Workspace ws(s);
  return fused_layer(X, G, mask, C, sigma, seed, offset, denom, accumulate, grad_out, norms_out,
                     s, ws);
}

dpf_status dpfused_linear_clip_accumulate_noalloc(const dpf_act* X, const dpf_act* G,
                                                  const uint8_t* mask, float C, float sigma,
                                                  uint64_t seed, uint64_t offset,
                                                  float* grad_out, float* norms_out,
                                                  void* stream) {
  CallScope call_("dpfused_linear_clip_accumulate_noalloc");
  dpf_status st = check_pair(X, G);
  if (st != DPF_OK) return st;
  if ((st = check_clip(C, sigma)) != DPF_OK) return st;
  if (grad_out == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "grad_out is NULL");
  if (!aligned16(grad_out)) return fail(DPF_ERR_UNSUPPORTED, "grad_out is not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int dev = stream_device(s);
  if (dev < 0 || dev >= kMaxDevices) return fail(DPF_ERR_HIP, "cannot tell the stream's device");
  // Never the staged form: its tiles are far larger than the scratch.  The
  // single pass (small workspace) when not under graph capture.
  LayerPlan L = plan_layer(X, G, mask, false, !stream_capturing(s));
  L.args.noise_std = sigma * C;
  L.args.seed = seed;
  L.args.offset = offset;
  L.args.out = grad_out;
  if (g_norm_path.load() == 0 && dpf::tiny_eligible(L.args)) {
    const hipError_t e = dpf::launch_tiny_layer(L.args, C, norms_out, s);
    if (e != hipSuccess) return hip_fail(e, "tiny layer launch");
    return ok();
  }
  // The call's own plan if its workspace fits the scratch; else the same
  // norm path without split tiles or items (no split partials); else, for
  // the Gram path, the direct form without splits (no parked Gram blocks).
  size_t need = layer_ws_bytes(L, s);
  if (need > kScratchBytes) {
    L.args.max_split = 1;
    need = layer_ws_bytes(L, s);
  }
  if (need > kScratchBytes && L.path == dpf::NormPath::kGram && g_norm_path.load() != 1) {
    L.path = dpf::NormPath::kDirect;
    L.np = dpf::norm_partials_per_sample(L.args, L.path, L.vec);
    need = layer_ws_bytes(L, s);
  }
  if (need > kScratchBytes)
    return fail(DPF_ERR_UNSUPPORTED,
                "the call needs " + std::to_string(need) + " bytes of workspace, more than the " +
                    std::to_string(kScratchBytes) + " bytes of static scratch");
  std::string why;
  void* base = scratch_ptr(dev, &why);
  if (base == nullptr) return fail(DPF_ERR_HIP, why);
  Workspace ws(s);
  const LayerWs o = reserve_layer(L, ws, true, true, true);
  if (!ws.use_external(base, kScratchBytes))
    return fail(DPF_ERR_UNSUPPORTED, "workspace larger than the static scratch");
  hipError_t e = bind_layer(L, ws, o, s);
  if (e != hipSuccess) return hip_fail(e, "mask preparation launch");
  if (L.path == dpf::NormPath::kOnePass) {
    e = dpf::launch_onepass(L.args, C, norms_out, s);
    if (e != hipSuccess) return hip_fail(e, "single-pass launch");
    return ok();
  }
  float* c = ws.at<float>(o.c);
  e = norm_phase(L, nullptr, 0, C, c, norms_out, s);
  if (e != hipSuccess) return hip_fail(e, "norm phase launch");
  L.args.c = c;
  e = accumulate_phase(L, s);
  if (e != hipSuccess) return hip_fail(e, "accumulate launch");
  return ok();
}

dpf_status dpfused_linear_clip_accumulate_projected(const dpf_act* X, const dpf_act* G,
                                                    const uint8_t* mask, const void* P, int64_t r,
                                                    float C, float sigma, uint64_t seed,
                                                    uint64_t offset, float* grad_out,
                                                    float* norms_out, void* stream) {
  CallScope call_("dpfused_linear_clip_accumulate_projected");
  dpf_status st = check_pair(X, G);
  if (st != DPF_OK) return st;
  if ((st = check_clip(C, sigma)) != DPF_OK) return st;
  if (P == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "P is NULL");
  if (r < 1) return fail(DPF_ERR_INVALID_ARGUMENT, "r must be >= 1");
  if (r > kMaxDim) return fail(DPF_ERR_UNSUPPORTED, "r too large");
  if (!aligned16(P)) return fail(DPF_ERR_UNSUPPORTED, "P is not 16-byte aligned");
  if (grad_out == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "grad_out is NULL");
  if (!aligned16(grad_out)) return fail(DPF_ERR_UNSUPPORTED, "grad_out is not 16-byte aligned");
  return projected_layer(X, G, mask, P, 0, 0, 0, 0.0f, r, C, sigma, seed, offset, grad_out,
                         norms_out, stream);
}

// Streams of the library for the calls that run several linears side by
// side: per device, created on first use at the default priority and kept
// until the process ends, with a fork event (recorded on the caller's stream)
// and one join event per stream.  The lock is held while a call queues its
// work, so the events' records and the waits on them pair up.
constexpr int kSideStreams = 4;
// Library streams a call uses beside the caller's own (0 .. kSideStreams).
// Measured on the RoBERTa layer (six calls): with one, the host's queueing
// (about 210 us per layer: each fork and join costs event records and waits)
// and the GPU's time meet at about 217 us; more streams overlap more on the
// GPU but cost more on the host (235 us with three, 253 with four); none
// gives the six calls back to back (281 us).
std::atomic<int> g_side_streams{1};
struct SidePool {
  std::mutex mu;
  int state = 0;   // 0: not yet created, 1: ready, -1: creation failed
  hipStream_t s[kSideStreams] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kSideStreams] = {};
};
SidePool g_side[kMaxDevices];

// Device dev's pool with its lock taken into lk, or nullptr (then the calls
// run one after another on the caller's stream).
SidePool* side_pool(int dev, std::unique_lock<std::mutex>& lk) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  SidePool& sp = g_side[dev];
  lk = std::unique_lock<std::mutex>(sp.mu);
  if (sp.state == 0) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    for (int k = 0; k < kSideStreams && e == hipSuccess; ++k)
      e = hipStreamCreateWithFlags(&sp.s[k], hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&sp.fork, hipEventDisableTiming);
    for (int k = 0; k < kSideStreams && e == hipSuccess; ++k)
      e = hipEventCreateWithFlags(&sp.join[k], hipEventDisableTiming);
    if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) (void)hipGetLastError();
    sp.state = e == hipSuccess ? 1 : -1;
  }
  return sp.state == 1 ? &sp : nullptr;
}

dpf_status dpfused_linear_clip_accumulate_projected_many(
    int32_t n, const dpf_act* X, const dpf_act* G, const uint8_t* const* masks,
    const void* const* P, int64_t r, float C, float sigma, uint64_t seed, const uint64_t* offsets,
    float* const* grad_out, float* const* norms_out, void* stream) {
  CallScope call_("dpfused_linear_clip_accumulate_projected_many");
  if (n < 1 || n > 64) return fail(DPF_ERR_INVALID_ARGUMENT, "n must be in 1 .. 64");
  if (X == nullptr || G == nullptr || P == nullptr || offsets == nullptr || grad_out == nullptr)
    return fail(DPF_ERR_INVALID_ARGUMENT, "X, G, P, offsets and grad_out must not be NULL");
  dpf_status st = check_clip(C, sigma);
  if (st != DPF_OK) return st;
  if (r < 1) return fail(DPF_ERR_INVALID_ARGUMENT, "r must be >= 1");
  if (r > kMaxDim) return fail(DPF_ERR_UNSUPPORTED, "r too large");
  for (int32_t l = 0; l < n; ++l) {
    if ((st = check_pair(&X[l], &G[l])) != DPF_OK) return st;
    if (P[l] == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "P[l] is NULL");
    if (!aligned16(P[l])) return fail(DPF_ERR_UNSUPPORTED, "P[l] is not 16-byte aligned");
    if (grad_out[l] == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "grad_out[l] is NULL");
    if (!aligned16(grad_out[l]))
      return fail(DPF_ERR_UNSUPPORTED, "grad_out[l] is not 16-byte aligned");
  }
  // With noise, two calls drawing the same Philox blocks would carry the same
  // normals, which cancel when their outputs are subtracted.
  if (sigma > 0.0f) {
    for (int32_t l = 0; l < n; ++l)
      for (int32_t m = l + 1; m < n; ++m)
        if (blocks_overlap(offsets[l], noise_blocks_of(G[l].D * r), offsets[m],
                           noise_blocks_of(G[m].D * r)))
          return fail(DPF_ERR_INVALID_ARGUMENT,
                      "the noise block ranges of two calls overlap (offsets[l] .. offsets[l] + "
                      "dpfused_noise_blocks(dout_l * r) must be disjoint)");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mask_of = [&](int32_t l) { return masks != nullptr ? masks[l] : nullptr; };
  auto norms_of = [&](int32_t l) { return norms_out != nullptr ? norms_out[l] : nullptr; };
  // One workspace for every call, on the caller's stream, taken before the
  // first launch: a failed allocation leaves every output untouched.
  Workspace ws(s);
  std::vector<ProjectedCall> pcs((size_t)n);
  bool staged = false;
  for (int32_t l = 0; l < n; ++l) {
    reserve_projected(pcs[(size_t)l], &X[l], &G[l], mask_of(l), P[l], 0, 0, 0, 0.0f, r, ws);
    staged = staged || pcs[(size_t)l].L.path == dpf::NormPath::kStaged;
  }
  if (staged) {
    // A forced staged path keeps its tiles in the per-device staged buffer,
    // which one call holds at a time: the calls run one after another.
    for (int32_t l = 0; l < n; ++l) {
      st = projected_layer(&X[l], &G[l], mask_of(l), P[l], 0, 0, 0, 0.0f, r, C, sigma, seed,
                           offsets[l], grad_out[l], norms_of(l), stream);
      if (st != DPF_OK) return st;
    }
    return ok();
  }
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  const int side = std::min(n - 1, g_side_streams.load());
  std::unique_lock<std::mutex> lk;
  SidePool* sp = (side > 0 && !stream_capturing(s)) ? side_pool(stream_device(s), lk) : nullptr;
  if (sp == nullptr) {
    for (int32_t l = 0; l < n; ++l) {
      st = queue_projected(pcs[(size_t)l], &G[l], mask_of(l), ws, nullptr, C, sigma, seed,
                           offsets[l], grad_out[l], norms_of(l), s);
      if (st != DPF_OK) return st;
    }
    return ok();
  }
  // Fork: the library's streams start after the caller's earlier work (and
  // the workspace allocation).  Call l runs on branch l mod (side + 1):
  // branch 0 is the caller's stream itself, branch k the library's stream k-1.
  hipError_t e = hipEventRecord(sp->fork, s);
  for (int k = 0; k < side && e == hipSuccess; ++k) e = hipStreamWaitEvent(sp->s[k], sp->fork, 0);
  if (e != hipSuccess) return hip_fail(e, "stream fork");
  st = DPF_OK;
  for (int32_t l = 0; l < n && st == DPF_OK; ++l) {
    const int br = l % (side + 1);
    st = queue_projected(pcs[(size_t)l], &G[l], mask_of(l), ws, nullptr, C, sigma, seed,
                         offsets[l], grad_out[l], norms_of(l), br == 0 ? s : sp->s[br - 1]);
  }
  // Join, also after a failed launch: the caller's stream (and the release
  // of the workspace on it) waits for whatever was queued.
  hipError_t ej = hipSuccess;
  for (int k = 0; k < side; ++k) {
    if (ej == hipSuccess) ej = hipEventRecord(sp->join[k], sp->s[k]);
    if (ej == hipSuccess) ej = hipStreamWaitEvent(s, sp->join[k], 0);
  }
  if (st != DPF_OK) return st;
  if (ej != hipSuccess) return hip_fail(ej, "stream join");
  return ok();
}

dpf_status dpfused_linear_clip_accumulate_projected_seeded(
    const dpf_act* X, const dpf_act* G, const uint8_t* mask, int64_t r, uint64_t p_seed,
    uint64_t p_offset, float p_scale, float C, float sigma, uint64_t seed, uint64_t offset,
    float* grad_out, float* norms_out, void* stream) {
  CallScope call_("dpfused_linear_clip_accumulate_projected_seeded");
  dpf_status st = check_pair(X, G);
  if (st != DPF_OK) return st;
  if ((st = check_clip(C, sigma)) != DPF_OK) return st;
  if (r < 1) return fail(DPF_ERR_INVALID_ARGUMENT, "r must be >= 1");
  if (r > kMaxDim) return fail(DPF_ERR_UNSUPPORTED, "r too large");
  if (r % 8 != 0) return fail(DPF_ERR_UNSUPPORTED, "r must be a multiple of 8");
  if (std::isinf(p_scale)) return fail(DPF_ERR_INVALID_ARGUMENT, "p_scale must be finite");
  if (grad_out == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "grad_out is NULL");
  if (!aligned16(grad_out)) return fail(DPF_ERR_UNSUPPORTED, "grad_out is not 16-byte aligned");
  // Noise drawn from the projection's own blocks would be a copy of P's
  // entries (scaled): anyone who can draw P again would know the noise.
  if (sigma > 0.0f && seed == p_seed &&
      blocks_overlap(offset, noise_blocks_of(G->D * r), p_offset, noise_blocks_of(X->D * r)))
    return fail(DPF_ERR_INVALID_ARGUMENT,
                "the noise blocks overlap the projection's blocks under the same seed");
  return projected_layer(X, G, mask, nullptr, 1, p_seed, p_offset, projection_scale(p_scale, r),
                         r, C, sigma, seed, offset, grad_out, norms_out, stream);
}

dpf_status dpfused_project(const dpf_act* X, const uint8_t* mask, const void* P, int64_t r,
                           void* Y, void* stream) {
  CallScope call_("dpfused_project");
  dpf_status st = check_act(X, "X");
  if (st != DPF_OK) return st;
  if (P == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "P is NULL");
  if (Y == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "Y is NULL");
  if (r < 1) return fail(DPF_ERR_INVALID_ARGUMENT, "r must be >= 1");
  if (r > kMaxDim) return fail(DPF_ERR_UNSUPPORTED, "r too large");
  if (!aligned16(P)) return fail(DPF_ERR_UNSUPPORTED, "P is not 16-byte aligned");
  if (!aligned16(Y)) return fail(DPF_ERR_UNSUPPORTED, "Y is not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t es = elem_size(X->dtype);
  dpf::ProjArgs pa{};
  pa.X = to_act(X);
  pa.P = P;
  pa.Y = Y;
  pa.dtype = X->dtype;
  pa.B = (int)X->B;
  pa.T = (int)X->T;
  pa.din = (int)X->D;
  pa.r = (int)r;
  pa.mask = mask;
  const bool pvec = vec_ok(X) && ((size_t)r * es) % 16 == 0;
  pa.splits = dpf::project_splits(pa, pvec);
  const size_t pbytes = dpf::project_workspace_bytes(pa, pvec);
  Workspace ws(s);
  const size_t off_part = pbytes != 0 ? ws.reserve(pbytes) : 0;
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  pa.part = pbytes != 0 ? ws.at<float>(off_part) : nullptr;
  const hipError_t e = dpf::launch_project(pa, pvec, s);
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  return ok();
}

dpf_status dpfused_per_sample_sqnorms(const dpf_act* X, const dpf_act* G, const uint8_t* mask,
                                      double* sqnorms_out, int32_t accumulate, void* stream) {
  CallScope call_("dpfused_per_sample_sqnorms");
  dpf_status st = check_pair(X, G);
  if (st != DPF_OK) return st;
  if (sqnorms_out == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "sqnorms_out is NULL");
  return sqnorms_into(X, G, mask, sqnorms_out, accumulate, static_cast<hipStream_t>(stream));
}

dpf_status dpfused_clip_factors(const double* sqnorms, int64_t n, float C, float* c_out,
                                float* norms_out, void* stream) {
  CallScope call_("dpfused_clip_factors");
  if (sqnorms == nullptr || c_out == nullptr)
    return fail(DPF_ERR_INVALID_ARGUMENT, "sqnorms and c_out must not be NULL");
  if (n < 1) return fail(DPF_ERR_INVALID_ARGUMENT, "n must be >= 1");
  if (!std::isfinite(C) || !(C > 0.0f)) return fail(DPF_ERR_INVALID_ARGUMENT, "C must be finite and > 0");
  hipError_t e = dpf::launch_clip_from_sq(sqnorms, n, C, c_out, norms_out,
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "clip factor launch");
  return ok();
}

dpf_status dpfused_scaled_accumulate(const dpf_act* X, const dpf_act* G, const uint8_t* mask,
                                     const float* c, float noise_std, uint64_t seed,
                                     uint64_t offset, float* grad_out, void* stream) {
  CallScope call_("dpfused_scaled_accumulate");
  dpf_status st = check_pair(X, G);
  if (st != DPF_OK) return st;
  if (c == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "c is NULL");
  if (!std::isfinite(noise_std) || noise_std < 0.0f)
    return fail(DPF_ERR_INVALID_ARGUMENT, "noise_std must be finite and >= 0");
  if (grad_out == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "grad_out is NULL");
  if (!aligned16(grad_out)) return fail(DPF_ERR_UNSUPPORTED, "grad_out is not 16-byte aligned");
  return accumulate_with(X, G, mask, c, noise_std, seed, offset, grad_out,
                         static_cast<hipStream_t>(stream));
}

dpf_status dpfused_linear_clip_accumulate_bias(const dpf_act* X, const dpf_act* G,
                                               const uint8_t* mask, float C, float sigma,
                                               uint64_t seed, uint64_t offset, float* grad_out,
                                               float* bias_grad_out, float* norms_out,
                                               void* stream) {
  CallScope call_("dpfused_linear_clip_accumulate_bias");
  dpf_status st = check_pair(X, G);
  if (st != DPF_OK) return st;
  if ((st = check_clip(C, sigma)) != DPF_OK) return st;
  if (grad_out == nullptr || bias_grad_out == nullptr)
    return fail(DPF_ERR_INVALID_ARGUMENT, "grad_out and bias_grad_out must not be NULL");
  if (!aligned16(grad_out)) return fail(DPF_ERR_UNSUPPORTED, "grad_out is not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(bias_grad_out) & 3u) != 0)
    return fail(DPF_ERR_UNSUPPORTED, "bias_grad_out is not 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t B = X->B, dout = G->D;
  // Everything the call needs is reserved, and allocated, before the first
  // launch: a failed allocation leaves every output untouched.
  Workspace ws(s);
  const size_t off_sq = ws.reserve((size_t)B * sizeof(double));
  const size_t off_c = ws.reserve((size_t)B * sizeof(float));
  const size_t off_gb = ws.reserve((size_t)B * dout * sizeof(float));
  const size_t off_part = ws.reserve(dpf::bias_workspace_bytes((int)B, (int)G->T, (int)dout));
  LayerPlan L = plan_layer(X, G, mask, true);
  const LayerWs o = reserve_layer(L, ws, true, false, true);
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  // On the staged path the weight's per-sample tiles are kept until the
  // clip factors (which need the bias's norms too) exist.
  StagedLease lease;
  if (L.path == dpf::NormPath::kStaged && !lease.acquire(s, o.staged))
    return fail(DPF_ERR_OUT_OF_MEMORY, "staged workspace allocation failed");
  double* sq = ws.at<double>(off_sq);
  float* c = ws.at<float>(off_c);
  float* gb = ws.at<float>(off_gb);
  hipError_t e = bind_layer(L, ws, o, s);
  if (e != hipSuccess) return hip_fail(e, "mask preparation launch");
  if (L.path == dpf::NormPath::kStaged) L.args.skws = static_cast<float*>(lease.ptr());
  // ||g_i||^2 of the weight, then + ||gb_i||^2 of the bias
  if ((e = norm_phase(L, sq, 0, 1.0f, nullptr, nullptr, s)) != hipSuccess)
    return hip_fail(e, "norm phase launch");
  e = dpf::launch_bias_grads(to_act(G), G->dtype, (int)B, (int)G->T, (int)dout, mask,
                             ws.at<float>(off_part), gb, sq, s);
  if (e != hipSuccess) return hip_fail(e, "bias gradient launch");
  e = dpf::launch_clip_from_sq(sq, B, C, c, norms_out, s);
  if (e != hipSuccess) return hip_fail(e, "clip factor launch");
  L.args.c = c;
  L.args.noise_std = sigma * C;
  L.args.seed = seed;
  L.args.offset = offset;
  L.args.out = grad_out;
  if ((e = accumulate_phase(L, s)) != hipSuccess) return hip_fail(e, "accumulate launch");
  // the bias noise continues the weight's Philox stream
  const uint64_t boff = offset + noise_blocks_of(dout * X->D);
  e = dpf::launch_bias_accumulate(gb, c, (int)B, (int)dout, sigma * C, seed, boff, bias_grad_out,
                                  s);
  if (e != hipSuccess) return hip_fail(e, "bias accumulate launch");
  return ok();
}

dpf_status dpfused_group_clip_accumulate(int32_t n, const dpf_act* X, const dpf_act* G,
                                         const uint8_t* mask, float C, float sigma, uint64_t seed,
                                         const uint64_t* offsets, float* const* grad_out,
                                         float* norms_out, void* stream) {
  CallScope call_("dpfused_group_clip_accumulate");
  if (n < 1) return fail(DPF_ERR_INVALID_ARGUMENT, "n must be >= 1");
  if (X == nullptr || G == nullptr || offsets == nullptr || grad_out == nullptr)
    return fail(DPF_ERR_INVALID_ARGUMENT, "X, G, offsets and grad_out must not be NULL");
  dpf_status st = check_clip(C, sigma);
  if (st != DPF_OK) return st;
  for (int32_t l = 0; l < n; ++l) {
    if ((st = check_pair(&X[l], &G[l])) != DPF_OK) return st;
    if (X[l].B != X[0].B || X[l].T != X[0].T)
      return fail(DPF_ERR_INVALID_ARGUMENT, "every linear must have the same B and T");
    if (grad_out[l] == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "grad_out[l] is NULL");
    if (!aligned16(grad_out[l]))
      return fail(DPF_ERR_UNSUPPORTED, "grad_out[l] is not 16-byte aligned");
  }
  // With noise, two linears drawing the same Philox blocks would carry the
  // same normals, which cancel when their outputs are subtracted.
  if (sigma > 0.0f) {
    for (int32_t l = 0; l < n; ++l)
      for (int32_t m = l + 1; m < n; ++m)
        if (blocks_overlap(offsets[l], noise_blocks_of(X[l].D * G[l].D), offsets[m],
                           noise_blocks_of(X[m].D * G[m].D)))
          return fail(DPF_ERR_INVALID_ARGUMENT,
                      "the noise block ranges of two linears overlap (offsets[l] .. offsets[l] + "
                      "dpfused_noise_blocks(dout_l * din_l) must be disjoint)");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t B = X[0].B;
  // Plan every linear.  A linear on the staged path keeps its per-sample
  // tiles, at its own place in one staged buffer, from its norm phase until
  // its accumulate phase (after the group's clip factors exist).  The group's
  // staged tiles stay within the per-call limit; the linears past it take
  // their two-pass path.
  std::vector<LayerPlan> lin((size_t)n);
  std::vector<size_t> at((size_t)n, 0);
  size_t staged_total = 0;
  for (int32_t l = 0; l < n; ++l) {
    LayerPlan& L = lin[(size_t)l];
    L = plan_layer(&X[l], &G[l], mask, true);
    if (L.path != dpf::NormPath::kStaged) continue;
    const size_t bytes = dpf::staged_big_workspace_bytes(L.args);
    if ((double)(staged_total + bytes) > kStagedMaxBytes) {
      L = plan_layer(&X[l], &G[l], mask, false);
      continue;
    }
    at[(size_t)l] = staged_total;
    staged_total = (staged_total + bytes + 255) & ~(size_t)255;
  }
  // One workspace for the whole group, taken before the first launch: a
  // failed allocation leaves every output untouched.
  Workspace ws(s);
  const size_t off_sq = ws.reserve((size_t)B * sizeof(double));
  const size_t off_c = ws.reserve((size_t)B * sizeof(float));
  std::vector<const LayerPlan*> plans((size_t)n);
  for (int32_t l = 0; l < n; ++l) plans[(size_t)l] = &lin[(size_t)l];
  const LayerWs o = reserve_layers(plans.data(), n, ws, true, false, true);
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  StagedLease lease;
  if (staged_total != 0 && !lease.acquire(s, staged_total))
    return fail(DPF_ERR_OUT_OF_MEMORY, "staged workspace allocation failed");
  double* sq = ws.at<double>(off_sq);
  float* c = ws.at<float>(off_c);
  hipError_t e = prepare_mask(lin[0].args, ws, o, s);
  if (e != hipSuccess) return hip_fail(e, "mask preparation launch");
  for (int32_t l = 0; l < n; ++l) {
    LayerPlan& L = lin[(size_t)l];
    point_layer(L, ws, o);
    if (L.path == dpf::NormPath::kStaged)
      L.args.skws = reinterpret_cast<float*>(static_cast<char*>(lease.ptr()) + at[(size_t)l]);
  }
  // norm phase of every linear: n_i^2 summed over the group
  for (int32_t l = 0; l < n; ++l) {
    if ((e = norm_phase(lin[(size_t)l], sq, l > 0 ? 1 : 0, 1.0f, nullptr, nullptr, s)) !=
        hipSuccess)
      return hip_fail(e, "norm phase launch");
  }
  e = dpf::launch_clip_from_sq(sq, B, C, c, norms_out, s);
  if (e != hipSuccess) return hip_fail(e, "clip factor launch");
  // accumulate phase of every linear with the group's factors
  for (int32_t l = 0; l < n; ++l) {
    LayerPlan& L = lin[(size_t)l];
    L.args.c = c;
    L.args.noise_std = sigma * C;
    L.args.seed = seed;
    L.args.offset = offsets[l];
    L.args.out = grad_out[l];
    if ((e = accumulate_phase(L, s)) != hipSuccess) return hip_fail(e, "accumulate launch");
  }
  return ok();
}

dpf_status dpfused_projected_adam_step(const float* grad, float* m, float* v, float* W,
                                       int64_t dout, int64_t din, int64_t r, int64_t step,
                                       float lr, float beta1, float beta2, float eps,
                                       const void* P, int32_t p_dtype, uint64_t p_seed,
                                       uint64_t p_offset, float p_scale, void* stream) {
  CallScope call_("dpfused_projected_adam_step");
  if (grad == nullptr || m == nullptr || v == nullptr || W == nullptr)
    return fail(DPF_ERR_INVALID_ARGUMENT, "grad, m, v and W must not be NULL");
  if (dout < 1 || din < 1 || r < 1) return fail(DPF_ERR_INVALID_ARGUMENT, "dout, din, r must be >= 1");
  if (dout > kMaxDim || din > kMaxDim || r > kMaxDim) return fail(DPF_ERR_UNSUPPORTED, "dimension too large");
  if (r % 4 != 0 || din % 4 != 0)
    return fail(DPF_ERR_UNSUPPORTED, "r and din must be multiples of 4");
  if (step < 1) return fail(DPF_ERR_INVALID_ARGUMENT, "step must be >= 1");
  if (!std::isfinite(lr)) return fail(DPF_ERR_INVALID_ARGUMENT, "lr must be finite");
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
    return fail(DPF_ERR_INVALID_ARGUMENT, "beta1 and beta2 must be in [0, 1)");
  if (!std::isfinite(eps) || !(eps > 0.0f)) return fail(DPF_ERR_INVALID_ARGUMENT, "eps must be finite and > 0");
  if (p_dtype != DPF_F32 && p_dtype != DPF_BF16) return fail(DPF_ERR_UNSUPPORTED, "unknown P dtype");
  if (P == nullptr && std::isinf(p_scale))
    return fail(DPF_ERR_INVALID_ARGUMENT, "p_scale must be finite");
  if (!aligned16(grad) || !aligned16(m) || !aligned16(v) || !aligned16(W) ||
      (P != nullptr && !aligned16(P)))
    return fail(DPF_ERR_UNSUPPORTED, "grad, m, v, W and P must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dpf::AdamArgs a{};
  a.grad = grad;
  a.m = m;
  a.v = v;
  a.W = W;
  a.dout = dout;
  a.din = din;
  a.r = r;
  a.lr = lr;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.eps = eps;
  a.bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
  a.bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
  if (!(a.bc1 > 0.0f) || !(a.bc2 > 0.0f))
    return fail(DPF_ERR_INVALID_ARGUMENT, "bias corrections underflow (beta^step == 1)");
  a.P = P;
  a.p_dtype = p_dtype;
  a.gen = P == nullptr ? 1 : 0;
  a.p_seed = p_seed;
  a.p_offset = p_offset;
  a.p_scale = P == nullptr ? projection_scale(p_scale, r) : p_scale;
  Workspace ws(s);
  const size_t off_u = ws.reserve((size_t)dout * r * sizeof(float));
  const bool pbuf = dpf::adam_draws_p_once(a);
  const size_t off_p = pbuf ? ws.reserve((size_t)din * r * elem_size(p_dtype)) : 0;
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  a.u = ws.at<float>(off_u);
  a.pbuf = pbuf ? ws.at<void>(off_p) : nullptr;
  hipError_t e = dpf::launch_projected_adam(a, s);
  if (e != hipSuccess) return hip_fail(e, "projected Adam launch");
  return ok();
}

dpf_status dpfused_philox4x32_10(uint64_t seed, uint64_t offset, int64_t nblocks, uint32_t* out,
                                 void* stream) {
  CallScope call_("dpfused_philox4x32_10");
  if (nblocks < 0) return fail(DPF_ERR_INVALID_ARGUMENT, "nblocks must be >= 0");
  if (nblocks == 0) return ok();
  if (out == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "out is NULL");
  if (!aligned16(out)) return fail(DPF_ERR_UNSUPPORTED, "out is not 16-byte aligned");
  hipError_t e = dpf::launch_philox_fill(seed, offset, nblocks, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "philox launch");
  return ok();
}

dpf_status dpfused_gaussian_fill(uint64_t seed, uint64_t offset, int64_t n, float scale,
                                 int32_t dtype, void* out, void* stream) {
  CallScope call_("dpfused_gaussian_fill");
  if (n < 0) return fail(DPF_ERR_INVALID_ARGUMENT, "n must be >= 0");
  if (dtype != DPF_F32 && dtype != DPF_BF16) return fail(DPF_ERR_UNSUPPORTED, "unknown dtype");
  if (!std::isfinite(scale)) return fail(DPF_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (n == 0) return ok();
  if (out == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "out is NULL");
  if (!aligned16(out)) return fail(DPF_ERR_UNSUPPORTED, "out is not 16-byte aligned");
  hipError_t e = dpf::launch_gaussian_fill(seed, offset, n, scale, dtype, out,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gaussian fill launch");
  return ok();
}

uint64_t dpfused_noise_blocks(int64_t n_elements) {
  return n_elements <= 0 ? 0 : ((uint64_t)n_elements + 3) / 4;
}

dpf_status dpfused_set_option(const char* name, int64_t value) {
  if (name == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "option name is NULL");
  if (std::strcmp(name, "norm_path") == 0) {
    if (value < 0 || value > 4)
      return fail(DPF_ERR_INVALID_ARGUMENT, "norm_path must be 0, 1, 2, 3 or 4");
    g_norm_path.store((int)value);
    return ok();
  }
  if (std::strcmp(name, "onepass_spin_limit") == 0) {
    if (value < 0 || value > (1 << 30))
      return fail(DPF_ERR_INVALID_ARGUMENT, "onepass_spin_limit must be in [0, 2^30]");
    g_onepass_spin.store((int)value);
    dpf::set_onepass_testing(g_onepass_spin.load(), g_onepass_never.load());
    return ok();
  }
  if (std::strcmp(name, "onepass_never_ready") == 0) {
    if (value != 0 && value != 1)
      return fail(DPF_ERR_INVALID_ARGUMENT, "onepass_never_ready must be 0 or 1");
    g_onepass_never.store((int)value);
    dpf::set_onepass_testing(g_onepass_spin.load(), g_onepass_never.load());
    return ok();
  }
  if (std::strcmp(name, "workspace_keep_bytes") == 0) {
    if (value < 0) return fail(DPF_ERR_INVALID_ARGUMENT, "workspace_keep_bytes must be >= 0");
    set_keep_bytes(value);
    return ok();
  }
  if (std::strcmp(name, "staged_keep_bytes") == 0) {
    if (value < 0) return fail(DPF_ERR_INVALID_ARGUMENT, "staged_keep_bytes must be >= 0");
    set_staged_keep(value);
    return ok();
  }
  if (std::strcmp(name, "workspace_limit_bytes") == 0) {
    if (value < 0) return fail(DPF_ERR_INVALID_ARGUMENT, "workspace_limit_bytes must be >= 0");
    g_ws_limit.store(value);
    return ok();
  }
  if (std::strcmp(name, "workspace_call_high") == 0) {
    if (value != 0) return fail(DPF_ERR_INVALID_ARGUMENT, "workspace_call_high can only be reset to 0");
    g_call_high.store(0);
    return ok();
  }
  if (std::strcmp(name, "side_streams") == 0) {
    if (value < 0 || value > kSideStreams)
      return fail(DPF_ERR_INVALID_ARGUMENT, "side_streams must be in [0, 4]");
    g_side_streams.store((int)value);
    return ok();
  }
  if (std::strcmp(name, "rspace_tiles") == 0) {
    if (value < 0 || value > 2) return fail(DPF_ERR_INVALID_ARGUMENT, "rspace_tiles must be 0, 1 or 2");
    g_rspace_tiles.store((int)value);
    return ok();
  }
  if (std::strcmp(name, "p_in_kernels") == 0) {
    if (value != 0 && value != 1) return fail(DPF_ERR_INVALID_ARGUMENT, "p_in_kernels must be 0 or 1");
    dpf::set_p_in_kernels(value != 0);
    return ok();
  }
  if (std::strcmp(name, "trace") == 0 || std::strcmp(name, "debug") == 0) {
    if (value != 0 && value != 1) return fail(DPF_ERR_INVALID_ARGUMENT, "trace and debug must be 0 or 1");
    (name[0] == 't' ? g_trace : g_debug).store((int)value);
    return ok();
  }
  if (std::strcmp(name, "timing") == 0) {
    if (value != 0 && value != 1) return fail(DPF_ERR_INVALID_ARGUMENT, "timing must be 0 or 1");
    g_timing.store((int)value);
    return ok();
  }
  return fail(DPF_ERR_INVALID_ARGUMENT, std::string("unknown option ") + name);
}

int64_t dpfused_get_option(const char* name) {
  if (name == nullptr) return -1;
  if (std::strcmp(name, "norm_path") == 0) return g_norm_path.load();
  if (std::strcmp(name, "onepass_spin_limit") == 0) return g_onepass_spin.load();
  if (std::strcmp(name, "onepass_never_ready") == 0) return g_onepass_never.load();
  if (std::strcmp(name, "timing") == 0) return g_timing.load();
  if (std::strcmp(name, "workspace_keep_bytes") == 0) return g_keep_bytes.load();
  if (std::strcmp(name, "workspace_limit_bytes") == 0) return g_ws_limit.load();
  if (std::strcmp(name, "staged_keep_bytes") == 0) return g_staged_keep.load();
  if (std::strcmp(name, "workspace_call_bytes") == 0) return t_call_bytes;
  if (std::strcmp(name, "workspace_call_high") == 0) return g_call_high.load();
  if (std::strcmp(name, "p_in_kernels") == 0) return dpf::p_in_kernels() ? 1 : 0;
  if (std::strcmp(name, "side_streams") == 0) return g_side_streams.load();
  if (std::strcmp(name, "rspace_tiles") == 0) return g_rspace_tiles.load();
  if (std::strcmp(name, "trace") == 0) return g_trace.load();
  if (std::strcmp(name, "debug") == 0) return g_debug.load();
  // Read-only: memory the current device's workspace pool holds now, and the
  // most it has held (-1 when there is no pool).
  const bool now = std::strcmp(name, "workspace_reserved_bytes") == 0;
  if (now || std::strcmp(name, "workspace_reserved_high") == 0) {
    hipMemPool_t pool = workspace_pool(nullptr);
    uint64_t v = 0;
    const hipMemPoolAttr attr = now ? hipMemPoolAttrReservedMemCurrent : hipMemPoolAttrReservedMemHigh;
    if (pool == nullptr || hipMemPoolGetAttribute(pool, attr, &v) != hipSuccess) return -1;
    return (int64_t)v;
  }
  return -1;
}

void dpfused_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto& p : g_pending) {
    if (p.start) (void)hipEventDestroy(p.start);
    if (p.stop) (void)hipEventDestroy(p.stop);
  }
  g_pending.clear();
  g_totals.clear();
}

int32_t dpfused_timing_collect(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto& p : g_pending) {
    float ms = 0.f;
    if (p.start && p.stop && hipEventSynchronize(p.stop) == hipSuccess &&
        hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      Total* t = nullptr;
      for (auto& x : g_totals)
        if (x.name == p.name) t = &x;
      if (t == nullptr) {
        g_totals.push_back(Total{p.name, 0.0, 0});
        t = &g_totals.back();
      }
      t->ms += ms;
      t->n += 1;
    }
    if (p.start) (void)hipEventDestroy(p.start);
    if (p.stop) (void)hipEventDestroy(p.stop);
  }
  g_pending.clear();
  return (int32_t)g_totals.size();
}

const char* dpfused_timing_name(int32_t k) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (k < 0 || k >= (int32_t)g_totals.size()) return "";
  return g_totals[k].name.c_str();
}

double dpfused_timing_total_ms(int32_t k) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (k < 0 || k >= (int32_t)g_totals.size()) return 0.0;
  return g_totals[k].ms;
}

int64_t dpfused_timing_launches(int32_t k) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (k < 0 || k >= (int32_t)g_totals.size()) return 0;
  return g_totals[k].n;
}

const char* dpfused_status_string(dpf_status s) {
  switch (s) {
    case DPF_OK: return "DPF_OK";
    case DPF_ERR_INVALID_ARGUMENT: return "DPF_ERR_INVALID_ARGUMENT";
    case DPF_ERR_UNSUPPORTED: return "DPF_ERR_UNSUPPORTED";
    case DPF_ERR_OUT_OF_MEMORY: return "DPF_ERR_OUT_OF_MEMORY";
    case DPF_ERR_HIP: return "DPF_ERR_HIP";
  }
  return "DPF_UNKNOWN_STATUS";
}

const char* dpfused_last_error(void) { return g_last_error.c_str(); }

int32_t dpfused_abi_version(void) { return DPFUSED_ABI_VERSION; }

}  // extern "C"
