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

namespace {

thread_local std::string g_last_error;
std::atomic<int> g_norm_path{0};   // 0 auto, 1 gram, 2 direct, 3 staged
std::atomic<int> g_timing{0};
std::atomic<int> g_trace{0};        // roctx range around every entry point
std::atomic<int> g_debug{0};        // synchronise after every launch, report errors
std::atomic<int64_t> g_ws_limit{0};   // workspace requests above this fail (0: no limit)

// Defaults from the environment, read once when the library is loaded:
// DPFUSED_NORM_PATH (auto, gram, direct, staged or 0-3), DPFUSED_TRACE,
// DPFUSED_DEBUG (0/1), DPFUSED_WS_LIMIT (bytes).
bool read_env() {
  if (const char* v = std::getenv("DPFUSED_NORM_PATH")) {
    const std::string t(v);
    const int path = t == "gram" ? 1 : t == "direct" ? 2 : t == "staged" ? 3
                   : (t.size() == 1 && t[0] >= '0' && t[0] <= '3') ? t[0] - '0' : 0;
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

// Rates used to price the norm paths against each other on the large-tile
// path, measured on MI355X at the Llama-13B, GPT-2 and RoBERTa shapes (flops
// or bytes per microsecond): the direct and staged norm kernels run the
// token contraction at ~1.25 PFLOP/s, the accumulate kernel at ~1.15, the
// Gram kernel at ~1.05 plus ~25 us of fills and fixup; the staged tiles
// cost ~1/20 us per MB to store (beyond the contraction: the persistent
// kernel's stores overlap the next unit's fill) and are read back at ~5 TB/s.
constexpr double kNormPerUs = 1.25e9, kAccPerUs = 1.15e9, kGramPerUs = 1.05e9;
constexpr double kStorePerUs = 20.0e6, kCombinePerUs = 5.0e6;
constexpr double kGramFixedUs = 25.0, kAccFixedUs = 15.0, kCombineFixedUs = 5.0;

// allow_staged: the caller keeps the per-sample tiles from the norm phase to
// the accumulate phase (the single-layer calls, and group clipping, which
// holds every linear's tiles until the group's clip factors exist).
dpf::NormPath choose_path(const dpf::LayerArgs& a, bool vec, bool allow_staged) {
  const bool big = dpf::big_path(a, vec);
  const double staged_bytes = (double)dpf::staged_big_workspace_bytes(a);
  const bool staged_ok = allow_staged && big && staged_bytes <= kStagedMaxBytes &&
                         (double)a.B * dpf::big_tiles(a.din, a.dout) < 2147483647.0;
  const int forced = g_norm_path.load();
  if (forced == 1) return dpf::NormPath::kGram;
  if (forced == 2) return dpf::NormPath::kDirect;
  if (forced == 3) return staged_ok ? dpf::NormPath::kStaged : dpf::NormPath::kDirect;
  const double T = a.T, din = a.din, dout = a.dout;
  const double direct = 2.0 * T * din * dout;   // flops per sample
  if (big) {
    // The large-tile Gram kernel works on 256 x 256 token blocks (padded),
    // with a fixed cost per block (two pipeline fills, a parked X Gram):
    // measured on MI355X it beats the direct kernel once it needs at most
    // half the direct kernel's flops.
    const double gram = 2.0 * dpf::gram_big_items_per_sample(a.T) * 65536.0 * (din + dout);
    const bool use_gram = 2.0 * gram <= direct;
    const dpf::NormPath two_pass = use_gram ? dpf::NormPath::kGram : dpf::NormPath::kDirect;
    // Staged: the direct kernel, storing its tiles, then a read of them in
    // place of the accumulate kernel's second contraction.  Masked calls
    // keep the two-pass paths: the host does not know their active tokens.
    if (staged_ok && a.mask == nullptr) {
      const double acc = a.B * direct;   // the contraction both forms run once
      const double t_two_pass =
          (use_gram ? a.B * gram / kGramPerUs + kGramFixedUs : acc / kNormPerUs) +
          acc / kAccPerUs + kAccFixedUs;
      const double t_staged = acc / kNormPerUs + staged_bytes / kStorePerUs +
                              staged_bytes / kCombinePerUs + kCombineFixedUs;
      if (t_staged < t_two_pass) return dpf::NormPath::kStaged;
    }
    return two_pass;
  }
  // Gram costs T^2 (din + dout) per sample, the direct form 2 T din dout.
  return T * T * (din + dout) <= direct ? dpf::NormPath::kGram : dpf::NormPath::kDirect;
}

// Per-device stream-ordered memory pool for workspace (everything but the
// staged tiles, which have a buffer of their own below).  It keeps up to
// g_keep_bytes reserved across synchronisations (the default pool returns
// freed memory at every synchronisation), so workspace is not mapped afresh
// on every step.
std::atomic<int64_t> g_keep_bytes{(int64_t)16 << 30};
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

// The staged per-sample tiles (up to gigabytes) live in one buffer per device
// that the library keeps and grows, not in the pool: pool allocations of that
// size, freed and made again by calls on several streams, were measured to
// stall for tens of milliseconds on MI355X.  Calls on any stream take the
// buffer in turn: each one's stream first waits (on the GPU) for the event
// recorded after the previous holder's last use, and records its own after
// its last launch.  A buffer larger than g_keep_bytes is freed after use.
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
  // Holds the calling thread's device buffer of at least `bytes` for work
  // queued on `s` until release(); false if it cannot be had.
  bool acquire(hipStream_t s, size_t bytes) {
    const int dev = stream_device(s);
    if (dev < 0 || dev >= kMaxDevices) return false;
    if (over_limit(bytes)) return false;
    buf_ = &g_staged[dev];
    lk_ = std::unique_lock<std::mutex>(buf_->mu);
    s_ = s;
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
    return true;
  }
  void* ptr() const { return held_ ? buf_->ptr : nullptr; }
  void release() {
    if (!held_) return;
    held_ = false;
    if (hipEventRecord(buf_->last, s_) == hipSuccess) buf_->recorded = true;
    if ((int64_t)buf_->size > g_keep_bytes.load()) {
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
  explicit Workspace(hipStream_t st) : s(st) {}
  ~Workspace() {
    if (base == nullptr) return;
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
    // A stream being captured into a graph (or one whose state cannot be
    // read) gets plain stream-ordered pool memory: kept blocks are ordered by
    // events recorded outside any capture.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    bool cacheable = false;
    if (hipStreamIsCapturing(s, &cs) == hipSuccess) cacheable = cs == hipStreamCaptureStatusNone;
    else (void)hipGetLastError();
    dev = cacheable ? stream_device(s) : -1;
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
                     bool allow_staged = false) {
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
  L.path = choose_path(L.args, L.vec, allow_staged);
  L.np = dpf::norm_partials_per_sample(L.args, L.path, L.vec);
  return L;
}

// Workspace pieces of one layer call (offsets into a Workspace).
struct LayerWs {
  size_t bits = 0, steps = 0, part = 0, c = 0, sk = 0;
  bool has_steps = false, has_sk = false;
  size_t staged = 0;   // staged path: bytes of per-sample tiles (held in a StagedLease)
};

// Reserve what the call needs: row bits and the active-step list when
// masked, norm partials, clip factors, split-tile accumulate partials.
LayerWs reserve_layer(const LayerPlan& L, Workspace& ws, bool norm, bool clip, bool accum) {
  LayerWs o;
  const dpf::LayerArgs& a = L.args;
  if (a.mask != nullptr) {
    o.bits = ws.reserve((size_t)a.B * a.nwords * sizeof(uint32_t));
    if (dpf::big_path(a, L.vec)) {
      o.has_steps = true;
      o.steps = ws.reserve(dpf::step_list_words(a.B, a.nwords) * sizeof(uint32_t));
    }
  }
  if (norm) o.part = ws.reserve((size_t)a.B * L.np * sizeof(double));
  if (clip) o.c = ws.reserve((size_t)a.B * sizeof(float));
  if (L.path == dpf::NormPath::kStaged) {
    o.staged = dpf::norm_workspace_bytes(a, L.path, L.vec);
    return o;
  }
  size_t bytes = 0;   // split-piece partials; the norm and accumulate phases share them
  if (norm) bytes = dpf::norm_workspace_bytes(a, L.path, L.vec);
  if (accum) bytes = std::max(bytes, dpf::accumulate_workspace_bytes(a, L.vec));
  if (bytes != 0) {
    o.has_sk = true;
    o.sk = ws.reserve(bytes);
  }
  return o;
}

// Once the workspace is allocated: point the layer at its pieces and queue
// the row bits and the active-step list of a masked call.
hipError_t bind_layer(LayerPlan& L, const Workspace& ws, const LayerWs& o, hipStream_t s) {
  dpf::LayerArgs& a = L.args;
  a.rowbits = nullptr;
  a.steps = o.has_steps ? ws.at<uint32_t>(o.steps) : nullptr;
  a.skws = o.has_sk ? ws.at<float>(o.sk) : nullptr;
  if (a.mask == nullptr) return hipSuccess;
  uint32_t* bits = ws.at<uint32_t>(o.bits);
  hipError_t e = dpf::launch_row_bits(a.mask, a.B, a.T, bits, a.nwords, s);
  if (e != hipSuccess) return e;
  a.rowbits = bits;
  if (o.has_steps) e = dpf::launch_step_list(bits, a.B, a.nwords, ws.at<uint32_t>(o.steps), s);
  return e;
}

// Accumulate phase of a single-layer call: the staged path combines the
// tiles its norm phase stored; the others run the scaled contraction.
hipError_t accumulate_phase(const LayerPlan& L, hipStream_t s) {
  if (L.path == dpf::NormPath::kStaged) return dpf::launch_staged_combine(L.args, s);
  return dpf::launch_accumulate(L.args, L.vec, s);
}

dpf_status fused_layer(const dpf_act* X, const dpf_act* G, const uint8_t* mask, float C,
                       float sigma, uint64_t seed, uint64_t offset, float denom, int beta,
                       float* grad_out, float* norms_out, hipStream_t s, Workspace& ws) {
  LayerPlan L = plan_layer(X, G, mask, true);
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
  hipError_t e = bind_layer(L, ws, o, s);
  if (e != hipSuccess) return hip_fail(e, "mask preparation launch");
  StagedLease lease;   // the staged path's per-sample tiles, until the combine is queued
  if (L.path == dpf::NormPath::kStaged) {
    if (!lease.acquire(s, o.staged))
      return fail(DPF_ERR_OUT_OF_MEMORY, "staged workspace allocation failed");
    L.args.skws = static_cast<float*>(lease.ptr());
  }
  L.args.partials = ws.at<double>(o.part);
  e = dpf::launch_norm(L.args, L.path, L.vec, s);
  if (e != hipSuccess) return hip_fail(e, "norm kernel launch");
  float* c = ws.at<float>(o.c);
  e = dpf::launch_finalize(L.args.partials, L.args.B, L.np, nullptr, 0, C, c, norms_out, s);
  if (e != hipSuccess) return hip_fail(e, "finalize launch");
  L.args.c = c;
  L.args.noise_std = sigma * C;
  L.args.seed = seed;
  L.args.offset = offset;
  L.args.out = grad_out;
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

// Shared body of the projected calls: P read from memory (gen == 0) or
// regenerated from (p_seed, p_offset, p_scale) inside the projection.
dpf_status projected_layer(const dpf_act* X, const dpf_act* G, const uint8_t* mask, const void* P,
                           int gen, uint64_t p_seed, uint64_t p_offset, float p_scale, int64_t r,
                           float C, float sigma, uint64_t seed, uint64_t offset, float* grad_out,
                           float* norms_out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t es = elem_size(X->dtype);

  Workspace ws(s);
  const size_t off_y = ws.reserve((size_t)X->B * X->T * r * es);
  dpf::ProjArgs pa{};
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
  pa.splits = dpf::project_splits(pa);
  const size_t pbytes = dpf::project_workspace_bytes(pa);
  const size_t off_part = pbytes != 0 ? ws.reserve(pbytes) : 0;
  // Reserve the layer workspace now so that a single allocation covers both.
  dpf_act Y{nullptr, X->dtype, 0, X->B, X->T, r, X->T * r, r};
  LayerPlan L = plan_layer(&Y, G, mask, true);
  const LayerWs o = reserve_layer(L, ws, true, true, true);
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  Y.data = ws.at<void>(off_y);
  pa.Y = const_cast<void*>(Y.data);
  pa.part = pbytes != 0 ? ws.at<float>(off_part) : nullptr;
  const bool pvec = vec_ok(X) && ((size_t)r * es) % 16 == 0;
  hipError_t e = dpf::launch_project(pa, pvec, s);
  if (e != hipSuccess) return hip_fail(e, "projection launch");

  L = plan_layer(&Y, G, mask, true);
  e = bind_layer(L, ws, o, s);
  if (e != hipSuccess) return hip_fail(e, "mask preparation launch");
  StagedLease lease;   // the staged path's per-sample tiles, until the combine is queued
  if (L.path == dpf::NormPath::kStaged) {
    if (!lease.acquire(s, o.staged))
      return fail(DPF_ERR_OUT_OF_MEMORY, "staged workspace allocation failed");
    L.args.skws = static_cast<float*>(lease.ptr());
  }

  L.args.partials = ws.at<double>(o.part);
  e = dpf::launch_norm(L.args, L.path, L.vec, s);
  if (e != hipSuccess) return hip_fail(e, "norm kernel launch");
  float* c = ws.at<float>(o.c);
  e = dpf::launch_finalize(L.args.partials, L.args.B, L.np, nullptr, 0, C, c, norms_out, s);
  if (e != hipSuccess) return hip_fail(e, "finalize launch");
  L.args.c = c;
  L.args.noise_std = sigma * C;
  L.args.seed = seed;
  L.args.offset = offset;
  L.args.out = grad_out;
  e = accumulate_phase(L, s);
  if (e != hipSuccess) return hip_fail(e, "accumulate launch");
  return ok();
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
  L.args.partials = ws.at<double>(o.part);
  e = dpf::launch_norm(L.args, L.path, L.vec, s);
  if (e != hipSuccess) return hip_fail(e, "norm kernel launch");
  e = dpf::launch_finalize(L.args.partials, L.args.B, L.np, sq, accumulate ? 1 : 0, 1.0f, nullptr,
                           nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "finalize launch");
  return ok();
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
  TraceRange trace_("dpfused_linear_clip_accumulate");
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
  TraceRange trace_("dpfused_linear_clip_accumulate_ex");
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

dpf_status dpfused_linear_clip_accumulate_projected(const dpf_act* X, const dpf_act* G,
                                                    const uint8_t* mask, const void* P, int64_t r,
                                                    float C, float sigma, uint64_t seed,
                                                    uint64_t offset, float* grad_out,
                                                    float* norms_out, void* stream) {
  TraceRange trace_("dpfused_linear_clip_accumulate_projected");
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

dpf_status dpfused_linear_clip_accumulate_projected_seeded(
    const dpf_act* X, const dpf_act* G, const uint8_t* mask, int64_t r, uint64_t p_seed,
    uint64_t p_offset, float p_scale, float C, float sigma, uint64_t seed, uint64_t offset,
    float* grad_out, float* norms_out, void* stream) {
  TraceRange trace_("dpfused_linear_clip_accumulate_projected_seeded");
  dpf_status st = check_pair(X, G);
  if (st != DPF_OK) return st;
  if ((st = check_clip(C, sigma)) != DPF_OK) return st;
  if (r < 1) return fail(DPF_ERR_INVALID_ARGUMENT, "r must be >= 1");
  if (r > kMaxDim) return fail(DPF_ERR_UNSUPPORTED, "r too large");
  if (r % 8 != 0) return fail(DPF_ERR_UNSUPPORTED, "r must be a multiple of 8");
  if (!std::isfinite(p_scale)) return fail(DPF_ERR_INVALID_ARGUMENT, "p_scale must be finite");
  if (grad_out == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "grad_out is NULL");
  if (!aligned16(grad_out)) return fail(DPF_ERR_UNSUPPORTED, "grad_out is not 16-byte aligned");
  return projected_layer(X, G, mask, nullptr, 1, p_seed, p_offset, p_scale, r, C, sigma, seed,
                         offset, grad_out, norms_out, stream);
}

dpf_status dpfused_per_sample_sqnorms(const dpf_act* X, const dpf_act* G, const uint8_t* mask,
                                      double* sqnorms_out, int32_t accumulate, void* stream) {
  TraceRange trace_("dpfused_per_sample_sqnorms");
  dpf_status st = check_pair(X, G);
  if (st != DPF_OK) return st;
  if (sqnorms_out == nullptr) return fail(DPF_ERR_INVALID_ARGUMENT, "sqnorms_out is NULL");
  return sqnorms_into(X, G, mask, sqnorms_out, accumulate, static_cast<hipStream_t>(stream));
}

dpf_status dpfused_clip_factors(const double* sqnorms, int64_t n, float C, float* c_out,
                                float* norms_out, void* stream) {
  TraceRange trace_("dpfused_clip_factors");
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
  TraceRange trace_("dpfused_scaled_accumulate");
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
  TraceRange trace_("dpfused_linear_clip_accumulate_bias");
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
  Workspace ws(s);
  const size_t off_sq = ws.reserve((size_t)B * sizeof(double));
  const size_t off_c = ws.reserve((size_t)B * sizeof(float));
  const size_t off_gb = ws.reserve((size_t)B * dout * sizeof(float));
  const size_t off_part = ws.reserve(dpf::bias_workspace_bytes((int)B, (int)G->T, (int)dout));
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  double* sq = ws.at<double>(off_sq);
  float* c = ws.at<float>(off_c);
  float* gb = ws.at<float>(off_gb);
  // On the staged path the weight's per-sample tiles are kept until the
  // clip factors (which need the bias's norms too) exist.
  LayerPlan L = plan_layer(X, G, mask, true);
  const bool staged = L.path == dpf::NormPath::kStaged;
  Workspace lws(s);
  StagedLease lease;
  hipError_t e = hipSuccess;
  // ||g_i||^2 of the weight, then + ||gb_i||^2 of the bias
  if (staged) {
    const LayerWs o = reserve_layer(L, lws, true, false, false);
    if (!lws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
    if ((e = bind_layer(L, lws, o, s)) != hipSuccess) return hip_fail(e, "mask preparation launch");
    if (!lease.acquire(s, o.staged))
      return fail(DPF_ERR_OUT_OF_MEMORY, "staged workspace allocation failed");
    L.args.skws = static_cast<float*>(lease.ptr());
    L.args.partials = lws.at<double>(o.part);
    if ((e = dpf::launch_norm(L.args, L.path, L.vec, s)) != hipSuccess)
      return hip_fail(e, "norm kernel launch");
    e = dpf::launch_finalize(L.args.partials, L.args.B, L.np, sq, 0, 1.0f, nullptr, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "finalize launch");
  } else if ((st = sqnorms_into(X, G, mask, sq, 0, s)) != DPF_OK) {
    return st;
  }
  e = dpf::launch_bias_grads(to_act(G), G->dtype, (int)B, (int)G->T, (int)dout, mask,
                             ws.at<float>(off_part), gb, sq, s);
  if (e != hipSuccess) return hip_fail(e, "bias gradient launch");
  e = dpf::launch_clip_from_sq(sq, B, C, c, norms_out, s);
  if (e != hipSuccess) return hip_fail(e, "clip factor launch");
  if (staged) {
    L.args.c = c;
    L.args.noise_std = sigma * C;
    L.args.seed = seed;
    L.args.offset = offset;
    L.args.out = grad_out;
    if ((e = dpf::launch_staged_combine(L.args, s)) != hipSuccess)
      return hip_fail(e, "accumulate launch");
  } else if ((st = accumulate_with(X, G, mask, c, sigma * C, seed, offset, grad_out, s)) !=
             DPF_OK) {
    return st;
  }
  // the bias noise continues the weight's Philox stream
  const uint64_t boff = offset + (uint64_t)((dout * X->D + 3) / 4);
  e = dpf::launch_bias_accumulate(gb, c, (int)B, (int)dout, sigma * C, seed, boff, bias_grad_out,
                                  s);
  if (e != hipSuccess) return hip_fail(e, "bias accumulate launch");
  return ok();
}

dpf_status dpfused_group_clip_accumulate(int32_t n, const dpf_act* X, const dpf_act* G,
                                         const uint8_t* mask, float C, float sigma, uint64_t seed,
                                         const uint64_t* offsets, float* const* grad_out,
                                         float* norms_out, void* stream) {
  TraceRange trace_("dpfused_group_clip_accumulate");
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t B = X[0].B;
  Workspace ws(s);
  const size_t off_sq = ws.reserve((size_t)B * sizeof(double));
  const size_t off_c = ws.reserve((size_t)B * sizeof(float));
  if (!ws.allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
  double* sq = ws.at<double>(off_sq);
  float* c = ws.at<float>(off_c);
  // A linear on the staged path keeps its per-sample tiles, in a workspace of
  // its own, from its norm phase until its accumulate phase (after the
  // group's clip factors exist).  The group's staged tiles stay within the
  // per-call limit; the linears past it take their two-pass path.
  struct StagedLinear {
    LayerPlan L;
    std::unique_ptr<Workspace> ws;
    size_t at = 0;   // offset of its tiles in the staged buffer
    bool on = false;
  };
  std::vector<StagedLinear> lin((size_t)n);
  size_t staged_total = 0;
  for (int32_t l = 0; l < n; ++l) {
    StagedLinear& z = lin[(size_t)l];
    z.L = plan_layer(&X[l], &G[l], mask, true);
    if (z.L.path != dpf::NormPath::kStaged) continue;
    const size_t bytes = dpf::staged_big_workspace_bytes(z.L.args);
    if ((double)(staged_total + bytes) > kStagedMaxBytes) continue;
    z.at = staged_total;
    staged_total = (staged_total + bytes + 255) & ~(size_t)255;
    z.ws.reset(new Workspace(s));
    const LayerWs o = reserve_layer(z.L, *z.ws, true, false, false);
    if (!z.ws->allocate()) return fail(DPF_ERR_OUT_OF_MEMORY, "workspace allocation failed");
    hipError_t e = bind_layer(z.L, *z.ws, o, s);
    if (e != hipSuccess) return hip_fail(e, "mask preparation launch");
    z.L.args.partials = z.ws->at<double>(o.part);
    z.on = true;
  }
  StagedLease lease;
  if (staged_total != 0) {
    if (!lease.acquire(s, staged_total))
      return fail(DPF_ERR_OUT_OF_MEMORY, "staged workspace allocation failed");
    for (auto& z : lin)
      if (z.on) z.L.args.skws = reinterpret_cast<float*>(static_cast<char*>(lease.ptr()) + z.at);
  }
  // norm phase of every linear: n_i^2 summed over the group
  for (int32_t l = 0; l < n; ++l) {
    StagedLinear& z = lin[(size_t)l];
    if (!z.on) {
      if ((st = sqnorms_into(&X[l], &G[l], mask, sq, l > 0, s)) != DPF_OK) return st;
      continue;
    }
    hipError_t e = dpf::launch_norm(z.L.args, z.L.path, z.L.vec, s);
    if (e != hipSuccess) return hip_fail(e, "norm kernel launch");
    e = dpf::launch_finalize(z.L.args.partials, z.L.args.B, z.L.np, sq, l > 0 ? 1 : 0, 1.0f,
                             nullptr, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "finalize launch");
  }
  hipError_t e = dpf::launch_clip_from_sq(sq, B, C, c, norms_out, s);
  if (e != hipSuccess) return hip_fail(e, "clip factor launch");
  // accumulate phase of every linear with the group's factors
  for (int32_t l = 0; l < n; ++l) {
    StagedLinear& z = lin[(size_t)l];
    if (!z.on) {
      if ((st = accumulate_with(&X[l], &G[l], mask, c, sigma * C, seed, offsets[l], grad_out[l],
                                s)) != DPF_OK)
        return st;
      continue;
    }
    z.L.args.c = c;
    z.L.args.noise_std = sigma * C;
    z.L.args.seed = seed;
    z.L.args.offset = offsets[l];
    z.L.args.out = grad_out[l];
    e = dpf::launch_staged_combine(z.L.args, s);
    if (e != hipSuccess) return hip_fail(e, "accumulate launch");
  }
  return ok();
}

dpf_status dpfused_projected_adam_step(const float* grad, float* m, float* v, float* W,
                                       int64_t dout, int64_t din, int64_t r, int64_t step,
                                       float lr, float beta1, float beta2, float eps,
                                       const void* P, int32_t p_dtype, uint64_t p_seed,
                                       uint64_t p_offset, float p_scale, void* stream) {
  TraceRange trace_("dpfused_projected_adam_step");
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
  if (P == nullptr && !std::isfinite(p_scale))
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
  a.p_scale = p_scale;
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
  TraceRange trace_("dpfused_philox4x32_10");
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
  TraceRange trace_("dpfused_gaussian_fill");
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
    if (value < 0 || value > 3)
      return fail(DPF_ERR_INVALID_ARGUMENT, "norm_path must be 0, 1, 2 or 3");
    g_norm_path.store((int)value);
    return ok();
  }
  if (std::strcmp(name, "workspace_keep_bytes") == 0) {
    if (value < 0) return fail(DPF_ERR_INVALID_ARGUMENT, "workspace_keep_bytes must be >= 0");
    set_keep_bytes(value);
    return ok();
  }
  if (std::strcmp(name, "workspace_limit_bytes") == 0) {
    if (value < 0) return fail(DPF_ERR_INVALID_ARGUMENT, "workspace_limit_bytes must be >= 0");
    g_ws_limit.store(value);
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
  if (std::strcmp(name, "timing") == 0) return g_timing.load();
  if (std::strcmp(name, "workspace_keep_bytes") == 0) return g_keep_bytes.load();
  if (std::strcmp(name, "workspace_limit_bytes") == 0) return g_ws_limit.load();
  if (std::strcmp(name, "p_in_kernels") == 0) return dpf::p_in_kernels() ? 1 : 0;
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
