// extern "C" entry points of libmole.so: argument checks on the host, then
// kernel dispatch on the caller's stream.  Declarations and contracts are in
// include/mole.h.
#include <hip/hip_runtime.h>

#include <fcntl.h>
#include <sys/uio.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <cerrno>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <unordered_map>
#include <vector>

#include "../../include/mole.h"
#include "mole_kernels.hpp"
#include "mole_tables.hpp"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t err) {
  if (err == hipSuccess) return MOLE_OK;
  g_last_hip_error = (int)err;
  return MOLE_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool dtype_ok(int dt) { return dt == MOLE_F32 || dt == MOLE_BF16; }
hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // sizes handed to kernels as int
constexpr int64_t kMaxExperts = 64;             // combine kernels keep N gates in registers
constexpr int64_t kMaxCombineDim = (int64_t)1 << 20;  // the routers address h and W_r rows with 32-bit offsets
constexpr int64_t kMaxPanelStride = (int64_t)1 << 22;  // bf16 build: row stride of G and of the LUT

int check_combine_common(int64_t T, int64_t V, int64_t D, int64_t N) {
  if (T < 0 || V <= 0 || D <= 0 || N <= 0) return MOLE_ERR_DIM;
  if (D > kMaxDim || T > kMaxDim) return MOLE_ERR_DIM;
  if (N > kMaxExperts || D > kMaxCombineDim) return MOLE_ERR_UNSUPPORTED;
  return MOLE_OK;
}

// Deduplicate ids in first-occurrence order.  Returns MOLE_ERR_ID on a bad id.
int dedupe(const int64_t* ids, int64_t T, int64_t V, std::vector<int64_t>& uniq, int64_t* remap) {
  std::unordered_map<int64_t, int64_t> pos;
  pos.reserve((size_t)T * 2 + 1);
  uniq.clear();
  for (int64_t t = 0; t < T; ++t) {
    const int64_t id = ids[t];
    if (id < 0 || id >= V) return MOLE_ERR_ID;
    auto it = pos.find(id);
    if (it == pos.end()) {
      const int64_t u = (int64_t)uniq.size();
      pos.emplace(id, u);
      uniq.push_back(id);
      remap[t] = u;
    } else {
      remap[t] = it->second;
    }
  }
  return MOLE_OK;
}

// Host worker threads for the gathers, created on first use and kept for
// the life of the process (spawning a thread per worker and call cost
// about 10 us each, more than a small batch's copies).  reserve(n) makes
// sure up to n workers exist and returns how many do (fewer if the system
// refuses more threads, 0 if none).  start(n, fn), n <= reserve's answer,
// runs fn(0) .. fn(n-1) on n pool threads and returns at once; wait()
// returns when all have finished.  One job at a time: a second caller's
// start() blocks until the first caller's wait().
class WorkerPool {
 public:
  static constexpr int kMaxWorkers = 64;
  static WorkerPool& instance() {
    static WorkerPool* p = new WorkerPool();  // never destroyed: its threads outlive static destructors
    return *p;
  }
  int reserve(int n) {
    std::lock_guard<std::mutex> lk(mu_);
    while (nthreads_ < n) {
      try {
        std::thread(&WorkerPool::loop, this).detach();
      } catch (...) {
        break;  // no more threads: run with those there are
      }
      ++nthreads_;
    }
    return std::min(n, nthreads_);
  }
  void start(int n, std::function<void(int)> fn) {
    job_mu_.lock();
    std::unique_lock<std::mutex> lk(mu_);
    fn_ = std::move(fn);
    want_ = n;
    claimed_ = 0;
    pending_ = n;
    ++gen_;
    lk.unlock();
    cv_.notify_all();
  }
  void wait() {
    {
      std::unique_lock<std::mutex> lk(mu_);
      done_cv_.wait(lk, [&] { return pending_ == 0; });
      fn_ = nullptr;
    }
    job_mu_.unlock();
  }
  // Ends every worker thread (after any job in flight) and waits until they
  // have left; a later reserve() starts new ones.
  void shutdown() {
    std::lock_guard<std::mutex> job(job_mu_);
    std::unique_lock<std::mutex> lk(mu_);
    stop_ = true;
    ++gen_;
    cv_.notify_all();
    done_cv_.wait(lk, [&] { return nthreads_ == 0; });
    stop_ = false;
  }

 private:
  void loop() {
    uint64_t seen = 0;
    std::unique_lock<std::mutex> lk(mu_);
    for (;;) {
      cv_.wait(lk, [&] { return gen_ != seen; });
      seen = gen_;
      if (stop_) {
        if (--nthreads_ == 0) done_cv_.notify_all();
        return;
      }
      if (claimed_ >= want_) continue;  // this job needs fewer workers
      const int idx = claimed_++;
      std::function<void(int)>* fn = &fn_;
      lk.unlock();
      (*fn)(idx);  // fn_ is not replaced before pending_ reaches 0
      lk.lock();
      if (--pending_ == 0) done_cv_.notify_all();
    }
  }
  std::mutex job_mu_, mu_;
  std::condition_variable cv_, done_cv_;
  std::function<void(int)> fn_;
  int nthreads_ = 0, want_ = 0, claimed_ = 0, pending_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

int default_threads(int nthreads, int cap) {
  const int hw = (int)std::max(1u, std::thread::hardware_concurrency());
  return std::min(WorkerPool::kMaxWorkers, nthreads > 0 ? nthreads : std::min(cap, hw));
}

// work(lo, hi) over [0, n) in nt equal ranges on the pool (inline for nt <= 1
// or when no worker thread can be had).
void parallel_ranges(int64_t n, int nt, const std::function<void(int64_t, int64_t)>& work) {
  nt = (int)std::min<int64_t>(nt, std::max<int64_t>(n, 1));
  WorkerPool& pool = WorkerPool::instance();
  if (nt > 1) nt = pool.reserve(nt);
  if (nt <= 1) {
    work(0, n);
    return;
  }
  const int64_t per = (n + nt - 1) / nt;
  pool.start(nt, [&](int w) {
    const int64_t lo = std::min<int64_t>(n, w * per), hi = std::min<int64_t>(n, lo + per);
    if (lo < hi) work(lo, hi);
  });
  pool.wait();
}

void gather_rows(const std::vector<int64_t>& uniq, const uint8_t* codes, const uint16_t* scales,
                 int64_t N, int64_t D, uint8_t* codes_out, uint16_t* scales_out, int nthreads) {
  const size_t crow = (size_t)(N * 3 * D / 8), srow = (size_t)(N * (D / 64));
  const int64_t U = (int64_t)uniq.size();
  auto work = [&](int64_t lo, int64_t hi) {
    for (int64_t u = lo; u < hi; ++u) {
      std::memcpy(codes_out + (size_t)u * crow, codes + (size_t)uniq[u] * crow, crow);
      std::memcpy(scales_out + (size_t)u * srow, scales + (size_t)uniq[u] * srow, srow * 2);
    }
  };
  int nt = default_threads(nthreads, 16);
  const size_t bytes = (size_t)U * (crow + 2 * srow);
  if (bytes < ((size_t)1 << 20)) nt = 1;  // workers are not worth it below ~1 MB
  parallel_ranges(U, nt, work);
}

// One event per pinned staging area of the host-resident combine, recorded
// after the copy out of it: the next call that reuses the area waits for
// that copy only, not for everything queued on the stream.  Created on first
// use and kept for the life of the process (a few bytes per distinct area).
std::mutex g_stage_mu;
std::unordered_map<const void*, hipEvent_t> g_stage_events;

int stage_event(const void* stage_host, hipEvent_t* ev) {
  std::lock_guard<std::mutex> lock(g_stage_mu);
  auto it = g_stage_events.find(stage_host);
  if (it != g_stage_events.end()) {
    *ev = it->second;
    return MOLE_OK;
  }
  const int rc = hip_status(hipEventCreateWithFlags(ev, hipEventDisableTiming));
  if (rc == MOLE_OK) g_stage_events.emplace(stage_host, *ev);
  return rc;
}

// Staging area of the host-resident combine for T tokens and U distinct
// ids: remap int64[T] | codes [U][N][3D/8] | scales fp16 [U][N][D/64],
// each section 16-byte aligned.  total = bytes in use.
struct Nf3Staging {
  size_t codes_off, scales_off, total;
};
inline size_t round16(size_t x) { return (x + 15u) & ~(size_t)15u; }
Nf3Staging nf3_staging(int64_t T, int64_t U, int64_t N, int64_t D) {
  Nf3Staging st;
  st.codes_off = round16((size_t)T * 8u);
  st.scales_off = st.codes_off + round16((size_t)U * (size_t)(N * 3 * D / 8));
  st.total = st.scales_off + (size_t)U * (size_t)(N * (D / 64)) * 2u;
  return st;
}

// Staging area of the layer-stack prefetch for T tokens, U distinct ids and
// L layers: remap int64[T], then per layer codes [U][N][3D/8] and scales
// fp16 [U][N][D/64], each section 16-byte aligned.
size_t nf3_stack_staging(int64_t T, int64_t U, int64_t L, int64_t N, int64_t D, size_t* codes_off,
                         size_t* scales_off) {
  size_t off = round16((size_t)T * 8u);
  for (int64_t l = 0; l < L; ++l) {
    if (codes_off) codes_off[l] = off;
    off += round16((size_t)U * (size_t)(N * 3 * D / 8));
    if (scales_off) scales_off[l] = off;
    off += round16((size_t)U * (size_t)(N * (D / 64)) * 2u);
  }
  return off;
}

// Gather of the U distinct rows of L tables, pipelined with the host->device
// copy: the layers are cut into up to kStackChunks consecutive chunks; every
// worker thread copies its share of chunk k's (layer, row) pairs, then
// counts itself done with k; the calling thread enqueues chunk k's copy
// (one contiguous byte range of the staging area) as soon as every worker
// is done with it, so the bus moves chunk k while chunk k+1 is gathered.
// Returns a mole status.
constexpr int kStackChunks = 4;

int gather_copy_stack(const std::vector<int64_t>& uniq, const uint8_t* const* codes, const uint16_t* const* scales,
                      int64_t L, int64_t N, int64_t D, uint8_t* base_h, uint8_t* base_d,
                      const size_t* codes_off, const size_t* scales_off, size_t total, int nthreads, hipStream_t s) {
  const size_t crow = (size_t)(N * 3 * D / 8), srow = (size_t)(N * (D / 64));
  const int64_t U = (int64_t)uniq.size();
  const int nchunks = (int)std::min<int64_t>(L, kStackChunks);
  // chunk k = layers [l0(k), l0(k+1)); bytes [begin(k), begin(k+1)) of the staging area
  auto l0 = [&](int k) { return (int64_t)k * L / nchunks; };
  auto begin = [&](int k) { return k == 0 ? (size_t)0 : (k == nchunks ? total : codes_off[l0(k)]); };
  auto gather = [&](int k, int64_t lo, int64_t hi) {  // flattened (layer, row) range within chunk k
    const int64_t first = l0(k) * U;
    for (int64_t i = first + lo; i < first + hi; ++i) {
      const int64_t l = i / U, u = i - l * U;
      std::memcpy(base_h + codes_off[l] + (size_t)u * crow, codes[l] + (size_t)uniq[u] * crow, crow);
      std::memcpy(reinterpret_cast<uint16_t*>(base_h + scales_off[l]) + (size_t)u * srow,
                  scales[l] + (size_t)uniq[u] * srow, srow * 2);
    }
  };
  int nt = default_threads(nthreads, 16);
  if ((size_t)(L * U) * (crow + 2 * srow) < ((size_t)1 << 20)) nt = 1;  // workers are not worth it below ~1 MB
  WorkerPool& pool = WorkerPool::instance();
  if (nt > 1) nt = pool.reserve(nt);
  int rc = MOLE_OK;
  if (nt <= 1) {
    for (int k = 0; k < nchunks && rc == MOLE_OK; ++k) {
      gather(k, 0, (l0(k + 1) - l0(k)) * U);
      rc = hip_status(hipMemcpyAsync(base_d + begin(k), base_h + begin(k), begin(k + 1) - begin(k),
                                     hipMemcpyHostToDevice, s));
    }
    return rc;
  }
  std::vector<std::atomic<int>> done(nchunks);
  for (auto& d : done) d.store(0);
  auto worker = [&](int w) {
    for (int k = 0; k < nchunks; ++k) {
      const int64_t n = (l0(k + 1) - l0(k)) * U, per = (n + nt - 1) / nt;
      const int64_t lo = std::min<int64_t>(n, w * per), hi = std::min<int64_t>(n, lo + per);
      if (lo < hi) gather(k, lo, hi);
      done[k].fetch_add(1, std::memory_order_release);
    }
  };
  pool.start(nt, worker);
  for (int k = 0; k < nchunks; ++k) {
    while (done[k].load(std::memory_order_acquire) < nt) std::this_thread::yield();
    if (rc == MOLE_OK)
      rc = hip_status(hipMemcpyAsync(base_d + begin(k), base_h + begin(k), begin(k + 1) - begin(k),
                                     hipMemcpyHostToDevice, s));
  }
  pool.wait();
  return rc;
}


// Host-side entry points allocate (maps, vectors, file buffers) and start
// threads; an exception must not cross the C ABI, so it becomes a status.
template <typename F>
int guarded(F f) {
  try {
    return f();
  } catch (...) {
    return MOLE_ERR_HOST;
  }
}

}  // namespace

extern "C" {

const char* mole_status_string(int status) {
  switch (status) {
    case MOLE_OK: return "ok";
    case MOLE_ERR_NULL: return "a required pointer is NULL";
    case MOLE_ERR_DIM: return "invalid or inconsistent size";
    case MOLE_ERR_DTYPE: return "unknown dtype";
    case MOLE_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MOLE_ERR_WORKSPACE: return "workspace too small";
    case MOLE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOLE_ERR_HIP: return "HIP runtime error (see mole_last_hip_error)";
    case MOLE_ERR_ID: return "token id outside [0, V)";
    case MOLE_ERR_IO: return "table file read or write failed";
    case MOLE_ERR_FORMAT: return "not a MoLE NF3 table file of this version";
    case MOLE_ERR_HOST: return "host memory or thread allocation failed";
    case MOLE_ERR_MEMORY: return "host table not in page-locked memory the device can read";
    default: return "unknown status";
  }
}

int mole_last_hip_error(void) { return g_last_hip_error; }

int mole_abi_version(void) { return 12; }

int mole_release_host_state(void) {
  return guarded([&] {
    WorkerPool::instance().shutdown();
    std::lock_guard<std::mutex> lock(g_stage_mu);
    int rc = MOLE_OK;
    for (auto& kv : g_stage_events) {
      const int r = hip_status(hipEventDestroy(kv.second));
      if (rc == MOLE_OK) rc = r;
    }
    g_stage_events.clear();
    return rc;
  });
}

namespace {
void copy_bits(const uint32_t* bits, int n, float* out) {
  for (int i = 0; i < n; ++i) std::memcpy(out + i, bits + i, 4);
}
}  // namespace

int mole_nf3_levels(float* levels_host) {
  if (!levels_host) return MOLE_ERR_NULL;
  copy_bits(mole::kNf3LevelBits, 8, levels_host);
  return MOLE_OK;
}

int mole_nf3_midpoints(float* mid_host) {
  if (!mid_host) return MOLE_ERR_NULL;
  copy_bits(mole::kNf3MidBits, 7, mid_host);
  return MOLE_OK;
}

int mole_nf4_levels(float* levels_host) {
  if (!levels_host) return MOLE_ERR_NULL;
  copy_bits(mole::kNf4LevelBits, 16, levels_host);
  return MOLE_OK;
}

int mole_nf4_midpoints(float* mid_host) {
  if (!mid_host) return MOLE_ERR_NULL;
  copy_bits(mole::kNf4MidBits, 15, mid_host);
  return MOLE_OK;
}

int mole_gelu_phi_coefficients(float* coef_host, int n, float* range) {
  if (n < mole::kPhiPolyTerms) return MOLE_ERR_DIM;
  if (!coef_host || !range) return MOLE_ERR_NULL;
  for (int i = 0; i < mole::kPhiPolyTerms; ++i) coef_host[i] = mole::kPhiPolyCoef[i];
  *range = mole::kPhiPolyRange;
  return MOLE_OK;
}

int mole_build_lut_workspace_size(int64_t V, int64_t D, int64_t F, int64_t N, int dtype,
                                  size_t* min_bytes, size_t* rec_bytes) {
  if (!dtype_ok(dtype)) return MOLE_ERR_DTYPE;
  if (V <= 0 || D <= 0 || F <= 0 || N <= 0 || D > kMaxDim || F > kMaxDim ||
      N * F > kMaxDim)
    return MOLE_ERR_DIM;
  size_t mn = 0, rec = 0;
  if (dtype == MOLE_BF16) {
    mn = mole::build_lut_min_workspace(D, F, N);
    rec = mole::build_lut_rec_workspace(V, D, F, N);
  }
  if (min_bytes) *min_bytes = mn;
  if (rec_bytes) *rec_bytes = rec;
  return MOLE_OK;
}

int mole_build_lut(const void* emb, const void* w_up, const void* w_down, void* lut, int64_t V,
                   int64_t D, int64_t F, int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (!dtype_ok(dtype)) return MOLE_ERR_DTYPE;
  if (!emb || !w_up || !w_down || !lut) return MOLE_ERR_NULL;
  if (V <= 0 || D <= 0 || F <= 0 || N <= 0 || D > kMaxDim || F > kMaxDim ||
      N * F > kMaxDim || V > kMaxDim)
    return MOLE_ERR_DIM;
  if (!aligned16(emb) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(lut)) return MOLE_ERR_ALIGN;
  if (dtype == MOLE_F32) {
    if (D + F > mole::kBuildF32MaxLds) return MOLE_ERR_UNSUPPORTED;
    return hip_status(mole::launch_build_lut_f32((const float*)emb, (const float*)w_up,
                                                 (const float*)w_down, (float*)lut, V, D, F, N,
                                                 as_stream(stream)));
  }
  if (D % 8 != 0 || F % 8 != 0) return MOLE_ERR_DIM;
  // Each 256-row operand or output panel of the build GEMMs is addressed with
  // 32-bit byte offsets (256 rows x stride x 2 bytes < 2^31).
  if (N * F > kMaxPanelStride || N * D > kMaxPanelStride) return MOLE_ERR_UNSUPPORTED;
  if (!workspace) return MOLE_ERR_NULL;
  if (!aligned16(workspace)) return MOLE_ERR_ALIGN;
  if (workspace_bytes < mole::build_lut_min_workspace(D, F, N)) return MOLE_ERR_WORKSPACE;
  return hip_status(mole::launch_build_lut_bf16((const uint16_t*)emb, (const uint16_t*)w_up,
                                                (const uint16_t*)w_down, (uint16_t*)lut, V, D, F, N,
                                                workspace, workspace_bytes, as_stream(stream)));
}

int mole_lookup_combine(const int64_t* ids, const void* h, const void* w_r, const void* lut, float* y,
                        int64_t T, int64_t V, int64_t D, int64_t N, int dtype, void* stream) {
  if (!dtype_ok(dtype)) return MOLE_ERR_DTYPE;
  int rc = check_combine_common(T, V, D, N);
  if (rc != MOLE_OK) return rc;
  if (T == 0) return MOLE_OK;
  if (!ids || !h || !w_r || !lut || !y) return MOLE_ERR_NULL;
  if (!aligned8(ids) || !aligned16(h) || !aligned16(w_r) || !aligned16(lut) || !aligned16(y))
    return MOLE_ERR_ALIGN;
  return hip_status(mole::launch_lookup_combine(ids, h, w_r, lut, y, T, D, N, dtype, true,
                                                as_stream(stream)));
}

int mole_pack_nf3(const void* lut, uint8_t* codes, uint16_t* scales, int64_t V, int64_t N, int64_t D,
                  int dtype, void* stream) {
  if (!dtype_ok(dtype)) return MOLE_ERR_DTYPE;
  if (V <= 0 || N <= 0 || D <= 0 || D > kMaxDim) return MOLE_ERR_DIM;
  if (D % 64 != 0) return MOLE_ERR_DIM;
  if (!lut || !codes || !scales) return MOLE_ERR_NULL;
  if (!aligned16(lut) || !aligned16(codes) || !aligned16(scales)) return MOLE_ERR_ALIGN;
  return hip_status(mole::launch_pack_nf3(lut, codes, scales, V * N, D, dtype, as_stream(stream)));
}

int mole_lookup_combine_nf3(const int64_t* ids, const void* h, const void* w_r, const uint8_t* codes,
                            const uint16_t* scales, float* y, int64_t T, int64_t V, int64_t D,
                            int64_t N, int dtype_h, void* stream) {
  if (!dtype_ok(dtype_h)) return MOLE_ERR_DTYPE;
  int rc = check_combine_common(T, V, D, N);
  if (rc != MOLE_OK) return rc;
  if (D % 64 != 0) return MOLE_ERR_DIM;
  if (T == 0) return MOLE_OK;
  if (!ids || !h || !w_r || !codes || !scales || !y) return MOLE_ERR_NULL;
  if (!aligned8(ids) || !aligned16(h) || !aligned16(w_r) || !aligned16(codes) || !aligned16(scales) ||
      !aligned16(y))
    return MOLE_ERR_ALIGN;
  return hip_status(mole::launch_lookup_combine_nf3(ids, h, w_r, codes, scales, y, T, D, N, dtype_h,
                                                    as_stream(stream)));
}

// The device address of the host range [p, p + bytes) if all of it lies in
// one page-locked host allocation that the device can read, else null.  (A
// failed query leaves an error behind in the runtime's last-error slot; it is
// cleared so that the caller's next error check does not see it.)  Both ends
// being mapped is not enough: a page-locked allocation's device address
// equals its host address, so a range whose ends fall in two allocations
// passes the end-to-end test with unmapped memory between them.  The range
// must also fit inside the allocation that holds its first byte.
static const char* mapped_host_range(const void* p, size_t bytes) {
  const char* first = static_cast<const char*>(p);
  const char* last = first + bytes - 1;
  const char* dev[2] = {nullptr, nullptr};
  const char* q[2] = {first, last};
  for (int i = 0; i < 2; ++i) {
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, q[i]) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    if (a.type != hipMemoryTypeHost || !a.devicePointer || !a.hostPointer) return nullptr;
    // (the runtime may report the allocation's base or the queried address
    // itself; the offset from its host address covers both)
    dev[i] = static_cast<const char*>(a.devicePointer) + (q[i] - static_cast<const char*>(a.hostPointer));
  }
  if (dev[1] - dev[0] != (ptrdiff_t)(bytes - 1)) return nullptr;
  void* start = nullptr;
  size_t size = 0;
  void* q0 = const_cast<char*>(first);
  if (hipPointerGetAttribute(&start, HIP_POINTER_ATTRIBUTE_RANGE_START_ADDR, q0) != hipSuccess ||
      hipPointerGetAttribute(&size, HIP_POINTER_ATTRIBUTE_RANGE_SIZE, q0) != hipSuccess || !start) {
    (void)hipGetLastError();
    return nullptr;
  }
  // (the start may come back as the allocation's host or device address)
  const char* s0 = static_cast<const char*>(start);
  auto fits = [&](const char* a) { return a >= s0 && (size_t)(a - s0) <= size && size - (size_t)(a - s0) >= bytes; };
  return fits(first) || fits(dev[0]) ? dev[0] : nullptr;
}

int mole_lookup_combine_nf3_mapped(const int64_t* ids, const void* h, const void* w_r, const uint8_t* codes_host,
                                   const uint16_t* scales_host, float* y, int64_t T, int64_t V, int64_t D,
                                   int64_t N, int dtype_h, void* stream) {
  if (!dtype_ok(dtype_h)) return MOLE_ERR_DTYPE;
  int rc = check_combine_common(T, V, D, N);
  if (rc != MOLE_OK) return rc;
  if (D % 64 != 0) return MOLE_ERR_DIM;
  if (T == 0) return MOLE_OK;
  if (!ids || !h || !w_r || !codes_host || !scales_host || !y) return MOLE_ERR_NULL;
  if (!aligned8(ids) || !aligned16(h) || !aligned16(w_r) || !aligned16(codes_host) || !aligned16(scales_host) ||
      !aligned16(y))
    return MOLE_ERR_ALIGN;
  if (V > INT64_MAX / (4 * N * D)) return MOLE_ERR_DIM;  // (the table's byte count must not wrap)
  const char* codes_d = mapped_host_range(codes_host, (size_t)(V * N * (3 * D / 8)));
  const char* scales_d = mapped_host_range(scales_host, (size_t)(V * N * (D / 64)) * 2);
  if (!codes_d || !scales_d) return MOLE_ERR_MEMORY;
  return hip_status(mole::launch_lookup_combine_nf3(ids, h, w_r, reinterpret_cast<const uint8_t*>(codes_d),
                                                    reinterpret_cast<const uint16_t*>(scales_d), y, T, D, N, dtype_h,
                                                    as_stream(stream)));
}

int mole_lookup_combine_mapped(const int64_t* ids, const void* h, const void* w_r, const void* lut_host, float* y,
                               int64_t T, int64_t V, int64_t D, int64_t N, int dtype, void* stream) {
  if (!dtype_ok(dtype)) return MOLE_ERR_DTYPE;
  int rc = check_combine_common(T, V, D, N);
  if (rc != MOLE_OK) return rc;
  if (T == 0) return MOLE_OK;
  if (!ids || !h || !w_r || !lut_host || !y) return MOLE_ERR_NULL;
  if (!aligned8(ids) || !aligned16(h) || !aligned16(w_r) || !aligned16(lut_host) || !aligned16(y))
    return MOLE_ERR_ALIGN;
  const size_t esz = dtype == MOLE_F32 ? 4 : 2;
  if (V > INT64_MAX / (4 * N * D)) return MOLE_ERR_DIM;  // (the table's byte count must not wrap)
  const char* lut_d = mapped_host_range(lut_host, (size_t)(V * N * D) * esz);
  if (!lut_d) return MOLE_ERR_MEMORY;
  return hip_status(mole::launch_lookup_combine(ids, h, w_r, lut_d, y, T, D, N, dtype, true, as_stream(stream)));
}

int mole_pack_nf4(const void* lut, uint8_t* codes, uint16_t* scales, int64_t V, int64_t N, int64_t D,
                  int dtype, void* stream) {
  if (!dtype_ok(dtype)) return MOLE_ERR_DTYPE;
  if (V <= 0 || N <= 0 || D <= 0 || D > kMaxDim || D % 64 != 0) return MOLE_ERR_DIM;
  if (!lut || !codes || !scales) return MOLE_ERR_NULL;
  if (!aligned16(lut) || !aligned16(codes) || !aligned16(scales)) return MOLE_ERR_ALIGN;
  return hip_status(mole::launch_pack_nf4(lut, codes, scales, V * N, D, dtype, as_stream(stream)));
}

int mole_pack_int8(const void* lut, int8_t* codes, float* scales, int64_t V, int64_t N, int64_t D, int dtype,
                   void* stream) {
  if (!dtype_ok(dtype)) return MOLE_ERR_DTYPE;
  if (V <= 0 || N <= 0 || D <= 0 || D > kMaxDim || D % 64 != 0) return MOLE_ERR_DIM;
  if (V * N > kMaxDim) return MOLE_ERR_DIM;  // four rows per workgroup, grid in 32 bits
  if (!lut || !codes || !scales) return MOLE_ERR_NULL;
  if (!aligned16(lut) || !aligned16(codes) || !aligned16(scales)) return MOLE_ERR_ALIGN;
  return hip_status(mole::launch_pack_int8(lut, codes, scales, V * N, D, dtype, as_stream(stream)));
}

namespace {
int combine_q(int fmt, const int64_t* ids, const void* h, const void* w_r, const void* codes, const void* scales,
              float* y, int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h, void* stream) {
  if (!dtype_ok(dtype_h)) return MOLE_ERR_DTYPE;
  int rc = check_combine_common(T, V, D, N);
  if (rc != MOLE_OK) return rc;
  if (D % 64 != 0) return MOLE_ERR_DIM;
  if (T == 0) return MOLE_OK;
  if (!ids || !h || !w_r || !codes || !scales || !y) return MOLE_ERR_NULL;
  if (!aligned8(ids) || !aligned16(h) || !aligned16(w_r) || !aligned16(codes) || !aligned16(scales) ||
      !aligned16(y))
    return MOLE_ERR_ALIGN;
  return hip_status(mole::launch_lookup_combine_q(fmt, ids, h, w_r, static_cast<const uint8_t*>(codes), scales, y,
                                                  T, D, N, dtype_h, as_stream(stream)));
}
}  // namespace

int mole_lookup_combine_nf4(const int64_t* ids, const void* h, const void* w_r, const uint8_t* codes,
                            const uint16_t* scales, float* y, int64_t T, int64_t V, int64_t D, int64_t N,
                            int dtype_h, void* stream) {
  return combine_q(mole::kFmtNf4, ids, h, w_r, codes, scales, y, T, V, D, N, dtype_h, stream);
}

int mole_lookup_combine_int8(const int64_t* ids, const void* h, const void* w_r, const int8_t* codes,
                             const float* scales, float* y, int64_t T, int64_t V, int64_t D, int64_t N,
                             int dtype_h, void* stream) {
  return combine_q(mole::kFmtI8, ids, h, w_r, codes, scales, y, T, V, D, N, dtype_h, stream);
}

static int mole_train_index_impl(const int64_t* ids_host, int64_t T, int64_t V, int64_t* uniq_host, int64_t* remap_host,
                                 int64_t* row_ptr_host, int64_t* tok_host, int64_t* n_unique) {
  if (T < 0 || V <= 0) return MOLE_ERR_DIM;
  if (T > 0 && (!ids_host || !uniq_host || !remap_host || !row_ptr_host || !tok_host)) return MOLE_ERR_NULL;
  if (!n_unique) return MOLE_ERR_NULL;
  std::vector<int64_t> uniq;
  int rc = dedupe(ids_host, T, V, uniq, remap_host);
  if (rc != MOLE_OK) return rc;
  const int64_t U = (int64_t)uniq.size();
  std::copy(uniq.begin(), uniq.end(), uniq_host);
  // Tokens grouped by row, in token order within a row (a counting sort).
  if (row_ptr_host) {
    std::fill(row_ptr_host, row_ptr_host + U + 1, (int64_t)0);
    for (int64_t t = 0; t < T; ++t) row_ptr_host[remap_host[t] + 1] += 1;
    for (int64_t u = 0; u < U; ++u) row_ptr_host[u + 1] += row_ptr_host[u];
    std::vector<int64_t> next(row_ptr_host, row_ptr_host + U);
    for (int64_t t = 0; t < T; ++t) tok_host[next[remap_host[t]]++] = t;
  }
  *n_unique = U;
  return MOLE_OK;
}

int mole_train_index(const int64_t* ids_host, int64_t T, int64_t V, int64_t* uniq_host, int64_t* remap_host,
                     int64_t* row_ptr_host, int64_t* tok_host, int64_t* n_unique) {
  return guarded([&] {
    return mole_train_index_impl(ids_host, T, V, uniq_host, remap_host, row_ptr_host, tok_host, n_unique);
  });
}

namespace {
// 256-row fp32 panels of N*F and D, and 64-row slices of the MN-major
// operands (row pitch N*D or N*F), stay under 2^31 bytes.
constexpr int64_t kMaxTrainDim = (int64_t)1 << 20;

int check_train(int64_t T, int64_t U, int64_t V, int64_t D, int64_t F, int64_t N, int dtype) {
  if (!dtype_ok(dtype)) return MOLE_ERR_DTYPE;
  if (T < 0 || U < 0 || V <= 0 || D <= 0 || F <= 0 || N <= 0) return MOLE_ERR_DIM;
  if (U > T || U > V || (T > 0 && U == 0)) return MOLE_ERR_DIM;
  if (D % 8 != 0 || F % 8 != 0) return MOLE_ERR_DIM;
  if (N > kMaxExperts) return MOLE_ERR_UNSUPPORTED;
  if (dtype != MOLE_BF16) return MOLE_ERR_UNSUPPORTED;
  if (N * D > kMaxTrainDim || N * F > kMaxTrainDim || T > kMaxTrainDim) return MOLE_ERR_UNSUPPORTED;
  return MOLE_OK;
}
}  // namespace

int mole_check_ids(const int64_t* ids, int64_t T, int64_t V, int32_t* count, void* stream) {
  if (T < 0 || V <= 0) return MOLE_ERR_DIM;
  if (T == 0) return MOLE_OK;
  if (!ids || !count) return MOLE_ERR_NULL;
  if (!aligned8(ids) || (reinterpret_cast<uintptr_t>(count) & 3u) != 0) return MOLE_ERR_ALIGN;
  return hip_status(mole::launch_check_ids(ids, T, V, count, as_stream(stream)));
}

int mole_lookup_combine_grouped_workspace_size(int64_t T, size_t* bytes) {
  if (T < 0 || T > kMaxDim) return MOLE_ERR_DIM;
  if (!bytes) return MOLE_ERR_NULL;
  *bytes = T == 0 ? 0 : mole::grouped_workspace_bytes(T);
  return MOLE_OK;
}

namespace {
int check_grouped(const int64_t* ids, const void* h, const void* w_r, const void* lut, float* y, int64_t T,
                  int64_t V, int64_t D, int64_t N, int dtype) {
  if (!dtype_ok(dtype)) return MOLE_ERR_DTYPE;
  int rc = check_combine_common(T, V, D, N);
  if (rc != MOLE_OK) return rc;
  if (dtype != MOLE_BF16 || N > 16 || D % 8 != 0 || V > INT32_MAX) return MOLE_ERR_UNSUPPORTED;
  if (T == 0) return MOLE_OK;
  if (!ids || !h || !w_r || !lut || !y) return MOLE_ERR_NULL;
  if (!aligned8(ids) || !aligned16(h) || !aligned16(w_r) || !aligned16(lut) || !aligned16(y)) return MOLE_ERR_ALIGN;
  return MOLE_OK;
}
}  // namespace

int mole_lookup_combine_grouped(const int64_t* ids, const void* h, const void* w_r, const void* lut, float* y,
                                int64_t T, int64_t V, int64_t D, int64_t N, int dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  int rc = check_grouped(ids, h, w_r, lut, y, T, V, D, N, dtype);
  if (rc != MOLE_OK || T == 0) return rc;
  if (!workspace) return MOLE_ERR_NULL;
  if (!aligned16(workspace)) return MOLE_ERR_ALIGN;
  if (workspace_bytes < mole::grouped_workspace_bytes(T)) return MOLE_ERR_WORKSPACE;
  return hip_status(mole::launch_lookup_combine_grouped(ids, (const uint16_t*)h, (const uint16_t*)w_r,
                                                        (const uint16_t*)lut, y, T, (int)D, (int)N, workspace,
                                                        as_stream(stream)));
}

int mole_lookup_combine_grouped_mapped(const int64_t* ids, const void* h, const void* w_r, const void* lut_host,
                                       float* y, int64_t T, int64_t V, int64_t D, int64_t N, int dtype,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_grouped(ids, h, w_r, lut_host, y, T, V, D, N, dtype);
  if (rc != MOLE_OK || T == 0) return rc;
  if (!workspace) return MOLE_ERR_NULL;
  if (!aligned16(workspace)) return MOLE_ERR_ALIGN;
  if (workspace_bytes < mole::grouped_workspace_bytes(T)) return MOLE_ERR_WORKSPACE;
  const char* lut_d = mapped_host_range(lut_host, (size_t)(V * N * D) * 2);
  if (!lut_d) return MOLE_ERR_MEMORY;
  return hip_status(mole::launch_lookup_combine_grouped(ids, (const uint16_t*)h, (const uint16_t*)w_r,
                                                        reinterpret_cast<const uint16_t*>(lut_d), y, T, (int)D,
                                                        (int)N, workspace, as_stream(stream)));
}

namespace {
// The NF3 combine over the batch grouped by id (codes and scales at device
// addresses: device memory, or a page-locked host table's mapping).
int nf3_grouped(const int64_t* ids, const void* h, const void* w_r, const uint8_t* codes, const uint16_t* scales,
                float* y, int64_t T, int64_t D, int64_t N, void* workspace, hipStream_t s) {
  const int* pos_tok;
  const int* pos_row;
  const float* gates;
  hipError_t err = mole::launch_group_route(ids, (const uint16_t*)h, (const uint16_t*)w_r, T, (int)D, (int)N,
                                            workspace, s, &pos_tok, &pos_row, &gates);
  if (err != hipSuccess) return hip_status(err);
  return hip_status(mole::launch_lookup_combine_nf3_grouped(pos_tok, pos_row, gates, codes, scales, y, T, D, N, s));
}

int check_nf3_grouped(const int64_t* ids, const void* h, const void* w_r, const void* codes, const void* scales,
                      float* y, int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h, void* workspace,
                      size_t workspace_bytes) {
  if (!dtype_ok(dtype_h)) return MOLE_ERR_DTYPE;
  int rc = check_combine_common(T, V, D, N);
  if (rc != MOLE_OK) return rc;
  if (D % 64 != 0) return MOLE_ERR_DIM;
  if (dtype_h != MOLE_BF16 || N > 16 || V > INT32_MAX) return MOLE_ERR_UNSUPPORTED;
  if (T == 0) return MOLE_OK;
  if (!ids || !h || !w_r || !codes || !scales || !y || !workspace) return MOLE_ERR_NULL;
  if (!aligned8(ids) || !aligned16(h) || !aligned16(w_r) || !aligned16(codes) || !aligned16(scales) ||
      !aligned16(y) || !aligned16(workspace))
    return MOLE_ERR_ALIGN;
  if (workspace_bytes < mole::grouped_workspace_bytes(T)) return MOLE_ERR_WORKSPACE;
  return MOLE_OK;
}
}  // namespace

int mole_lookup_combine_nf3_grouped(const int64_t* ids, const void* h, const void* w_r, const uint8_t* codes,
                                    const uint16_t* scales, float* y, int64_t T, int64_t V, int64_t D, int64_t N,
                                    int dtype_h, void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = check_nf3_grouped(ids, h, w_r, codes, scales, y, T, V, D, N, dtype_h, workspace, workspace_bytes);
  if (rc != MOLE_OK || T == 0) return rc;
  return nf3_grouped(ids, h, w_r, codes, scales, y, T, D, N, workspace, as_stream(stream));
}

int mole_lookup_combine_nf3_grouped_mapped(const int64_t* ids, const void* h, const void* w_r,
                                           const uint8_t* codes_host, const uint16_t* scales_host, float* y,
                                           int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  const int rc =
      check_nf3_grouped(ids, h, w_r, codes_host, scales_host, y, T, V, D, N, dtype_h, workspace, workspace_bytes);
  if (rc != MOLE_OK || T == 0) return rc;
  const char* codes_d = mapped_host_range(codes_host, (size_t)(V * N * (3 * D / 8)));
  const char* scales_d = mapped_host_range(scales_host, (size_t)(V * N * (D / 64)) * 2);
  if (!codes_d || !scales_d) return MOLE_ERR_MEMORY;
  return nf3_grouped(ids, h, w_r, reinterpret_cast<const uint8_t*>(codes_d),
                     reinterpret_cast<const uint16_t*>(scales_d), y, T, D, N, workspace, as_stream(stream));
}

int mole_lookup_combine_grouped_noalloc(const int64_t* ids, const void* h, const void* w_r, const void* lut,
                                        float* y, int64_t T, int64_t V, int64_t D, int64_t N, int dtype,
                                        void* stream) {
  int rc = check_grouped(ids, h, w_r, lut, y, T, V, D, N, dtype);
  if (rc != MOLE_OK || T == 0) return rc;
  if (T > MOLE_GROUPED_NOALLOC_MAX_T) return MOLE_ERR_UNSUPPORTED;
  return hip_status(mole::launch_lookup_combine_grouped_noalloc(ids, (const uint16_t*)h, (const uint16_t*)w_r,
                                                                (const uint16_t*)lut, y, T, (int)D, (int)N,
                                                                as_stream(stream)));
}

static_assert(MOLE_GROUPED_NOALLOC_MAX_T == mole::kGroupedNoAllocMaxT, "header and library agree on the limit");

int mole_train_workspace_size(int64_t T, int64_t U, int64_t D, int64_t F, int64_t N, size_t* fwd_bytes,
                              size_t* bwd_bytes) {
  if (T < 0 || U < 0 || U > T || D <= 0 || F <= 0 || N <= 0 || N * F > kMaxTrainDim || N * D > kMaxTrainDim ||
      T > kMaxTrainDim)
    return MOLE_ERR_DIM;
  const mole::TrainPlan p = mole::train_plan(T, U, D, F, N);
  if (fwd_bytes) *fwd_bytes = T == 0 ? 0 : p.fwd_total;
  if (bwd_bytes) *bwd_bytes = T == 0 ? 0 : p.bwd_total;
  return MOLE_OK;
}

int mole_train_forward(const int64_t* uniq, const int64_t* remap, const void* emb, const void* w_up,
                       const void* w_down, const void* h, const void* w_r, float* y, int64_t T, int64_t U,
                       int64_t V, int64_t D, int64_t F, int64_t N, int dtype, void* fwd_ws, size_t fwd_bytes,
                       void* stream) {
  int rc = check_train(T, U, V, D, F, N, dtype);
  if (rc != MOLE_OK) return rc;
  if (T == 0) return MOLE_OK;
  if (!uniq || !remap || !emb || !w_up || !w_down || !h || !w_r || !y || !fwd_ws) return MOLE_ERR_NULL;
  if (!aligned8(uniq) || !aligned8(remap) || !aligned16(emb) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(h) || !aligned16(w_r) || !aligned16(y) || !aligned16(fwd_ws))
    return MOLE_ERR_ALIGN;
  if (fwd_bytes < mole::train_plan(T, U, D, F, N).fwd_total) return MOLE_ERR_WORKSPACE;
  return hip_status(mole::launch_train_forward(uniq, remap, (const uint16_t*)emb, (const uint16_t*)w_up,
                                               (const uint16_t*)w_down, (const uint16_t*)h, (const uint16_t*)w_r, y,
                                               fwd_ws, T, U, D, F, N, as_stream(stream)));
}

int mole_train_backward(const int64_t* remap, const int64_t* row_ptr, const int64_t* tok, const void* w_up,
                        const void* w_down, const void* h, const void* w_r, const float* dy, const void* fwd_ws,
                        size_t fwd_bytes, void* bwd_ws, size_t bwd_bytes, float* d_w_up, float* d_w_down,
                        float* d_w_r, float* d_h, float* d_x, int64_t T, int64_t U, int64_t V, int64_t D, int64_t F,
                        int64_t N, int dtype, void* stream) {
  int rc = check_train(T, U, V, D, F, N, dtype);
  if (rc != MOLE_OK) return rc;
  if (T == 0) return MOLE_OK;
  if (!remap || !row_ptr || !tok || !w_up || !w_down || !h || !w_r || !dy || !fwd_ws || !bwd_ws || !d_w_up ||
      !d_w_down || !d_w_r || !d_h || !d_x)
    return MOLE_ERR_NULL;
  if (!aligned8(remap) || !aligned8(row_ptr) || !aligned8(tok) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(h) || !aligned16(w_r) || !aligned16(dy) || !aligned16(fwd_ws) || !aligned16(bwd_ws) ||
      !aligned16(d_w_up) || !aligned16(d_w_down) || !aligned16(d_w_r) || !aligned16(d_h) || !aligned16(d_x))
    return MOLE_ERR_ALIGN;
  const mole::TrainPlan p = mole::train_plan(T, U, D, F, N);
  if (fwd_bytes < p.fwd_total || bwd_bytes < p.bwd_total) return MOLE_ERR_WORKSPACE;
  return hip_status(mole::launch_train_backward(nullptr, remap, row_ptr, tok, nullptr, (const uint16_t*)w_up,
                                                (const uint16_t*)w_down, (const uint16_t*)h, (const uint16_t*)w_r,
                                                dy, fwd_ws, bwd_ws, d_w_up, d_w_down, d_w_r, d_h, d_x, T, U, D, F, N,
                                                as_stream(stream)));
}

int mole_layer_workspace_size(int64_t T, int64_t D, int64_t F, size_t* bytes) {
  if (!bytes) return MOLE_ERR_NULL;
  if (T < 0 || D <= 0 || F <= 0 || T > kMaxDim || D > kMaxDim || F > kMaxDim) return MOLE_ERR_DIM;
  *bytes = T == 0 ? 0 : mole::layer_plan(T, D, F).total;
  return MOLE_OK;
}

int mole_layer_forward(const int64_t* ids, const void* h, const void* w_r, const void* lut, const void* w_s_up,
                       const void* w_s_down, float* x, int64_t T, int64_t V, int64_t D, int64_t N, int64_t F,
                       int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return MOLE_ERR_DTYPE;
  int rc = check_combine_common(T, V, D, N);
  if (rc != MOLE_OK) return rc;
  if (F <= 0 || F > kMaxDim) return MOLE_ERR_DIM;
  if (dtype != MOLE_BF16) return MOLE_ERR_UNSUPPORTED;
  if (D % 8 != 0 || F % 8 != 0) return MOLE_ERR_DIM;
  // The projections address 256-row operand panels with 32-bit byte offsets.
  if (D > kMaxPanelStride || F > kMaxPanelStride) return MOLE_ERR_UNSUPPORTED;
  if (T == 0) return MOLE_OK;
  if (!ids || !h || !w_r || !lut || !w_s_up || !w_s_down || !x || !workspace) return MOLE_ERR_NULL;
  if (!aligned8(ids) || !aligned16(h) || !aligned16(w_r) || !aligned16(lut) || !aligned16(w_s_up) ||
      !aligned16(w_s_down) || !aligned16(x) || !aligned16(workspace))
    return MOLE_ERR_ALIGN;
  if (workspace_bytes < mole::layer_plan(T, D, F).total) return MOLE_ERR_WORKSPACE;
  return hip_status(mole::launch_layer_forward(ids, (const uint16_t*)h, (const uint16_t*)w_r, (const uint16_t*)lut,
                                               (const uint16_t*)w_s_up, (const uint16_t*)w_s_down, x, T, D, N, F,
                                               workspace, as_stream(stream)));
}

static int mole_gather_nf3_host_impl(const int64_t* ids_host, int64_t T, const uint8_t* codes_host,
                                     const uint16_t* scales_host, int64_t V, int64_t N, int64_t D,
                                     uint8_t* codes_stage_host, uint16_t* scales_stage_host, int64_t* remap_host,
                                     int64_t* n_unique, int nthreads) {
  if (T < 0 || V <= 0 || N <= 0 || D <= 0 || D % 64 != 0) return MOLE_ERR_DIM;
  if (T > 0 && (!ids_host || !codes_host || !scales_host || !codes_stage_host || !scales_stage_host ||
                !remap_host))
    return MOLE_ERR_NULL;
  if (!n_unique) return MOLE_ERR_NULL;
  std::vector<int64_t> uniq;
  int rc = dedupe(ids_host, T, V, uniq, remap_host);
  if (rc != MOLE_OK) return rc;
  gather_rows(uniq, codes_host, scales_host, N, D, codes_stage_host, scales_stage_host, nthreads);
  *n_unique = (int64_t)uniq.size();
  return MOLE_OK;
}

int mole_gather_nf3_host(const int64_t* ids_host, int64_t T, const uint8_t* codes_host,
                         const uint16_t* scales_host, int64_t V, int64_t N, int64_t D,
                         uint8_t* codes_stage_host, uint16_t* scales_stage_host, int64_t* remap_host,
                         int64_t* n_unique, int nthreads) {
  return guarded([&] {
    return mole_gather_nf3_host_impl(ids_host, T, codes_host, scales_host, V, N, D, codes_stage_host,
        scales_stage_host, remap_host, n_unique, nthreads);
  });
}

int mole_nf3_host_staging_size(int64_t T, int64_t N, int64_t D, size_t* bytes) {
  if (!bytes) return MOLE_ERR_NULL;
  if (T < 0 || N <= 0 || D <= 0 || D % 64 != 0 || D > kMaxDim || T > kMaxDim || N > kMaxExperts)
    return MOLE_ERR_DIM;
  const Nf3Staging st = nf3_staging(T, T, N, D);
  *bytes = st.total;
  return MOLE_OK;
}

extern "C++" {  // (a template inside the C-linkage block)
namespace {
// The host-resident NF3 combine with a row source: gather(uniq, codes_out,
// scales_out) copies the distinct rows into the pinned staging area and
// returns a status; source_ok says whether the source's own pointers or
// handle are present (checked with the other arguments).
template <typename Gather>
int combine_nf3_staged(const int64_t* ids_host, const void* h, const void* w_r, void* stage_host, void* stage_dev,
                       size_t stage_bytes, float* y, int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h,
                       int64_t* n_unique, void* stream, bool source_ok, Gather gather) {
  if (!dtype_ok(dtype_h)) return MOLE_ERR_DTYPE;
  int rc = check_combine_common(T, V, D, N);
  if (rc != MOLE_OK) return rc;
  if (D % 64 != 0) return MOLE_ERR_DIM;
  if (T == 0) {
    if (n_unique) *n_unique = 0;
    return MOLE_OK;
  }
  if (!ids_host || !h || !w_r || !source_ok || !stage_host || !stage_dev || !y) return MOLE_ERR_NULL;
  if (!aligned16(h) || !aligned16(w_r) || !aligned16(stage_host) || !aligned16(stage_dev) || !aligned16(y))
    return MOLE_ERR_ALIGN;
  if (stage_bytes < nf3_staging(T, T, N, D).total) return MOLE_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  hipEvent_t ev;
  rc = stage_event(stage_host, &ev);
  if (rc == MOLE_OK) rc = hip_status(hipEventSynchronize(ev));  // the last copy out of stage_host
  if (rc != MOLE_OK) return rc;
  // The remap section comes first (its size depends on T only); the codes
  // and scales sections follow at offsets that depend on U, so the used part
  // of the staging area is one contiguous range and moves in one copy.
  std::vector<int64_t> uniq;
  uint8_t* base_h = static_cast<uint8_t*>(stage_host);
  int64_t* remap_h = reinterpret_cast<int64_t*>(base_h);
  rc = dedupe(ids_host, T, V, uniq, remap_h);
  if (rc != MOLE_OK) return rc;
  const int64_t U = (int64_t)uniq.size();
  const Nf3Staging st = nf3_staging(T, U, N, D);
  rc = gather(uniq, base_h + st.codes_off, reinterpret_cast<uint16_t*>(base_h + st.scales_off));
  if (rc != MOLE_OK) return rc;
  uint8_t* base_d = static_cast<uint8_t*>(stage_dev);
  rc = hip_status(hipMemcpyAsync(base_d, base_h, st.total, hipMemcpyHostToDevice, s));
  if (rc == MOLE_OK) rc = hip_status(hipEventRecord(ev, s));
  if (rc == MOLE_OK)
    rc = hip_status(mole::launch_lookup_combine_nf3(reinterpret_cast<const int64_t*>(base_d), h, w_r,
                                                    base_d + st.codes_off,
                                                    reinterpret_cast<const uint16_t*>(base_d + st.scales_off), y,
                                                    T, D, N, dtype_h, s));
  if (rc == MOLE_OK && n_unique) *n_unique = U;
  return rc;
}
}  // namespace
}  // extern "C++"

static int mole_lookup_combine_nf3_host_impl(const int64_t* ids_host, const void* h, const void* w_r,
                                             const uint8_t* codes_host, const uint16_t* scales_host,
                                             void* stage_host, void* stage_dev, size_t stage_bytes, float* y,
                                             int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h,
                                             int nthreads, int64_t* n_unique, void* stream) {
  return combine_nf3_staged(ids_host, h, w_r, stage_host, stage_dev, stage_bytes, y, T, V, D, N, dtype_h, n_unique,
                            stream, codes_host && scales_host,
                            [&](const std::vector<int64_t>& uniq, uint8_t* codes_out, uint16_t* scales_out) {
                              gather_rows(uniq, codes_host, scales_host, N, D, codes_out, scales_out, nthreads);
                              return (int)MOLE_OK;
                            });
}

int mole_lookup_combine_nf3_host(const int64_t* ids_host, const void* h, const void* w_r,
                                 const uint8_t* codes_host, const uint16_t* scales_host,
                                 void* stage_host, void* stage_dev, size_t stage_bytes, float* y,
                                 int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h,
                                 int nthreads, int64_t* n_unique, void* stream) {
  return guarded([&] {
    return mole_lookup_combine_nf3_host_impl(ids_host, h, w_r, codes_host, scales_host, stage_host, stage_dev,
        stage_bytes, y, T, V, D, N, dtype_h, nthreads, n_unique, stream);
  });
}

// ---------------------------------------------------------------------------
// Disk tier: the NF3 table in a file, one record per vocabulary row
// ---------------------------------------------------------------------------
namespace {
constexpr char kNf3FileMagic[8] = {'M', 'O', 'L', 'E', 'N', 'F', '3', '\0'};
constexpr uint32_t kNf3FileVersion = 1;

// 64-byte header, little-endian; records follow at data_offset.
struct Nf3FileHeader {
  char magic[8];
  uint32_t version;
  uint32_t header_bytes;
  int64_t V, N, D;
  int64_t record_bytes;  // N*3D/8 code bytes, then N*(D/64) fp16 scales
  int64_t data_offset;
  int64_t reserved;
};
static_assert(sizeof(Nf3FileHeader) == 64, "the file header is 64 bytes");

int64_t nf3_record_bytes(int64_t N, int64_t D) { return N * 3 * D / 8 + N * (D / 64) * 2; }

// pread / pwrite of exactly n bytes (retrying short transfers and EINTR).
bool read_full(int fd, void* buf, size_t n, int64_t off) {
  char* p = static_cast<char*>(buf);
  while (n > 0) {
    const ssize_t r = pread(fd, p, n, (off_t)off);
    if (r < 0 && errno == EINTR) continue;
    if (r <= 0) return false;
    p += r;
    n -= (size_t)r;
    off += r;
  }
  return true;
}

bool write_full(int fd, const void* buf, size_t n, int64_t off) {
  const char* p = static_cast<const char*>(buf);
  while (n > 0) {
    const ssize_t r = pwrite(fd, p, n, (off_t)off);
    if (r < 0 && errno == EINTR) continue;
    if (r <= 0) return false;
    p += r;
    n -= (size_t)r;
    off += r;
  }
  return true;
}

int read_nf3_header(int fd, Nf3FileHeader* hd) {
  if (fd < 0) return MOLE_ERR_IO;
  if (!read_full(fd, hd, sizeof(*hd), 0)) return MOLE_ERR_IO;
  if (std::memcmp(hd->magic, kNf3FileMagic, 8) != 0 || hd->version != kNf3FileVersion ||
      hd->header_bytes != sizeof(Nf3FileHeader))
    return MOLE_ERR_FORMAT;
  if (hd->V <= 0 || hd->N <= 0 || hd->D <= 0 || hd->D % 64 != 0 || hd->N > kMaxExperts || hd->D > kMaxDim ||
      hd->record_bytes != nf3_record_bytes(hd->N, hd->D) || hd->data_offset < (int64_t)sizeof(Nf3FileHeader))
    return MOLE_ERR_FORMAT;
  return MOLE_OK;
}

// Rows uniq[u] of the file into codes_out [U][N][3D/8] and scales_out
// [U][N][D/64]: one preadv per row (two segments, straight into the two
// staging sections), split over threads for larger batches.
int gather_rows_file(int fd, const Nf3FileHeader& hd, const std::vector<int64_t>& uniq, uint8_t* codes_out,
                     uint16_t* scales_out, int nthreads) {
  const size_t crow = (size_t)(hd.N * 3 * hd.D / 8), srow = (size_t)(hd.N * (hd.D / 64)) * 2;
  const int64_t U = (int64_t)uniq.size();
  std::atomic<int> failed{0};
  auto work = [&](int64_t lo, int64_t hi) {
    for (int64_t u = lo; u < hi && !failed.load(std::memory_order_relaxed); ++u) {
      const int64_t off = hd.data_offset + uniq[u] * hd.record_bytes;
      uint8_t* cp = codes_out + (size_t)u * crow;
      uint8_t* sp = reinterpret_cast<uint8_t*>(scales_out) + (size_t)u * srow;
      struct iovec iov[2] = {{cp, crow}, {sp, srow}};
      ssize_t r;
      do r = preadv(fd, iov, 2, (off_t)off); while (r < 0 && errno == EINTR);
      if (r == (ssize_t)(crow + srow)) continue;
      // a short read: finish the record with plain reads
      const size_t got = r > 0 ? (size_t)r : 0;
      bool ok = r >= 0;
      if (ok && got < crow) ok = read_full(fd, cp + got, crow - got, off + (int64_t)got);
      const size_t sgot = got > crow ? got - crow : 0;
      if (ok) ok = read_full(fd, sp + sgot, srow - sgot, off + (int64_t)(crow + sgot));
      if (!ok) failed.store(1);
    }
  };
  // Reads mostly wait on the device: more workers than cores keep more of
  // them in flight (32 by default, at least 4 rows each).
  int nt = nthreads > 0 ? std::min(nthreads, WorkerPool::kMaxWorkers) : 32;
  nt = (int)std::min<int64_t>(nt, std::max<int64_t>(1, U / 4));
  parallel_ranges(U, nt, work);
  return failed.load() ? MOLE_ERR_IO : MOLE_OK;
}

int check_nf3_file(int fd, int64_t V, int64_t N, int64_t D, Nf3FileHeader* hd) {
  const int rc = read_nf3_header(fd, hd);
  if (rc != MOLE_OK) return rc;
  if (hd->V != V || hd->N != N || hd->D != D) return MOLE_ERR_DIM;
  return MOLE_OK;
}
}  // namespace

static int mole_nf3_file_write_impl(const char* path, const uint8_t* codes_host, const uint16_t* scales_host, int64_t V,
                                    int64_t N, int64_t D) {
  if (!path || !codes_host || !scales_host) return MOLE_ERR_NULL;
  if (V <= 0 || N <= 0 || D <= 0 || D % 64 != 0 || D > kMaxDim) return MOLE_ERR_DIM;
  if (N > kMaxExperts) return MOLE_ERR_UNSUPPORTED;
  Nf3FileHeader hd;
  std::memset(&hd, 0, sizeof(hd));
  std::memcpy(hd.magic, kNf3FileMagic, 8);
  hd.version = kNf3FileVersion;
  hd.header_bytes = sizeof(Nf3FileHeader);
  hd.V = V;
  hd.N = N;
  hd.D = D;
  hd.record_bytes = nf3_record_bytes(N, D);
  hd.data_offset = sizeof(Nf3FileHeader);
  const int fd = open(path, O_CREAT | O_TRUNC | O_WRONLY, 0644);
  if (fd < 0) return MOLE_ERR_IO;
  bool ok = write_full(fd, &hd, sizeof(hd), 0);
  // records assembled in blocks of rows (about 4 MB per write)
  const size_t crow = (size_t)(N * 3 * D / 8), srow = (size_t)(N * (D / 64)) * 2;
  const int64_t rows_per = std::max<int64_t>(1, ((int64_t)4 << 20) / hd.record_bytes);
  std::vector<uint8_t> buf((size_t)(rows_per * hd.record_bytes));
  for (int64_t v0 = 0; ok && v0 < V; v0 += rows_per) {
    const int64_t nr = std::min(rows_per, V - v0);
    for (int64_t i = 0; i < nr; ++i) {
      uint8_t* rec = buf.data() + (size_t)(i * hd.record_bytes);
      std::memcpy(rec, codes_host + (size_t)(v0 + i) * crow, crow);
      std::memcpy(rec + crow, reinterpret_cast<const uint8_t*>(scales_host) + (size_t)(v0 + i) * srow, srow);
    }
    ok = write_full(fd, buf.data(), (size_t)(nr * hd.record_bytes), hd.data_offset + v0 * hd.record_bytes);
  }
  if (close(fd) != 0) ok = false;
  return ok ? MOLE_OK : MOLE_ERR_IO;
}

int mole_nf3_file_write(const char* path, const uint8_t* codes_host, const uint16_t* scales_host, int64_t V,
                        int64_t N, int64_t D) {
  return guarded([&] { return mole_nf3_file_write_impl(path, codes_host, scales_host, V, N, D); });
}

static int mole_nf3_file_shape_impl(int fd, int64_t* V, int64_t* N, int64_t* D) {
  if (!V || !N || !D) return MOLE_ERR_NULL;
  Nf3FileHeader hd;
  const int rc = read_nf3_header(fd, &hd);
  if (rc != MOLE_OK) return rc;
  *V = hd.V;
  *N = hd.N;
  *D = hd.D;
  return MOLE_OK;
}

int mole_nf3_file_shape(int fd, int64_t* V, int64_t* N, int64_t* D) {
  return guarded([&] { return mole_nf3_file_shape_impl(fd, V, N, D); });
}

static int mole_gather_nf3_file_impl(int fd, const int64_t* ids_host, int64_t T, int64_t V, int64_t N, int64_t D,
                                     uint8_t* codes_stage_host, uint16_t* scales_stage_host, int64_t* remap_host,
                                     int64_t* n_unique, int nthreads) {
  if (T < 0 || V <= 0 || N <= 0 || D <= 0 || D % 64 != 0) return MOLE_ERR_DIM;
  if (T > 0 && (!ids_host || !codes_stage_host || !scales_stage_host || !remap_host)) return MOLE_ERR_NULL;
  if (!n_unique) return MOLE_ERR_NULL;
  Nf3FileHeader hd;
  int rc = check_nf3_file(fd, V, N, D, &hd);
  if (rc != MOLE_OK) return rc;
  std::vector<int64_t> uniq;
  rc = dedupe(ids_host, T, V, uniq, remap_host);
  if (rc != MOLE_OK) return rc;
  rc = gather_rows_file(fd, hd, uniq, codes_stage_host, scales_stage_host, nthreads);
  if (rc != MOLE_OK) return rc;
  *n_unique = (int64_t)uniq.size();
  return MOLE_OK;
}

int mole_gather_nf3_file(int fd, const int64_t* ids_host, int64_t T, int64_t V, int64_t N, int64_t D,
                         uint8_t* codes_stage_host, uint16_t* scales_stage_host, int64_t* remap_host,
                         int64_t* n_unique, int nthreads) {
  return guarded([&] {
    return mole_gather_nf3_file_impl(fd, ids_host, T, V, N, D, codes_stage_host, scales_stage_host, remap_host,
        n_unique, nthreads);
  });
}

static int mole_lookup_combine_nf3_file_impl(int fd, const int64_t* ids_host, const void* h, const void* w_r,
                                             void* stage_host, void* stage_dev, size_t stage_bytes, float* y,
                                             int64_t T, int64_t V, int64_t D, int64_t N, int dtype_h, int nthreads,
                                             int64_t* n_unique, void* stream) {
  Nf3FileHeader hd;
  int hdr = MOLE_OK;
  if (T > 0) hdr = check_nf3_file(fd, V, N, D, &hd);
  return combine_nf3_staged(ids_host, h, w_r, stage_host, stage_dev, stage_bytes, y, T, V, D, N, dtype_h, n_unique,
                            stream, true,
                            [&](const std::vector<int64_t>& uniq, uint8_t* codes_out, uint16_t* scales_out) {
                              if (hdr != MOLE_OK) return hdr;
                              return gather_rows_file(fd, hd, uniq, codes_out, scales_out, nthreads);
                            });
}

int mole_lookup_combine_nf3_file(int fd, const int64_t* ids_host, const void* h, const void* w_r,
                                 void* stage_host, void* stage_dev, size_t stage_bytes, float* y, int64_t T,
                                 int64_t V, int64_t D, int64_t N, int dtype_h, int nthreads, int64_t* n_unique,
                                 void* stream) {
  return guarded([&] {
    return mole_lookup_combine_nf3_file_impl(fd, ids_host, h, w_r, stage_host, stage_dev, stage_bytes, y, T, V, D, N,
        dtype_h, nthreads, n_unique, stream);
  });
}

int mole_nf3_host_stack_staging_size(int64_t T, int64_t L, int64_t N, int64_t D, size_t* bytes) {
  if (!bytes) return MOLE_ERR_NULL;
  if (T < 0 || L <= 0 || N <= 0 || D <= 0 || D % 64 != 0 || D > kMaxDim || T > kMaxDim || N > kMaxExperts ||
      L > kMaxDim)
    return MOLE_ERR_DIM;
  *bytes = nf3_stack_staging(T, T, L, N, D, nullptr, nullptr);
  return MOLE_OK;
}

static int mole_prefetch_nf3_host_stack_impl(const int64_t* ids_host, int64_t T,
                                             const uint8_t* const* codes_host, const uint16_t* const* scales_host,
                                             int64_t L, int64_t V, int64_t N, int64_t D, void* stage_host,
                                             void* stage_dev, size_t stage_bytes, size_t* codes_off,
                                             size_t* scales_off, int nthreads, int64_t* n_unique, void* stream) {
  if (T < 0 || L <= 0 || V <= 0 || N <= 0 || D <= 0 || D % 64 != 0 || D > kMaxDim || T > kMaxDim ||
      N > kMaxExperts || L > kMaxDim)
    return MOLE_ERR_DIM;
  if (!codes_host || !scales_host || !stage_host || !stage_dev || !codes_off || !scales_off) return MOLE_ERR_NULL;
  for (int64_t l = 0; l < L; ++l)
    if (!codes_host[l] || !scales_host[l]) return MOLE_ERR_NULL;
  if (T > 0 && !ids_host) return MOLE_ERR_NULL;
  if (!aligned16(stage_host) || !aligned16(stage_dev)) return MOLE_ERR_ALIGN;
  if (stage_bytes < nf3_stack_staging(T, T, L, N, D, nullptr, nullptr)) return MOLE_ERR_WORKSPACE;
  if (T == 0) {
    nf3_stack_staging(0, 0, L, N, D, codes_off, scales_off);
    if (n_unique) *n_unique = 0;
    return MOLE_OK;
  }
  hipStream_t s = as_stream(stream);
  hipEvent_t ev;
  int rc = stage_event(stage_host, &ev);
  if (rc == MOLE_OK) rc = hip_status(hipEventSynchronize(ev));  // the last copy out of stage_host
  if (rc != MOLE_OK) return rc;
  std::vector<int64_t> uniq;
  uint8_t* base_h = static_cast<uint8_t*>(stage_host);
  rc = dedupe(ids_host, T, V, uniq, reinterpret_cast<int64_t*>(base_h));
  if (rc != MOLE_OK) return rc;
  const int64_t U = (int64_t)uniq.size();
  const size_t total = nf3_stack_staging(T, U, L, N, D, codes_off, scales_off);
  rc = gather_copy_stack(uniq, codes_host, scales_host, L, N, D, base_h, static_cast<uint8_t*>(stage_dev),
                         codes_off, scales_off, total, nthreads, s);
  if (rc == MOLE_OK) rc = hip_status(hipEventRecord(ev, s));
  if (rc == MOLE_OK && n_unique) *n_unique = U;
  return rc;
}

int mole_prefetch_nf3_host_stack(const int64_t* ids_host, int64_t T,
                                 const uint8_t* const* codes_host, const uint16_t* const* scales_host,
                                 int64_t L, int64_t V, int64_t N, int64_t D, void* stage_host,
                                 void* stage_dev, size_t stage_bytes, size_t* codes_off,
                                 size_t* scales_off, int nthreads, int64_t* n_unique, void* stream) {
  return guarded([&] {
    return mole_prefetch_nf3_host_stack_impl(ids_host, T, codes_host, scales_host, L, V, N, D, stage_host, stage_dev,
        stage_bytes, codes_off, scales_off, nthreads, n_unique, stream);
  });
}

}  // extern "C"
