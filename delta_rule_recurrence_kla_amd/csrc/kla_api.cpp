// libkla host side: the C ABI declared in include/kla.h.
//
// Every entry point validates its arguments before any HIP call, plans the
// launch, takes a stream-ordered workspace when it needs one, enqueues the
// kernels on the caller's stream and returns. No exception crosses the ABI.
#include "kla.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kla_launch.h"

namespace {

constexpr int kChunk = 64;
constexpr int kMaxGridYZ = 65535;

thread_local std::string g_err;

kla_status fail(kla_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

// ---------------------------------------------------------------------------
// timing hook
struct TimedLaunch {
  const char* name;
  hipEvent_t start, stop;
};
struct TimingState {
  bool enabled = false;
  char only[32] = {0};  // when set, only launches of this kernel are stamped
  std::vector<TimedLaunch> rec;
};
thread_local TimingState g_timing;

thread_local kla::LaunchEvents g_launch_events;
}  // namespace

kla::LaunchEvents& kla::launch_events() { return g_launch_events; }

namespace {

// With timing on, the kernels a launcher enqueues stamp a pair of events from their own
// dispatches (kla::launch_kernel): the interval runs from the first kernel's start to the
// last one's end, with no host-side gap in it.
template <class F>
hipError_t timed(const char* name, hipStream_t stream, F&& launch) {
  (void)stream;
  if (!g_timing.enabled || (g_timing.only[0] && std::strcmp(g_timing.only, name) != 0)) return launch();
  TimedLaunch t{name, nullptr, nullptr};
  // no system-scope fences around the stamps: they would add a cache flush to every launch
  hipError_t e = hipEventCreateWithFlags(&t.start, hipEventDisableSystemFence);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&t.stop, hipEventDisableSystemFence);
  if (e == hipSuccess) {
    g_launch_events = {t.start, t.stop};
    e = launch();
    g_launch_events = {};
  }
  if (e == hipSuccess) {
    g_timing.rec.push_back(t);
  } else {  // the stamps of a launch that did not happen are never read: release them now
    if (t.start) (void)hipEventDestroy(t.start);
    if (t.stop) (void)hipEventDestroy(t.stop);
  }
  return e;
}

// ---------------------------------------------------------------------------
// workspace: the library's own stream-ordered pool, one per device
//
// Prefill and backward workspaces come from a memory pool the library creates on a
// device's first call. Its release threshold is raised so that freed blocks stay
// reserved for the next call instead of going back to the driver at each
// synchronisation. The device's default pool, which other code in the process may
// use, is never touched. kla_workspace_trim() hands the reserved blocks back.
constexpr int kMaxDevices = 64;
std::once_flag g_pool_once[kMaxDevices];
hipMemPool_t g_pool[kMaxDevices] = {};
hipError_t g_pool_err[kMaxDevices] = {};

hipError_t library_pool(hipMemPool_t* pool) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_pool_once[dev], [dev] {
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t p = nullptr;
    hipError_t err = hipMemPoolCreate(&p, &props);
    if (err == hipSuccess) {
      uint64_t thr = UINT64_MAX;
      err = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &thr);
      if (err != hipSuccess) (void)hipMemPoolDestroy(p);
    }
    if (err == hipSuccess) g_pool[dev] = p;
    g_pool_err[dev] = err;
  });
  if (!g_pool[dev]) return g_pool_err[dev] != hipSuccess ? g_pool_err[dev] : hipErrorNotInitialized;
  *pool = g_pool[dev];
  return hipSuccess;
}

// Stream-ordered workspace of `bytes` from the library pool; KLA_ERR_OOM (with the
// message set) if it cannot be had. Nothing has been enqueued on failure.
kla_status workspace_alloc(void** ws, size_t bytes, hipStream_t stream) {
  *ws = nullptr;
  if (const char* f = std::getenv("KLA_TEST_FAIL_ALLOC")) {
    if (f[0] == '1') return fail(KLA_ERR_OOM, "workspace allocation failed (forced by KLA_TEST_FAIL_ALLOC)");
  }
  hipMemPool_t pool = nullptr;
  hipError_t e = library_pool(&pool);
  if (e == hipSuccess) e = hipMallocFromPoolAsync(ws, bytes, pool, stream);
  if (e != hipSuccess || !*ws) {
    (void)hipGetLastError();
    *ws = nullptr;
    return fail(KLA_ERR_OOM, "workspace of %zu bytes from the library pool failed: %s", bytes, hipGetErrorString(e));
  }
  return KLA_OK;
}

// Every array argument must be 16-byte aligned: the kernels move rows, states and
// gates with 16-byte vector and buffer accesses.
bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

template <class... P>
kla_status check_aligned(const char* names, P... ptrs) {
  const void* list[] = {static_cast<const void*>(ptrs)...};
  for (const void* p : list)
    if (p && misaligned(p)) return fail(KLA_ERR_INVALID_ARG, "every array must be 16-byte aligned (%s)", names);
  return KLA_OK;
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// ---------------------------------------------------------------------------
// validation and planning
bool supported_dk(int dk) { return dk == 64 || dk == 128 || dk == 256; }
bool supported_dv(int dv) { return dv == 64 || dv == 128; }

kla_status check_prefill_sizes(kla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk) {
  if (dtype != KLA_DTYPE_BF16 && dtype != KLA_DTYPE_F32) return fail(KLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 1 || H < 1 || T < 0) return fail(KLA_ERR_INVALID_ARG, "sizes must satisfy B >= 1, H >= 1, T >= 0 (got B=%d T=%d H=%d)", B, T, H);
  if (dk < 1 || dv < 1 || chunk < 1) return fail(KLA_ERR_INVALID_ARG, "dk, dv and chunk must be positive");
  if (!supported_dk(dk)) return fail(KLA_ERR_UNSUPPORTED, "dk=%d not supported (64, 128, 256)", dk);
  if (!supported_dv(dv)) return fail(KLA_ERR_UNSUPPORTED, "dv=%d not supported (64, 128)", dv);
  if (chunk != kChunk) return fail(KLA_ERR_UNSUPPORTED, "chunk=%d not supported (64)", chunk);
  if (dtype == KLA_DTYPE_F32 && dk > 128) return fail(KLA_ERR_UNSUPPORTED, "fp32 prefill supports dk <= 128 (got %d)", dk);
  if (static_cast<long long>(B) * H > kMaxGridYZ) return fail(KLA_ERR_UNSUPPORTED, "B*H=%lld exceeds %d", static_cast<long long>(B) * H, kMaxGridYZ);
  // kernels address one chunk (64 tokens of every head) with 32-bit buffer offsets below 2^30
  if (64LL * H * std::max(dk, dv) * 4 >= (1LL << 30)) return fail(KLA_ERR_UNSUPPORTED, "H=%d too large for dk=%d, dv=%d", H, dk, dv);
  return KLA_OK;
}

struct Plan {
  kla_path path;
  int segs;        // scan segments (1 for sequential)
  int seg_chunks;  // chunks per segment
  size_t rec_off, rec_bytes, maps_off, maps_bytes, starts_off, starts_bytes;
  size_t lift_off, lift_bytes;  // PSD lift: the lifted query rows, then the key rows (0 bytes without the lift)
  size_t total;
};

Plan make_plan(kla_dtype dtype, int B, int T, int H, int dk, int dv, kla_path path, int segments, int cus) {
  Plan p{};
  const int nc = (T + kChunk - 1) / kChunk;
  const long long bh = static_cast<long long>(B) * H;
  const long long seq_wgs = bh * (dv / 64);
  kla_path chosen = path;
  int segs = 1;
  if (nc >= 2 && path != KLA_PATH_SEQUENTIAL) {
    // cost in chunk steps: rounds of workgroups times chunks per walk. A walk with outputs runs one
    // workgroup per CU; the bf16 map walks run two (the copy-wave map walk in 76 KB of LDS, the
    // dk = 256 one held to the registers of two).
    auto rounds = [cus](long long wgs, int per_cu) { return (wgs + per_cu * cus - 1) / (per_cu * cus); };
    const int maps_per_cu = dtype == KLA_DTYPE_BF16 ? 2 : 1;
    const double seq_cost = static_cast<double>(rounds(seq_wgs, 1)) * nc;
    double best = 1e300;
    int best_g = 1;
    const int gmax = std::min(nc, 256);
    for (int g = 2; g <= gmax; ++g) {
      const int L = (nc + g - 1) / g;
      const int G = (nc + L - 1) / L;
      if (G < 2) continue;
      // (calls without an initial state: segment 0's identity columns are not walked)
      const long long wg1 = bh * ((G - 1) * ((dk + dv) / 64) - dk / 64);
      const long long wg3 = bh * G * (dv / 64);
      // a map walk skips the output products (about 0.6 of an output walk); each step of the
      // serial fold of the maps costs about two chunk steps (measured at dk = 128 and 256)
      const double cost = 0.6 * rounds(wg1, maps_per_cu) * L + rounds(wg3, 1) * L + 2.0 * (G - 1);
      if (cost < best) {
        best = cost;
        best_g = G;
      }
    }
    if (path == KLA_PATH_SCAN) {
      segs = segments > 0 ? std::min(segments, nc) : best_g;
      chosen = KLA_PATH_SCAN;
    } else if (best_g >= 2 && best < 0.8 * seq_cost) {
      segs = best_g;
      chosen = KLA_PATH_SCAN;
    } else {
      chosen = KLA_PATH_SEQUENTIAL;
    }
  } else {
    chosen = KLA_PATH_SEQUENTIAL;
  }
  int seg_chunks = nc;
  if (chosen == KLA_PATH_SCAN) {
    segs = std::max(segs, 1);
    seg_chunks = (nc + segs - 1) / segs;
    segs = (nc + seg_chunks - 1) / seg_chunks;  // no empty segment
    if (segs < 2) {
      chosen = KLA_PATH_SEQUENTIAL;
      segs = 1;
      seg_chunks = nc;
    }
  }
  p.path = chosen;
  p.segs = segs;
  p.seg_chunks = seg_chunks;
  p.rec_off = 0;
  const int rec_bytes = kla::record_bytes(dtype == KLA_DTYPE_BF16 ? 0 : 1, dk);  // per chunk
  p.rec_bytes = align256(static_cast<size_t>(bh) * nc * rec_bytes);
  p.maps_off = p.rec_off + p.rec_bytes;
  p.maps_bytes = chosen == KLA_PATH_SCAN ? align256(static_cast<size_t>(bh) * (segs - 1) * dk * (dk + dv) * 4) : 0;
  p.starts_off = p.maps_off + p.maps_bytes;
  p.starts_bytes = chosen == KLA_PATH_SCAN ? align256(static_cast<size_t>(bh) * segs * dk * dv * 4) : 0;
  p.lift_off = p.starts_off + p.starts_bytes;
  p.lift_bytes = 0;
  p.total = p.lift_off;
  return p;
}

// Room for the lifted query and key rows of a PSD call (dk bf16 features per row).
void plan_lift(Plan& p, int B, int T, int H, int dk) {
  p.lift_bytes = align256(static_cast<size_t>(B) * T * H * dk * 2);
  p.total = p.lift_off + 2 * p.lift_bytes;
}

kla_status hip_fail(hipError_t e, const char* what) {
  return fail(KLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Everything a prefill call checks before it touches HIP; on KLA_OK the call has work
// to enqueue (T > 0) or has already handled T == 0 (`done` set).
kla_status chunk_fwd_check(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* eta, const float* init_state, float* out,
                           float* final_state, int B, int T, int H, int dk, int dv, int chunk, kla_path path,
                           int segments) {
  kla_status st = check_prefill_sizes(dtype, B, T, H, dk, dv, chunk);
  if (st != KLA_OK) return st;
  if (beta_mode != KLA_BETA_KACZMARZ && beta_mode != KLA_BETA_DIRECT)
    return fail(KLA_ERR_INVALID_ARG, "unknown beta_mode %d", (int)beta_mode);
  if (path != KLA_PATH_AUTO && path != KLA_PATH_SEQUENTIAL && path != KLA_PATH_SCAN)
    return fail(KLA_ERR_INVALID_ARG, "unknown path %d", (int)path);
  if (segments < 0) return fail(KLA_ERR_INVALID_ARG, "segments must be >= 0");
  if (T > 0 && (!q || !k || !v || !log_alpha || !eta || !out))
    return fail(KLA_ERR_INVALID_ARG, "q, k, v, log_alpha, eta and out must be non-null when T > 0");
  return check_aligned("q, k, v, log_alpha, eta, init_state, out, final_state", q, k, v, log_alpha, eta, init_state,
                       out, final_state);
}

// T == 0: final_state receives init_state (or zeros).
kla_status chunk_fwd_empty(const float* init_state, float* final_state, size_t state_n, hipStream_t stream) {
  if (final_state && final_state != init_state) {
    hipError_t e = timed("kla_copy_or_zero", stream, [&] { return kla::launch_copy_or_zero(init_state, final_state, state_n, stream); });
    if (e != hipSuccess) return hip_fail(e, "launch");
  }
  return KLA_OK;
}

// Enqueues prep and the state walk(s) of plan `p` with the workspace at `base`
// (p.total bytes, 256-byte aligned, owned by the caller of this function).
hipError_t chunk_fwd_enqueue(const Plan& p, kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k,
                             const void* v, const float* log_alpha, const float* eta, float eps,
                             const float* init_state, float* out, float* final_state, int B, int T, int H, int dk,
                             int dv, int lift, uint8_t* base, hipStream_t stream) {
  const kla::Dims dp{B, T, H, dk, dv, (T + kChunk - 1) / kChunk, lift};
  const kla::Dims d{B, T, H, dk, dv, (T + kChunk - 1) / kChunk, 0};
  const int mode = dtype == KLA_DTYPE_BF16 ? 0 : 1;
  uint8_t* rec = base + p.rec_off;
  float* maps = reinterpret_cast<float*>(base + p.maps_off);
  float* starts = reinterpret_cast<float*>(base + p.starts_off);
  const int direct = beta_mode == KLA_BETA_DIRECT;
  // PSD lift: prep forms its fragments from the u rows and writes the lifted rows, which the
  // walks read in their place
  void* fq = lift ? base + p.lift_off : nullptr;
  void* fk = lift ? base + p.lift_off + p.lift_bytes : nullptr;
  hipError_t e = timed("kla_prep", stream, [&] {
    return kla::launch_prep(mode, dp, q, k, log_alpha, eta, eps, direct, rec, stream, fq, fk);
  });
  if (lift) {
    q = fq;
    k = fk;
  }
  if (e == hipSuccess) {
    if (p.path == KLA_PATH_SEQUENTIAL) {
      e = timed("kla_state_seq", stream, [&] {
        return kla::launch_state_seq(mode, d, q, k, v, rec, init_state, out, final_state, stream);
      });
    } else {
      e = timed("kla_scan_maps", stream, [&] {
        return kla::launch_scan_maps(mode, d, k, v, rec, p.seg_chunks, p.segs, maps, init_state == nullptr, stream);
      });
      if (e == hipSuccess)
        e = timed("kla_scan_starts", stream, [&] { return kla::launch_scan_starts(d, maps, init_state, p.segs, starts, stream); });
      if (e == hipSuccess)
        e = timed("kla_scan_apply", stream, [&] {
          return kla::launch_scan_apply(mode, d, q, k, v, rec, p.seg_chunks, p.segs, starts, out, final_state, stream);
        });
    }
  }
  return e;
}

kla_status chunk_fwd_impl(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k, const void* v,
                          const float* log_alpha, const float* eta, float eps, const float* init_state, float* out,
                          float* final_state, int B, int T, int H, int dk, int dv, int chunk, kla_path path,
                          int segments, hipStream_t stream, int lift = 0) {
  kla_status st = chunk_fwd_check(dtype, beta_mode, q, k, v, log_alpha, eta, init_state, out, final_state, B, T, H,
                                  dk, dv, chunk, path, segments);
  if (st != KLA_OK) return st;
  if (T == 0) return chunk_fwd_empty(init_state, final_state, static_cast<size_t>(B) * H * dk * dv, stream);

  Plan p = make_plan(dtype, B, T, H, dk, dv, path, segments, device_cus());
  if (lift) plan_lift(p, B, T, H, dk);
  void* ws = nullptr;
  st = workspace_alloc(&ws, p.total, stream);
  if (st != KLA_OK) return st;
  hipError_t e = chunk_fwd_enqueue(p, dtype, beta_mode, q, k, v, log_alpha, eta, eps, init_state, out, final_state,
                                   B, T, H, dk, dv, lift, static_cast<uint8_t*>(ws), stream);
  hipError_t ef = hipFreeAsync(ws, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync");
  return KLA_OK;
}

kla_status decode_impl(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* eta, float eps, float* state, float* out, int N, int H,
                       int dk, int dv, hipStream_t stream) {
  if (dtype != KLA_DTYPE_BF16 && dtype != KLA_DTYPE_F32) return fail(KLA_ERR_INVALID_ARG, "unknown dtype");
  if (beta_mode != KLA_BETA_KACZMARZ && beta_mode != KLA_BETA_DIRECT)
    return fail(KLA_ERR_INVALID_ARG, "unknown beta_mode %d", (int)beta_mode);
  if (N < 0 || H < 1) return fail(KLA_ERR_INVALID_ARG, "sizes must satisfy N >= 0, H >= 1 (got N=%d H=%d)", N, H);
  if (dk < 1 || dv < 1) return fail(KLA_ERR_INVALID_ARG, "dk and dv must be positive");
  if (!supported_dk(dk)) return fail(KLA_ERR_UNSUPPORTED, "dk=%d not supported (64, 128, 256)", dk);
  if (!supported_dv(dv)) return fail(KLA_ERR_UNSUPPORTED, "dv=%d not supported (64, 128)", dv);
  if (static_cast<long long>(N) * H > 2147483647LL) return fail(KLA_ERR_UNSUPPORTED, "N*H too large");
  if (N == 0) return KLA_OK;
  if (!q || !k || !v || !log_alpha || !eta || !state || !out)
    return fail(KLA_ERR_INVALID_ARG, "q, k, v, log_alpha, eta, state and out must be non-null");
  kla_status st = check_aligned("q, k, v, log_alpha, eta, state, out", q, k, v, log_alpha, eta, state, out);
  if (st != KLA_OK) return st;
  const int mode = dtype == KLA_DTYPE_BF16 ? 0 : 1;
  hipError_t e = timed("kla_decode", stream, [&] {
    return kla::launch_decode(mode, N, H, dk, dv, q, k, v, log_alpha, eta, eps, beta_mode == KLA_BETA_DIRECT, state,
                              out, stream);
  });
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return KLA_OK;
}

}  // namespace

extern "C" {

kla_status kla_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* eta,
                         float eps, const float* init_state, float* out, float* final_state, int B, int T, int H,
                         int dk, int dv, int chunk, hipStream_t stream) {
  return chunk_fwd_impl(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, q, k, v, log_alpha, eta, eps, init_state, out, final_state,
                        B, T, H, dk, dv, chunk, KLA_PATH_AUTO, 0, stream);
}

kla_status kla_chunk_fwd_f32(const float* q, const float* k, const float* v, const float* log_alpha,
                             const float* eta, float eps, const float* init_state, float* out, float* final_state,
                             int B, int T, int H, int dk, int dv, int chunk, hipStream_t stream) {
  return chunk_fwd_impl(KLA_DTYPE_F32, KLA_BETA_KACZMARZ, q, k, v, log_alpha, eta, eps, init_state, out, final_state,
                        B, T, H, dk, dv, chunk, KLA_PATH_AUTO, 0, stream);
}

kla_status kla_chunk_fwd_ex(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k, const void* v,
                            const float* log_alpha, const float* eta, float eps, const float* init_state, float* out,
                            float* final_state, int B, int T, int H, int dk, int dv, int chunk, kla_path path,
                            int segments, hipStream_t stream) {
  return chunk_fwd_impl(dtype, beta_mode, q, k, v, log_alpha, eta, eps, init_state, out, final_state, B, T, H, dk, dv,
                        chunk, path, segments, stream);
}

kla_status kla_chunk_fwd_noalloc(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k,
                                 const void* v, const float* log_alpha, const float* eta, float eps,
                                 const float* init_state, float* out, float* final_state, int B, int T, int H, int dk,
                                 int dv, int chunk, kla_path path, int segments, hipStream_t stream) {
  kla_status st = chunk_fwd_check(dtype, beta_mode, q, k, v, log_alpha, eta, init_state, out, final_state, B, T, H,
                                  dk, dv, chunk, path, segments);
  if (st != KLA_OK) return st;
  if (T == 0) return chunk_fwd_empty(init_state, final_state, static_cast<size_t>(B) * H * dk * dv, stream);
  const Plan p = make_plan(dtype, B, T, H, dk, dv, path, segments, device_cus());
  if (p.total > static_cast<size_t>(KLA_NOALLOC_SCRATCH_BYTES))
    return fail(KLA_ERR_UNSUPPORTED,
                "the workspace of this call (%zu bytes) exceeds the static scratch buffer of kla_chunk_fwd_noalloc "
                "(%zu bytes); use kla_chunk_fwd_ex, or fewer tokens or heads per call",
                p.total, static_cast<size_t>(KLA_NOALLOC_SCRATCH_BYTES));
  void* base = nullptr;
  size_t cap = 0;
  hipError_t e = kla::scratch_buffer(&base, &cap);
  if (e != hipSuccess) return hip_fail(e, "device address of the scratch buffer");
  if (cap < p.total) return fail(KLA_ERR_UNSUPPORTED, "scratch buffer of %zu bytes too small for %zu", cap, p.total);
  e = chunk_fwd_enqueue(p, dtype, beta_mode, q, k, v, log_alpha, eta, eps, init_state, out, final_state, B, T, H, dk,
                        dv, 0, static_cast<uint8_t*>(base), stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return KLA_OK;
}

kla_status kla_chunk_fwd_psd(const void* uq, const void* uk, const void* v, const float* log_alpha,
                             const float* eta, float eps, const float* init_state, float* out, float* final_state,
                             int B, int T, int H, int p, int dv, int chunk, kla_path path, int segments,
                             hipStream_t stream) {
  if (p < 1) return fail(KLA_ERR_INVALID_ARG, "p must be positive");
  if (p != kla::LIFT_P_HOST) return fail(KLA_ERR_UNSUPPORTED, "psd lift supports p=%d only (got %d)", kla::LIFT_P_HOST, p);
  return chunk_fwd_impl(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, uq, uk, v, log_alpha, eta, eps, init_state, out,
                        final_state, B, T, H, p * p, dv, chunk, path, segments, stream, /*lift=*/1);
}

kla_status kla_plan(kla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk, kla_path path, int segments,
                    int num_cus, kla_path* chosen_path, int* chosen_segments, size_t* workspace_bytes) {
  if (dtype != KLA_DTYPE_BF16 && dtype != KLA_DTYPE_F32) return fail(KLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  kla_status st = check_prefill_sizes(dtype, B, T, H, dk, dv, chunk);
  if (st != KLA_OK) return st;
  if (path != KLA_PATH_AUTO && path != KLA_PATH_SEQUENTIAL && path != KLA_PATH_SCAN)
    return fail(KLA_ERR_INVALID_ARG, "unknown path %d", (int)path);
  if (segments < 0) return fail(KLA_ERR_INVALID_ARG, "segments must be >= 0");
  const int cus = num_cus > 0 ? num_cus : device_cus();
  Plan p{};
  if (T > 0) p = make_plan(dtype, B, T, H, dk, dv, path, segments, cus);
  else p.path = KLA_PATH_SEQUENTIAL, p.segs = 1;
  if (chosen_path) *chosen_path = p.path;
  if (chosen_segments) *chosen_segments = p.segs;
  if (workspace_bytes) *workspace_bytes = p.total;
  return KLA_OK;
}

kla_status kla_decode_step(const void* q, const void* k, const void* v, const float* log_alpha, const float* eta,
                           float eps, float* state, float* out, int N, int H, int dk, int dv, hipStream_t stream) {
  return decode_impl(KLA_DTYPE_BF16, KLA_BETA_KACZMARZ, q, k, v, log_alpha, eta, eps, state, out, N, H, dk, dv, stream);
}

kla_status kla_decode_step_f32(const float* q, const float* k, const float* v, const float* log_alpha,
                               const float* eta, float eps, float* state, float* out, int N, int H, int dk, int dv,
                               hipStream_t stream) {
  return decode_impl(KLA_DTYPE_F32, KLA_BETA_KACZMARZ, q, k, v, log_alpha, eta, eps, state, out, N, H, dk, dv, stream);
}

kla_status kla_loglinear_decode_step(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k,
                                     const void* v, const float* log_alpha, const float* eta, const float* lam,
                                     float eps, float* states, float* out, int N, int H, int dk, int dv, int levels,
                                     int t, hipStream_t stream) {
  if (dtype != KLA_DTYPE_BF16 && dtype != KLA_DTYPE_F32) return fail(KLA_ERR_INVALID_ARG, "unknown dtype");
  if (beta_mode != KLA_BETA_KACZMARZ && beta_mode != KLA_BETA_DIRECT)
    return fail(KLA_ERR_INVALID_ARG, "unknown beta_mode %d", (int)beta_mode);
  if (N < 0 || H < 1) return fail(KLA_ERR_INVALID_ARG, "sizes must satisfy N >= 0, H >= 1 (got N=%d H=%d)", N, H);
  if (dk < 1 || dv < 1) return fail(KLA_ERR_INVALID_ARG, "dk and dv must be positive");
  if (levels < 1 || levels > 31) return fail(KLA_ERR_INVALID_ARG, "levels must be in 1..31 (got %d)", levels);
  if (t < 0 || static_cast<long long>(t) >= (1LL << (levels - 1)))
    return fail(KLA_ERR_INVALID_ARG, "position t=%d needs 0 <= t < 2^(levels-1) with levels=%d", t, levels);
  if (!supported_dk(dk)) return fail(KLA_ERR_UNSUPPORTED, "dk=%d not supported (64, 128, 256)", dk);
  if (!supported_dv(dv)) return fail(KLA_ERR_UNSUPPORTED, "dv=%d not supported (64, 128)", dv);
  if (static_cast<long long>(N) * H > 2147483647LL) return fail(KLA_ERR_UNSUPPORTED, "N*H too large");
  if (N == 0) return KLA_OK;
  if (!q || !k || !v || !log_alpha || !eta || !lam || !states || !out)
    return fail(KLA_ERR_INVALID_ARG, "q, k, v, log_alpha, eta, lam, states and out must be non-null");
  kla_status st = check_aligned("q, k, v, log_alpha, eta, lam, states, out", q, k, v, log_alpha, eta, lam, states, out);
  if (st != KLA_OK) return st;
  const int mode = dtype == KLA_DTYPE_BF16 ? 0 : 1;
  hipError_t e = timed("kla_loglinear_decode", stream, [&] {
    return kla::launch_loglinear_decode(mode, N, H, dk, dv, q, k, v, log_alpha, eta, lam, eps,
                                        beta_mode == KLA_BETA_DIRECT, states, out, levels, t, stream);
  });
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return KLA_OK;
}

kla_status kla_loglinear_fwd(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* eta, const float* lam, float eps, float* out, int B,
                             int T, int H, int dk, int dv, int levels, int chunk, hipStream_t stream) {
  if (dtype != KLA_DTYPE_BF16 && dtype != KLA_DTYPE_F32) return fail(KLA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  kla_status st = check_prefill_sizes(dtype, B, T, H, dk, dv, chunk);
  if (st != KLA_OK) return st;
  if (beta_mode != KLA_BETA_KACZMARZ && beta_mode != KLA_BETA_DIRECT)
    return fail(KLA_ERR_INVALID_ARG, "unknown beta_mode %d", (int)beta_mode);
  if (levels < 1 || levels > 31) return fail(KLA_ERR_INVALID_ARG, "levels must be in 1..31 (got %d)", levels);
  if (static_cast<long long>(T) > (1LL << (levels - 1)))
    return fail(KLA_ERR_INVALID_ARG, "T=%d needs T <= 2^(levels-1) with levels=%d", T, levels);
  if (T == 0) return KLA_OK;
  if (!q || !k || !v || !log_alpha || !eta || !lam || !out)
    return fail(KLA_ERR_INVALID_ARG, "q, k, v, log_alpha, eta, lam and out must be non-null when T > 0");
  st = check_aligned("q, k, v, log_alpha, eta, lam, out", q, k, v, log_alpha, eta, lam, out);
  if (st != KLA_OK) return st;
  const int nc = (T + kChunk - 1) / kChunk;
  kla::Dims d{B, T, H, dk, dv, nc};
  d.full_rec = 1;
  const int mode = dtype == KLA_DTYPE_BF16 ? 0 : 1;
  const size_t bh = static_cast<size_t>(B) * H;
  // scales s >= 0 (level 7 + s): half-blocks of 2^s chunks while a right half-block exists
  int nscale = 0, half[32], nleft[32], nright[32];
  for (int hb = 1; hb < nc && nscale < 32; hb *= 2, ++nscale) {
    const int nblk = (nc + hb - 1) / hb;
    half[nscale] = hb;
    nleft[nscale] = (nblk + 1) / 2;
    nright[nscale] = nblk / 2;
  }
  const int direct = beta_mode == KLA_BETA_DIRECT;
  void* ws = nullptr;
  hipError_t e = hipSuccess;
  if (kla::state_dma_supported(mode, dk)) {
    // bf16 with dk <= 128: one prep pass of compact records (T' and the gates; the intra-chunk
    // kernel and the walks form P themselves); then per scale one walk over its right
    // half-blocks that starts from the end states of the scale below, held in two buffers
    // used in turn
    const size_t crec_bytes = align256(bh * nc * static_cast<size_t>(kla::record_bytes(mode, dk)));
    size_t carry = 0;
    for (int i = 1; i < nscale; ++i) carry = std::max(carry, bh * nright[i] * static_cast<size_t>(dk) * dv);
    const size_t carry_bytes = align256(carry * 4);
    st = workspace_alloc(&ws, crec_bytes + 2 * carry_bytes, stream);
    if (st != KLA_OK) return st;
    uint8_t* crec = static_cast<uint8_t*>(ws);
    float* carried[2] = {reinterpret_cast<float*>(crec + crec_bytes),
                         reinterpret_cast<float*>(crec + crec_bytes + carry_bytes)};
    kla::Dims dc = d;
    dc.full_rec = 0;
    e = timed("kla_prep", stream, [&] { return kla::launch_prep(mode, dc, q, k, log_alpha, eta, eps, direct, crec, stream); });
    if (e == hipSuccess)
      e = timed("kla_loglinear_intra", stream, [&] {
        return kla::launch_loglinear_intra_compact(d, q, k, crec, v, lam, levels, out, stream);
      });
    for (int i = 0; e == hipSuccess && i < nscale; ++i) {
      e = timed("kla_loglinear_scale", stream, [&] {
        return kla::launch_loglinear_scale_dma(dk, q, k, v, crec, T, H, dv, nc, static_cast<int>(bh), i, nright[i],
                                               i > 0 ? carried[(i - 1) & 1] : nullptr,
                                               i + 1 < nscale ? carried[i & 1] : nullptr,
                                               i + 1 < nscale ? nright[i + 1] : 0, lam, levels, out, stream);
      });
    }
  } else {
    // full records; every scale's left end states kept at once (at most nc states per head)
    const size_t rec_bytes = align256(bh * nc * kla::full_record_bytes());
    long long ends_off[32];
    long long ends_floats = 0;
    for (int i = 0; i < nscale; ++i) {
      ends_off[i] = ends_floats;
      ends_floats += static_cast<long long>(bh) * nleft[i] * dk * dv;
    }
    st = workspace_alloc(&ws, rec_bytes + align256(static_cast<size_t>(ends_floats) * 4), stream);
    if (st != KLA_OK) return st;
    uint8_t* rec = static_cast<uint8_t*>(ws);
    float* ends = reinterpret_cast<float*>(rec + rec_bytes);
    e = timed("kla_prep", stream, [&] { return kla::launch_prep(mode, d, q, k, log_alpha, eta, eps, direct, rec, stream); });
    if (e == hipSuccess)
      e = timed("kla_loglinear_intra", stream, [&] { return kla::launch_loglinear_intra(mode, d, rec, v, lam, levels, out, stream); });
    // every scale's left walks in one grid (they are independent), then the right walks scale by
    // scale (the scales add to the same outputs)
    if (e == hipSuccess && nscale > 0)
      e = timed("kla_loglinear_left", stream, [&] {
        return kla::launch_loglinear_left(mode, d, k, v, rec, nscale, half, nleft, ends_off, ends, stream);
      });
    for (int i = 0; e == hipSuccess && i < nscale; ++i) {
      e = timed("kla_loglinear_right", stream, [&] {
        return kla::launch_loglinear_right(mode, d, q, k, rec, half[i], nright[i], ends + ends_off[i], nleft[i], lam,
                                           levels, 7 + i, out, stream);
      });
    }
  }
  hipError_t ef = hipFreeAsync(ws, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync");
  return KLA_OK;
}

kla_status kla_chunk_bwd(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k, const void* v,
                         const float* log_alpha, const float* eta, float eps, const float* init_state,
                         const float* grad_out, const float* grad_final_state, float* grad_q, float* grad_k,
                         float* grad_v, float* grad_log_alpha, float* grad_eta, float* grad_init_state, int B, int T,
                         int H, int dk, int dv, int chunk, hipStream_t stream) {
  kla_status st = check_prefill_sizes(dtype, B, T, H, dk, dv, chunk);
  if (st != KLA_OK) return st;
  if (dk > 128 && dtype != KLA_DTYPE_BF16)
    return fail(KLA_ERR_UNSUPPORTED, "the fp32 backward supports dk in {64, 128} (got %d)", dk);
  if (beta_mode != KLA_BETA_KACZMARZ && beta_mode != KLA_BETA_DIRECT)
    return fail(KLA_ERR_INVALID_ARG, "unknown beta_mode %d", (int)beta_mode);
  if (T > 0 && (!q || !k || !v || !log_alpha || !eta || !grad_out || !grad_q || !grad_k || !grad_v ||
                !grad_log_alpha || !grad_eta))
    return fail(KLA_ERR_INVALID_ARG,
                "q, k, v, log_alpha, eta, grad_out and grad_q .. grad_eta must be non-null when T > 0");
  st = check_aligned("q, k, v, log_alpha, eta, init_state, grad_out, grad_final_state, grad_q .. grad_init_state", q,
                     k, v, log_alpha, eta, init_state, grad_out, grad_final_state, grad_q, grad_k, grad_v,
                     grad_log_alpha, grad_eta, grad_init_state);
  if (st != KLA_OK) return st;
  const size_t state_n = static_cast<size_t>(B) * H * dk * dv;
  if (T == 0) {  // the start state's gradient is the end state's
    if (grad_init_state && grad_init_state != grad_final_state) {
      hipError_t e = timed("kla_copy_or_zero", stream, [&] {
        return kla::launch_copy_or_zero(grad_final_state, grad_init_state, state_n, stream);
      });
      if (e != hipSuccess) return hip_fail(e, "launch");
    }
    return KLA_OK;
  }
  const int nc = (T + kChunk - 1) / kChunk;
  const size_t nch = static_cast<size_t>(B) * H * nc;
  const int mode = dtype == KLA_DTYPE_BF16 ? 0 : 1;
  // Few heads over a long sequence (where the forward takes the scan path): both walks run in
  // segments, in parallel. The forward walk starts each segment from the state the forward
  // scan's maps and fold give; the reverse walk folds the transposed segment maps over the
  // segments' zero-end walks, then walks every segment from its end gradient. Needs the DMA
  // map kernel (bf16, dk <= 128).
  const Plan fp = make_plan(dtype, B, T, H, dk, dv, KLA_PATH_AUTO, 0, device_cus());
  const bool segmented = fp.path == KLA_PATH_SCAN && fp.segs >= 2 && kla::state_dma_supported(mode, dk);
  const int segs = segmented ? fp.segs : 1, segc = segmented ? fp.seg_chunks : nc;
  const size_t bh = static_cast<size_t>(B) * H;
  const size_t map_bytes = segmented ? align256(bh * (segs - 1) * dk * (dk + dv) * 4) : 0;
  const size_t seg_state_bytes = segmented ? align256(bh * segs * dk * dv * 4) : 0;
  const size_t base_bytes = align256(kla::bwd_workspace_bytes(B, T, H, dk, dv));
  const size_t bytes = base_bytes + (segmented ? fp.rec_bytes + 2 * map_bytes + 3 * seg_state_bytes : 0);
  void* ws = nullptr;
  st = workspace_alloc(&ws, bytes, stream);
  if (st != KLA_OK) return st;
  hipError_t e = hipSuccess;
  kla::BwdArgs a{};
  a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv; a.nc = nc;
  a.direct = beta_mode == KLA_BETA_DIRECT;
  a.eps = eps;
  a.q = q; a.k = k; a.v = v;
  a.log_alpha = log_alpha; a.eta = eta; a.init = init_state; a.dout = grad_out; a.dfin = grad_final_state;
  a.rec = static_cast<float*>(ws);
  a.states = a.rec + nch * kla::bwd_record_floats();
  a.dstates = a.states + nch * dk * dv;
  a.vt = a.dstates + nch * dk * dv;
  a.gq = grad_q; a.gk = grad_k; a.gv = grad_v; a.gla = grad_log_alpha; a.geta = grad_eta; a.ginit = grad_init_state;
  static const char* const names[5] = {"kla_bwd_prep", "kla_bwd_states", "kla_bwd_dprep", "kla_bwd_dstates",
                                       "kla_bwd_grads"};
  if (!segmented) {
    for (int stage = 0; e == hipSuccess && stage < 5; ++stage)
      e = timed(names[stage], stream, [&] { return kla::launch_bwd(mode, a, stage, stream); });
  } else {
    uint8_t* x = static_cast<uint8_t*>(ws) + base_bytes;
    uint8_t* crec = x;
    float* maps_f = reinterpret_cast<float*>(crec + fp.rec_bytes);
    float* maps_r = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(maps_f) + map_bytes);
    float* starts = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(maps_r) + map_bytes);
    float* zero_ends = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(starts) + seg_state_bytes);
    float* gends = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(zero_ends) + seg_state_bytes);
    const kla::Dims d{B, T, H, dk, dv, nc};
    const int direct = beta_mode == KLA_BETA_DIRECT;
    const int ncg = (dk + dv) / 64;
    e = timed(names[0], stream, [&] { return kla::launch_bwd(mode, a, 0, stream); });
    // the forward walk: segment start states from the forward scan's maps and fold
    if (e == hipSuccess)
      e = timed("kla_prep", stream, [&] { return kla::launch_prep(mode, d, q, k, log_alpha, eta, eps, direct, crec, stream); });
    if (e == hipSuccess)
      e = timed("kla_scan_maps", stream, [&] { return kla::launch_scan_maps(mode, d, k, v, crec, segc, segs, maps_f, init_state == nullptr, stream); });
    if (e == hipSuccess)
      e = timed("kla_scan_starts", stream, [&] { return kla::launch_scan_starts(d, maps_f, init_state, segs, starts, stream); });
    if (e == hipSuccess)
      e = timed(names[1], stream, [&] {
        return kla::launch_bwd_walk_segs(mode, a, false, kla::WalkSegs{segc, segs, 0, starts, segs, nullptr, 1, 1}, stream);
      });
    if (e == hipSuccess) e = timed(names[2], stream, [&] { return kla::launch_bwd(mode, a, 2, stream); });
    // the reverse walk: maps of segments 1 .. segs - 1, their walks from a zero end gradient,
    // the fold, then every segment from its end gradient
    if (e == hipSuccess)
      e = timed("kla_bwd_rev_maps", stream, [&] {
        return kla::launch_state_dma(false, true, dk, ncg * (segs - 1) * B * H, nullptr, k, v, crec, T, H, dv, nc, segc,
                                     nullptr, 1, nullptr, maps_r, dk + dv, segs - 1, 0, ncg, segs - 1, stream, 1, 1);
      });
    if (e == hipSuccess)
      e = timed("kla_bwd_rev_zero", stream, [&] {
        return kla::launch_bwd_walk_segs(mode, a, true, kla::WalkSegs{segc, segs - 1, 1, nullptr, 1, zero_ends, segs, 0},
                                         stream);
      });
    if (e == hipSuccess)
      e = timed("kla_bwd_rev_fold", stream, [&] { return kla::launch_bwd_rev_fold(a, maps_r, zero_ends, gends, segs, stream); });
    if (e == hipSuccess)
      e = timed(names[3], stream, [&] {
        return kla::launch_bwd_walk_segs(mode, a, true, kla::WalkSegs{segc, segs, 0, gends, segs, a.ginit, 1, 1}, stream);
      });
    if (e == hipSuccess) e = timed(names[4], stream, [&] { return kla::launch_bwd(mode, a, 4, stream); });
  }
  hipError_t ef = hipFreeAsync(ws, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync");
  return KLA_OK;
}

kla_status kla_decode_step_ex(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k, const void* v,
                              const float* log_alpha, const float* eta, float eps, float* state, float* out, int N,
                              int H, int dk, int dv, hipStream_t stream) {
  return decode_impl(dtype, beta_mode, q, k, v, log_alpha, eta, eps, state, out, N, H, dk, dv, stream);
}

kla_status kla_workspace_trim(void) {
  hipMemPool_t pool = nullptr;
  hipError_t e = library_pool(&pool);
  if (e == hipSuccess) e = hipMemPoolTrimTo(pool, 0);
  if (e != hipSuccess) return hip_fail(e, "trimming the workspace pool");
  return KLA_OK;
}

const char* kla_last_error(void) { return g_err.c_str(); }

const char* kla_version(void) { return "kla-mi355x 0.1.0 (gfx950)"; }

kla_status kla_timing_enable(int enable) {
  g_timing.enabled = enable != 0;
  return KLA_OK;
}

kla_status kla_timing_select(const char* kernel) {
  if (kernel && std::strlen(kernel) >= sizeof g_timing.only)
    return fail(KLA_ERR_INVALID_ARG, "kernel name too long for the timing hook (%zu characters)", std::strlen(kernel));
  std::snprintf(g_timing.only, sizeof g_timing.only, "%s", kernel ? kernel : "");
  return KLA_OK;
}

int kla_timing_collect(kla_kernel_timing* out, int max) {
  struct Acc {
    const char* name;
    int n;
    double ms;
  };
  std::vector<Acc> acc;
  bool err = false;
  const TimedLaunch* prev = nullptr;
  for (auto& t : g_timing.rec) {
    float ms = 0.f;
    if (hipEventSynchronize(t.stop) != hipSuccess || hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess) {
      err = true;
    } else {
      // A dispatch can take its start stamp while it still waits for the kernel before it
      // on the stream; the kernel runs only from that kernel's end, so the overlap is not
      // counted (launches timed from one thread go to one stream in order).
      float overlap = 0.f;
      if (prev && hipEventElapsedTime(&overlap, t.start, prev->stop) == hipSuccess && overlap > 0.f)
        ms -= std::min(overlap, ms);
    }
    prev = &t;
    if (!err) {
      auto it = std::find_if(acc.begin(), acc.end(), [&](const Acc& a) { return std::strcmp(a.name, t.name) == 0; });
      if (it == acc.end()) acc.push_back({t.name, 1, ms});
      else {
        it->n += 1;
        it->ms += ms;
      }
    }
  }
  for (auto& t : g_timing.rec) {
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  g_timing.rec.clear();
  if (err) {
    fail(KLA_ERR_HIP, "timing events could not be read");
    return -1;
  }
  for (int i = 0; i < static_cast<int>(acc.size()) && i < max && out; ++i) {
    std::snprintf(out[i].name, sizeof out[i].name, "%s", acc[i].name);
    out[i].launches = acc[i].n;
    out[i].total_ms = acc[i].ms;
  }
  return static_cast<int>(acc.size());
}

}  // extern "C"
