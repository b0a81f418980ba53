// Host-side launchers of the KLA kernels (internal to libkla; not part of the C ABI).
// Every launcher only enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kla {

// Events the next kernel launch stamps with its own start and end (set by the library's
// timing hook, null otherwise). hipExtLaunchKernelGGL takes both timestamps from the
// kernel's dispatch, so the interval is the kernel's execution alone, as a profiler's
// kernel trace reports it.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

// Every kernel of the library is launched through this (arguments are converted to the
// kernel's parameter types); returns the launch status. With timing on, the first launch of a
// timed call stamps the start event from its dispatch and every launch restamps the stop
// event, so a call that enqueues several kernels is timed from the first one's start to the
// last one's end.
template <class F, class... A>
inline hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t stream, A... args) {
  LaunchEvents& ev = launch_events();
  hipEvent_t start = ev.start;
  ev.start = nullptr;
  hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, ev.stop, 0, args...);
  return hipGetLastError();
}

// Width of the u rows that the fused PSD lift takes (the kernels' LIFT_P).
constexpr int LIFT_P_HOST = 16;

// Per-launch size bundle shared by the prefill kernels.
struct Dims {
  int B, T, H, dk, dv;
  int nc;        // number of 64-token chunks, ceil(T / 64)
  int lift = 0;  // prep only: q and k hold 16-wide u rows, and prep forms the dk = 256 PSD features
  int full_rec = 0;  // prep writes the full record (T' and P) whatever the dtype and dk
};

// Chunk prep: one wavefront per (b, h, chunk); writes one record per chunk. `direct` takes
// beta = eta as given instead of the Kaczmarz step eta / (||k||^2 + eps). With d.lift, q and k
// are u rows and prep also writes the lifted query and key rows ([B, T, H, dk] bf16) to fq, fk.
hipError_t launch_prep(int mode, const Dims& d, const void* q, const void* k, const float* log_alpha,
                       const float* eta, float eps, int direct, uint8_t* rec, hipStream_t stream,
                       void* fq = nullptr, void* fk = nullptr);

// Sequential inter-chunk state + output: one workgroup per (b, h, 64-column group of dv).
// init may be null (zero state); fin may be null (not written).
hipError_t launch_state_seq(int mode, const Dims& d, const void* q, const void* k, const void* v,
                            const uint8_t* rec, const float* init, float* out, float* fin,
                            hipStream_t stream);

// Scan path.
//  phase 1: affine map [M | N] of each of the first `segs - 1` segments of `seg_chunks` chunks
//  phase 2: start state of every segment, sequentially over segments
//  phase 3: state + output inside every segment from its start state
// zero_start: the scan starts from a zero state (no init), so segment 0's M is not needed; the
// map walk skips it and launch_scan_starts (given init = null) never reads it.
hipError_t launch_scan_maps(int mode, const Dims& d, const void* k, const void* v, const uint8_t* rec,
                            int seg_chunks, int segs, float* maps, bool zero_start, hipStream_t stream);
hipError_t launch_scan_starts(const Dims& d, const float* maps, const float* init, int segs,
                              float* starts, hipStream_t stream);
hipError_t launch_scan_apply(int mode, const Dims& d, const void* q, const void* k, const void* v,
                             const uint8_t* rec, int seg_chunks, int segs, const float* starts,
                             float* out, float* fin, hipStream_t stream);

// DMA-fed state kernel (kla_state_dma.hip): bf16 inputs with dk in {64, 128}.
bool state_dma_supported(int mode, int dk);
// Bytes of one chunk record: compact (no P, T' without its zero quadrant) when the DMA-fed
// state kernel consumes it, else the full record.
int record_bytes(int mode, int dk);
int full_record_bytes();  // T' and P in full, for the kernels that read both
// Segment s walks chunks [(s * seg_mul + seg_add) * seg_chunks, + seg_chunks).
hipError_t launch_state_dma(bool with_out, bool aug, int dk, int nwg, const void* q, const void* k, const void* v,
                            const uint8_t* rec, int T, int H, int DV, int nc, int seg_chunks, const float* init,
                            int init_segs, float* out, float* fin, int fin_ld, int fin_segs, int fin_last_only,
                            int ncg, int nseg, hipStream_t stream, int seg_mul = 1, int seg_add = 0,
                            int skip_ident0 = 0);
// Log-linear prefill on compact records (bf16, dk in {64, 128}, DV a multiple of 64): the walk of
// chunk scale s (level 7 + s of L) over its nright right half-blocks of 2^s chunks per head, each
// from the state [B*H][nright][dk][DV] in init (written by scale s - 1; scale 0 starts every
// pair of chunks from zero and takes null), adding its weighted outputs to out, and leaving the
// end states of its even half-blocks in fin ([B*H][fin_segs][dk][DV], fin_segs = the next
// scale's nright; null for the last scale). See state_walk_kernel.
hipError_t launch_loglinear_scale_dma(int dk, const void* q, const void* k, const void* v, const uint8_t* rec, int T,
                                      int H, int DV, int nc, int BH, int s, int nright, const float* init, float* fin,
                                      int fin_segs, const float* lam, int L, float* out, hipStream_t stream);

// Log-linear decode: one token at position t for N x H heads, each with L bucket states
// [L, dk, dv] (only the occupied levels are read or written).
hipError_t launch_loglinear_decode(int mode, int N, int H, int dk, int dv, const void* q, const void* k,
                                   const void* v, const float* log_alpha, const float* eta, const float* lam,
                                   float eps, int direct, float* states, float* out, int L, int t,
                                   hipStream_t stream);

// Log-linear prefill (full records; fp32, or dk = 256). Intra-chunk levels 0..6 written to out;
// the zero-start end state of every left half-block of every scale l >= 7 (half-blocks of
// 2^(l-7) chunks) into ends, per scale [B*H][nleft][dk][dv]; then per scale the walk over every
// right half-block from its left sibling's end state with no values, lambda^(l)-weighted outputs
// added to out.
hipError_t launch_loglinear_intra(int mode, const Dims& d, const uint8_t* rec, const void* v, const float* lam,
                                  int L, float* out, hipStream_t stream);
// The intra-chunk levels from compact records (bf16, dk <= 128), forming P from q and k, for the
// scale walks of launch_loglinear_scale_dma: on chunk c >= 1 every pair's weight lambda^(l) is
// taken less lambda^(7 + lowest set bit of c).
hipError_t launch_loglinear_intra_compact(const Dims& d, const void* q, const void* k, const uint8_t* crec,
                                          const void* v, const float* lam, int L, float* out, hipStream_t stream);
// All scales' left walks in one grid: scale i has half-blocks of half[i] chunks, nleft[i] left
// ones per head, and writes their end states at ends + ends_off[i] (floats).
hipError_t launch_loglinear_left(int mode, const Dims& d, const void* k, const void* v, const uint8_t* rec,
                                 int nscale, const int* half, const int* nleft, const long long* ends_off,
                                 float* ends, hipStream_t stream);
hipError_t launch_loglinear_right(int mode, const Dims& d, const void* q, const void* k, const uint8_t* rec, int half,
                                  int nright, const float* ends, int nleft, const float* lam, int L, int level,
                                  float* out, hipStream_t stream);

// Device address and size of the static scratch buffer of kla_chunk_fwd_noalloc on the
// current device (kla_scratch.hip); the address is looked up once per device.
hipError_t scratch_buffer(void** addr, size_t* bytes);

// Copy (or zero when src is null) n floats; used for T == 0 and as a graph-safe fill.
hipError_t launch_copy_or_zero(const float* src, float* dst, size_t n, hipStream_t stream);

// Single-token decode for N x H states, in place (`direct` as for launch_prep).
hipError_t launch_decode(int mode, int N, int H, int dk, int dv, const void* q, const void* k,
                         const void* v, const float* log_alpha, const float* eta, float eps, int direct,
                         float* state, float* out, hipStream_t stream);

// Chunkwise backward (kla_bwd.hip). Workspace: per chunk one record, two dk x dv states and a
// 64 x dv block.
struct BwdArgs {
  int B, T, H, dk, dv, nc, direct;
  float eps;
  const void *q, *k, *v;
  const float *log_alpha, *eta, *init, *dout, *dfin;
  float *rec, *states, *dstates, *vt;               // workspace parts
  float *gq, *gk, *gv, *gla, *geta, *ginit;         // gradients (ginit may be null)
};
// Segments of a backward walk launch: segments seg0 .. seg0 + nseg - 1 of seg_chunks chunks;
// each starts from sin's slot (bh, segment) of sin_segs per head (null: zero), stores every
// chunk's carried matrix when dump is set, and leaves its final one in slast's slot
// (bh, segment) when segment < slast_segs.
struct WalkSegs {
  int seg_chunks, nseg, seg0;
  const float* sin;
  int sin_segs;
  float* slast;
  int slast_segs, dump;
};
size_t bwd_workspace_bytes(int B, int T, int H, int dk, int dv);
// One backward walk (rev: the reverse one) over the segments of g.
hipError_t launch_bwd_walk_segs(int mode, const BwdArgs& a, bool rev, const WalkSegs& g, hipStream_t stream);
// The reverse walk's fold over segs segments (see bwd_rev_fold_kernel): maps [M | N] of segments
// 1 .. segs - 1, D the zero-end reverse walks' results, gend the end gradients of every segment.
hipError_t launch_bwd_rev_fold(const BwdArgs& a, const float* maps, const float* D, float* gend, int segs,
                               hipStream_t stream);
size_t bwd_record_floats();
// stage 0: chunk records; 1: forward walk (chunk-start states); 2: chunk-local terms of the
// reverse walk; 3: reverse walk (chunk-end state gradients, and the start state's); 4: per-chunk
// gradients.
hipError_t launch_bwd(int mode, const BwdArgs& a, int stage, hipStream_t stream);

}  // namespace kla
