/*
 * kla.h - C ABI of libkla: the forward hot path of Kaczmarz Linear Attention
 * (KLA) on AMD Instinct MI355X (gfx950).
 *
 * The operation (KLA page, "KLA update rule"; decay gate kept from Gated
 * DeltaNet, KLA page "Implementation"), for every batch b, head h and token t,
 * with a dk x dv fp32 state S per (b, h):
 *
 *     beta_t = eta_t / (||k_t||^2 + eps)        Kaczmarz step size
 *     S~     = exp(log_alpha_t) * S_{t-1}       decayed previous state
 *     e_t    = v_t - S~^T k_t                   residual
 *     S_t    = S~ + beta_t k_t e_t^T            the write: for eta_t = 1, eps = 0 it is the
 *                                               orthogonal projection of S~ onto S^T k_t = v_t
 *                                               (KLA page, "Theoretical derivation")
 *     o_t    = S_t^T q_t                        readout after the write, no query scaling
 *
 * The pages do not state the readout or where the decay applies; the reading
 * above is the one this library implements. If ||k_t||^2 + eps == 0 the write is
 * skipped (beta_t = 0).
 *
 * Conventions shared by every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller. The library
 *    never keeps a pointer after the call returns.
 *  - Layouts are dense and row-major: q, k [B,T,H,dk]; v [B,T,H,dv];
 *    log_alpha, eta [B,T,H]; states [B,H,dk,dv] with dv fastest;
 *    out [B,T,H,dv]. bf16 arrays are IEEE bfloat16 bit patterns.
 *  - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *    without waiting. Faults during execution surface at the caller's next
 *    synchronisation.
 *  - Arguments are validated before anything is enqueued; on any non-OK return
 *    nothing has been enqueued except as stated for KLA_ERR_HIP, and
 *    kla_last_error() describes the problem. Nothing aborts or throws.
 *  - Supported sizes: dk in {64, 128, 256}, dv in {64, 128}, chunk == 64.
 *    The fp32 prefill entry points support dk in {64, 128}. Other sizes give
 *    KLA_ERR_UNSUPPORTED. T need not be a multiple of the chunk.
 *  - Every array pointer must be 16-byte aligned (the kernels move rows,
 *    states and gates with 16-byte accesses); a misaligned one gives
 *    KLA_ERR_INVALID_ARG before anything is enqueued.
 *  - Calls on different streams may run concurrently. The library's mutable
 *    global state is the per-thread error text, the per-thread timing record,
 *    and one workspace memory pool per device (see kla_workspace_trim); it
 *    never changes the device's default memory pool or any other setting of
 *    the process.
 */
#ifndef KLA_H_
#define KLA_H_

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KLA_OK = 0,
  KLA_ERR_INVALID_ARG = 1, /* null pointer, negative size, ... */
  KLA_ERR_UNSUPPORTED = 2, /* valid but not implemented (dk, dv, chunk, dtype) */
  KLA_ERR_HIP = 3,         /* a HIP call failed (launch, event, ...) */
  KLA_ERR_OOM = 4          /* the stream-ordered workspace allocation failed */
} kla_status;

/*
 * The *_RANGE_MIN / *_RANGE_MAX members of the enums below are not valid arguments.
 * They make every int a value of the enum type, so that whatever int a caller passes
 * is read by the library as it is (in C++ an out-of-range value of an enum without
 * them cannot be read safely) and rejected by validation as KLA_ERR_INVALID_ARG.
 */
typedef enum {
  KLA_DTYPE_BF16 = 0,
  KLA_DTYPE_F32 = 1,
  KLA_DTYPE_RANGE_MIN = -2147483647 - 1,
  KLA_DTYPE_RANGE_MAX = 2147483647
} kla_dtype;

/*
 * Write strength beta_t of each token's update.
 *   KLA_BETA_KACZMARZ  beta_t = eta_t / (||k_t||^2 + eps): the KLA rule (KLA page,
 *                      "KLA update rule"); what kla_chunk_fwd and kla_decode_step use.
 *   KLA_BETA_DIRECT    beta_t = eta_t as given: the learned-scalar step of Gated
 *                      DeltaNet that the KLA page sets KLA against (its "Problem
 *                      statement"). eps is unused. Same kernels, same layouts.
 */
typedef enum {
  KLA_BETA_KACZMARZ = 0,
  KLA_BETA_DIRECT = 1,
  KLA_BETA_RANGE_MIN = -2147483647 - 1,
  KLA_BETA_RANGE_MAX = 2147483647
} kla_beta_mode;

typedef enum {
  KLA_PATH_AUTO = 0,       /* let the library choose */
  KLA_PATH_SEQUENTIAL = 1, /* one walk over all chunks per (b, h, 64 dv columns) */
  KLA_PATH_SCAN = 2,       /* segments composed by an associative scan over affine chunk maps */
  KLA_PATH_RANGE_MIN = -2147483647 - 1,
  KLA_PATH_RANGE_MAX = 2147483647
} kla_path;

/*
 * Chunkwise-parallel prefill (the chunkwise solver of Gated DeltaNet with
 * B = Diag(beta_1..beta_C), KLA page "Implementation"; inter-chunk propagation
 * optionally by associative scan, KATA page section 2.3 and HLA page section 4).
 * Computes out and the end state of the recurrence above over T tokens.
 *
 *   q, k, v        bf16 device arrays, layouts above
 *   log_alpha, eta fp32 device arrays [B,T,H]; alpha_t = exp(log_alpha_t)
 *   eps            fp32 stabiliser added to ||k_t||^2
 *   init_state     fp32 [B,H,dk,dv], or NULL for a zero start state
 *   out            fp32 [B,T,H,dv] (required unless T == 0)
 *   final_state    fp32 [B,H,dk,dv], or NULL to skip; may alias init_state
 *   B, T, H        sizes (B, H >= 1; T >= 0); dk, dv, chunk as supported
 * The workspace (13 KB per chunk per head for bf16 with dk <= 128, 33 KB
 * otherwise, plus the scan's segment maps) is taken from the library's
 * workspace pool, stream-ordered on `stream`, and released on it before return.
 * With T == 0, final_state receives init_state (or zeros) and out is untouched.
 */
kla_status kla_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* eta, float eps, const float* init_state, float* out,
                         float* final_state, int B, int T, int H, int dk, int dv, int chunk,
                         hipStream_t stream);

/* Same as kla_chunk_fwd with fp32 q, k, v; all products in fp32 (dk in {64, 128}). */
kla_status kla_chunk_fwd_f32(const float* q, const float* k, const float* v, const float* log_alpha,
                             const float* eta, float eps, const float* init_state, float* out,
                             float* final_state, int B, int T, int H, int dk, int dv, int chunk,
                             hipStream_t stream);

/*
 * kla_chunk_fwd with the input dtype, the write strength and the inter-chunk
 * path chosen by the caller. `segments` is the number of scan segments for
 * KLA_PATH_SCAN (0 = library choice; clamped to the number of chunks); ignored
 * otherwise. Results of both paths agree to rounding. An unknown beta_mode or
 * path returns KLA_ERR_INVALID_ARG.
 */
kla_status kla_chunk_fwd_ex(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k,
                            const void* v, const float* log_alpha, const float* eta, float eps,
                            const float* init_state, float* out, float* final_state, int B, int T,
                            int H, int dk, int dv, int chunk, kla_path path, int segments,
                            hipStream_t stream);

/*
 * kla_chunk_fwd_ex for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments, kernels and results (bit for bit) as kla_chunk_fwd_ex; the workspace is
 * a static device buffer of KLA_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends, instead of memory from the workspace pool.
 *  - A call whose workspace (kla_plan's workspace_bytes) exceeds the buffer returns
 *    KLA_ERR_UNSUPPORTED before anything is enqueued. 128 MiB holds, e.g., the chunk
 *    records of B*H = 128 heads x 4096 tokens at dk = dv = 128 in bf16 (102 MiB).
 *  - The call makes no allocation (no hipMalloc, hipMallocAsync or hipFree) while the
 *    timing hook is off (its default); with the hook on, it creates HIP events.
 *  - Every call on one GPU uses that GPU's one buffer, which keeps the last call's
 *    contents. Calls that may overlap on one GPU (different streams without ordering
 *    between them) race on it; calls ordered on one stream do not. No part of the
 *    buffer needs clearing: each call writes every byte it reads before reading it.
 */
#define KLA_NOALLOC_SCRATCH_BYTES (128u << 20)

kla_status kla_chunk_fwd_noalloc(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k,
                                 const void* v, const float* log_alpha, const float* eta, float eps,
                                 const float* init_state, float* out, float* final_state, int B, int T,
                                 int H, int dk, int dv, int chunk, kla_path path, int segments,
                                 hipStream_t stream);

/*
 * Prefill with the rank-one PSD lift fused into the kernels (KATA page, section
 * 2.2, "Capacity theory": the feature psi(u) = vec(u u^T), whose inner products
 * are squared inner products of u). The caller passes the p-wide vectors u for
 * the queries and the keys instead of the p*p features; the kernels form
 *     q_t[a*p + b] = bf16(uq_t[a] * uq_t[b]),   k_t[a*p + b] = bf16(uk_t[a] * uk_t[b])
 * (the exact product of two bf16 values rounded to the nearest bf16, ties to
 * even), and compute exactly what kla_chunk_fwd_ex does on those features with
 * dk = p*p. Chunk prep forms its fragments from u as it loads them and writes
 * the lifted query and key rows, which the state walks read, into the
 * workspace; it grows by 2 * B*T*H*p*p*2 bytes over kla_chunk_fwd_ex's (taken
 * and released like it, stream-ordered on `stream`).
 *
 *   uq, uk      bf16 device arrays [B,T,H,p]; only p == 16 (dk = 256) is supported
 *   v, gates, eps, init_state, out, final_state, B, T, H, dv, chunk, path,
 *   segments    as for kla_chunk_fwd_ex; states are [B,H,p*p,dv]
 * The write strength is the Kaczmarz step (KLA_BETA_KACZMARZ). Other p, dv or
 * chunk give KLA_ERR_UNSUPPORTED.
 */
kla_status kla_chunk_fwd_psd(const void* uq, const void* uk, const void* v, const float* log_alpha,
                             const float* eta, float eps, const float* init_state, float* out,
                             float* final_state, int B, int T, int H, int p, int dv, int chunk,
                             kla_path path, int segments, hipStream_t stream);

/*
 * Chunkwise backward of the prefill, for training (KLA page, "Implementation": the
 * model keeps Gated DeltaNet's chunkwise parallel training algorithm; the HLA page,
 * section 4, trains chunked recurrences exactly rather than by truncated
 * backpropagation through time). The gradients are those of the exact recurrence,
 * taken in reverse through each chunk's UT form. Given the inputs of a kla_chunk_fwd_ex
 * call and the gradients of a loss with respect to its outputs, it writes the
 * gradients with respect to every input:
 *   grad_out          fp32 [B,T,H,dv]   d loss / d out
 *   grad_final_state  fp32 [B,H,dk,dv]  d loss / d final_state, or NULL (zero)
 *   grad_q, grad_k    fp32 [B,T,H,dk];  grad_v fp32 [B,T,H,dv]
 *   grad_log_alpha, grad_eta            fp32 [B,T,H]
 *   grad_init_state   fp32 [B,H,dk,dv], or NULL (not written)
 * Every output is overwritten (not accumulated). q, k, v, gates, eps, init_state
 * (NULL: zero), beta_mode and sizes are as for kla_chunk_fwd_ex; dk must be 64
 * or 128 for fp32 inputs, 64, 128 or 256 for bf16 inputs. In Kaczmarz mode a token
 * with ||k||^2 + eps == 0 has beta = 0 and passes no gradient to eta or through beta
 * to k. Products are fp32-accurate: fp32 MFMA, or for bf16 inputs the bf16 MFMA with
 * the exact bf16 keys and queries against hi + lo bf16 pairs of the fp32 operands;
 * sums are fp32. Where the forward would take the scan path (few heads over a long
 * sequence; bf16, dk <= 128), both walks run in segments: the forward walk from the
 * forward scan's segment start states, the reverse walk from end gradients folded
 * over the transposed segment maps (HLA page, section 4: the scan form of the
 * chunked recurrence). The call takes a stream-ordered workspace from the library's
 * pool of about B*H*ceil(T/64) * (34 KB + 8*dk*dv + 256*dv bytes) (chunk records,
 * every chunk-start state, every chunk-end state gradient and a 64 x dv block), plus
 * for segmented walks the forward's chunk records (13 KB per chunk) and per head two
 * sets of segment maps and three of segment states, and frees it on the stream.
 * T == 0 copies grad_final_state (or zeros) into grad_init_state.
 */
kla_status kla_chunk_bwd(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k,
                         const void* v, const float* log_alpha, const float* eta, float eps,
                         const float* init_state, const float* grad_out, const float* grad_final_state,
                         float* grad_q, float* grad_k, float* grad_v, float* grad_log_alpha,
                         float* grad_eta, float* grad_init_state, int B, int T, int H, int dk, int dv,
                         int chunk, hipStream_t stream);

/*
 * Host-only planning query: which path and segment count kla_chunk_fwd_ex would
 * use for these sizes and input dtype, and the workspace bytes it would allocate
 * (the per-chunk record is smaller for bf16 with dk <= 128). `num_cus` is the
 * compute-unit count to plan for (0 = ask the current HIP device, 256 if there is
 * none). Makes no allocation and enqueues nothing.
 */
kla_status kla_plan(kla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                    kla_path path, int segments, int num_cus, kla_path* chosen_path,
                    int* chosen_segments, size_t* workspace_bytes);

/*
 * One recurrent decode step for N x H states, updated in place (KLA page,
 * "KLA update rule", one token; the state keeps a constant size per head).
 *   q, k   bf16 [N,H,dk];  v bf16 [N,H,dv]
 *   log_alpha, eta  fp32 [N,H]
 *   state  fp32 [N,H,dk,dv], read and overwritten with S_t
 *   out    fp32 [N,H,dv], o_t = S_t^T q_t
 * Needs no workspace.
 */
kla_status kla_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* eta, float eps, float* state, float* out, int N, int H,
                           int dk, int dv, hipStream_t stream);

/* Same as kla_decode_step with fp32 q, k, v. */
kla_status kla_decode_step_f32(const float* q, const float* k, const float* v,
                               const float* log_alpha, const float* eta, float eps, float* state,
                               float* out, int N, int H, int dk, int dv, hipStream_t stream);

/* kla_decode_step with the input dtype and the write strength chosen by the caller. */
kla_status kla_decode_step_ex(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k,
                              const void* v, const float* log_alpha, const float* eta, float eps,
                              float* state, float* out, int N, int H, int dk, int dv,
                              hipStream_t stream);

/*
 * Log-linear KLA decode: one token at position t for N x H heads, each with L
 * Fenwick-bucketed states (Log-Linear page, "Mathematical formalization",
 * recurrent form: one state per bucket of the prefix, output
 * o_t = sum_l lambda_t^(l) q_t^T S_t^(l); O(log T) work and memory per token).
 * The buckets carry the KLA recurrence: every occupied bucket takes the token's
 * transition S -> exp(log_alpha) (S - beta k (k^T S)), and the buckets sum to the
 * KLA state, so all-ones weights reproduce kla_decode_step_ex.
 * Buckets at position t (0-based): level 0 holds token t; level l >= 1 holds the
 * 2^(l-1) tokens below bit l-1 of t when that bit is set. From t-1 to t, levels
 * 0..j (j = trailing zeros of t) join into level j+1 and the token opens level 0.
 *
 *   q, k, v, log_alpha, eta, eps, dtype, beta_mode   as for kla_decode_step_ex
 *   lam      fp32 [N,H,L]: lambda_t^(l), the weight of level l in the output
 *   states   fp32 [N,H,L,dk,dv], updated in place: the buckets at position t-1 on
 *            entry (zeros, or anything, at t == 0) and at position t on return.
 *            Only occupied levels are read or written (1 + popcount(t-1) in,
 *            1 + popcount(t) out); other slots are left as they are.
 *   out      fp32 [N,H,dv]
 *   levels   L, 1..31; t must satisfy 0 <= t < 2^(L-1), else KLA_ERR_INVALID_ARG
 */
kla_status kla_loglinear_decode_step(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k,
                                     const void* v, const float* log_alpha, const float* eta,
                                     const float* lam, float eps, float* states, float* out, int N, int H,
                                     int dk, int dv, int levels, int t, hipStream_t stream);

/*
 * Log-linear KLA prefill over T tokens from empty buckets (the parallel side of the
 * Log-Linear page's "Mathematical formalization"): for every token,
 *     o_t = sum over s <= t of lambda_t^(level(t,s)) beta_s (q_t^T A_t ... A_{s+1} k_s) v_s
 * with the buckets and transitions of kla_loglinear_decode_step. Work is O(T log T):
 * the pairs inside a 64-token chunk (levels 0..6) from the chunk's pair matrix P T'; the
 * coarser levels l = 7 + s from walks over chunk blocks of 2^s: for bf16 with dk <= 128 one
 * walk per scale over its right half-blocks that carries the KLA state of the enclosing
 * 2^(s+1)-chunk block (weights lambda^(l) - lambda^(next level present) telescope to the
 * definition), otherwise a zero-start walk over every left half-block and a walk over its
 * right sibling from that end state with no values.
 *
 *   q, k, v, log_alpha, eta, eps, dtype, beta_mode, B, T, H, dk, dv, chunk
 *            as for kla_chunk_fwd_ex (the fp32 dtype supports dk in {64, 128})
 *   lam      fp32 [B,T,H,L]: lambda_t^(l)
 *   out      fp32 [B,T,H,dv]
 *   levels   L, 1..31, with T <= 2^(L-1), else KLA_ERR_INVALID_ARG
 * The workspace (the chunk records and the scales' carried end states) comes from the
 * library's workspace pool on `stream`, as for kla_chunk_fwd.
 */
kla_status kla_loglinear_fwd(kla_dtype dtype, kla_beta_mode beta_mode, const void* q, const void* k,
                             const void* v, const float* log_alpha, const float* eta, const float* lam,
                             float eps, float* out, int B, int T, int H, int dk, int dv, int levels,
                             int chunk, hipStream_t stream);

/*
 * Workspace pool. The prefill, log-linear prefill and backward calls take their
 * workspace from a stream-ordered memory pool that the library creates for a
 * device on its first such call there (hipMemPoolCreate, never the device's
 * default pool). Freed workspace stays reserved in that pool for later calls, so
 * a call does not map fresh memory each time; the pool therefore holds as much
 * device memory as the largest concurrent set of calls has needed.
 * kla_workspace_trim() releases every reserved block of the current device's
 * pool that no enqueued call still uses (hipMemPoolTrimTo). Returns KLA_ERR_HIP
 * if the pool cannot be created or trimmed.
 */
kla_status kla_workspace_trim(void);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
const char* kla_last_error(void);

/* Library version string. */
const char* kla_version(void);

/*
 * Measurement hook. While enabled on the calling thread, every kernel the
 * library enqueues from that thread stamps a pair of HIP events from its own
 * dispatch (hipExtLaunchKernelGGL). kla_timing_collect waits for those events,
 * writes up to `max` per-kernel totals (name, launches, summed milliseconds)
 * and clears the record; it returns the number of distinct kernels recorded,
 * or -1 on a HIP error. A kernel's time runs from the later of its start stamp
 * and the end of the previous timed kernel to its end, which assumes the timed
 * launches of a thread share one stream. Off by default.
 */
typedef struct {
  char name[32];
  int launches;
  double total_ms;
} kla_kernel_timing;

kla_status kla_timing_enable(int enable);
int kla_timing_collect(kla_kernel_timing* out, int max);

/*
 * Restricts the hook, on the calling thread, to launches of the kernel named
 * `kernel` (a name as kla_timing_collect reports it, e.g. "kla_state_seq");
 * NULL or "" times every kernel again. Each pair of stamps costs the stream a
 * few microseconds, so a caller that needs one kernel's duration stamps only
 * that one. Returns KLA_ERR_INVALID_ARG for a name of 32 characters or more.
 */
kla_status kla_timing_select(const char* kernel);

#ifdef __cplusplus
}
#endif

#endif /* KLA_H_ */
