// Log-linear KLA: the single-token decode step over Fenwick-bucketed states.
//
// The Log-Linear page ("Mathematical formalization", recurrent form) keeps one state per
// Fenwick bucket of the prefix and reads out o_t = sum_l lambda_t^(l) q_t^T S_t^(l); its
// decoding takes O(log T) time and memory per token. Here the buckets carry the KLA
// recurrence (KLA page, "KLA update rule"): a bucket's state is the part of the KLA state
// that its tokens contributed, so every bucket takes the token's transition
//   A_t S = alpha (S - beta k (k^T S)),   alpha = exp(log_alpha), beta as in kla_decode,
// and the buckets sum to the KLA state.
//
// Buckets at position t (0-based): level 0 holds token t; level l >= 1 holds the 2^(l-1)
// tokens below bit l-1 of t when that bit is set. Going from t-1 to t (t >= 1, j = number
// of trailing zeros of t), levels 0..j of t-1 join into level j+1, higher levels keep their
// tokens, and the new token opens level 0:
//   S^(j+1) <- A_t (S^(0) + ... + S^(j)),   S^(l) <- A_t S^(l) for the other occupied l,
//   S^(0)   <- beta k v^T,
//   o       =  sum over occupied l of lambda^(l) S^(l)^T q
// with S^T q of a transformed bucket equal to alpha (S^T q - beta (k . q) S^T k), so one
// pass over a bucket gives both its new value and its output term. Only occupied levels
// are read or written: 1 + popcount(t-1) buckets in, 1 + popcount(t) out. Slots of levels
// emptied by a merge keep stale values and are never read again before being overwritten.
//
// One workgroup per (sequence, head), each thread owning 4 adjacent columns of a stripe of
// rows of a bucket, as in the KLA decode kernel; bound by HBM bandwidth. A step moves several
// GB of buckets, far more than the last-level cache holds, and a bucket is not touched again
// until a later step, so bucket reads and writes are non-temporal (the `nt` bit): streaming
// past the caches this way moved the same bytes about 7% faster on MI355X.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

// Threads per workgroup: 512 for the larger buckets, so that a thread's two tiles (the bucket
// being finished and the one being loaded) stay small enough for four waves per SIMD.
template <int DK, int DV>
constexpr int ll_threads() { return DK * DV >= 128 * 128 ? 512 : 256; }

template <int MODE, int DK, int DV>
__global__ __launch_bounds__((ll_threads<DK, DV>())) void loglinear_decode_kernel(
    const typename Tr<MODE>::in_t* __restrict__ q, const typename Tr<MODE>::in_t* __restrict__ k,
    const typename Tr<MODE>::in_t* __restrict__ v, const float* __restrict__ log_alpha,
    const float* __restrict__ eta, const float* __restrict__ lam, float eps, int direct,
    float* __restrict__ states, float* __restrict__ out, int L, int t) {
  using TR = Tr<MODE>;
  constexpr int NT = ll_threads<DK, DV>();
  constexpr int NW = NT / 64;     // waves
  constexpr int TPR = DV / 4;     // threads per state row
  constexpr int RPP = NT / TPR;   // rows per pass
  constexpr int NP = DK / RPP;    // rows per thread
  static_assert(DK % RPP == 0 && DK <= NT, "shape");

  __shared__ float sq[DK], sk[DK];
  __shared__ float4 spa[2][RPP][TPR], spb[2][RPP][TPR];  // alternate buckets use alternate halves
  __shared__ float sred[2][NW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rg = tid / TPR, c4 = tid - rg * TPR;
  const size_t nh = blockIdx.x;
  float* S = states + nh * static_cast<size_t>(L) * DK * DV;
  const float* lw = lam + nh * L;
  auto slot = [&](int l) __attribute__((always_inline)) { return S + static_cast<size_t>(l) * DK * DV; };

  float kk = 0.f, kq = 0.f;
  if (tid < DK) {
    const float qq = TR::to_f32(q[nh * DK + tid]);
    const float kv = TR::to_f32(k[nh * DK + tid]);
    sq[tid] = qq;
    sk[tid] = kv;
    kk = kv * kv;
    kq = kv * qq;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kk += __shfl_xor(kk, o);
    kq += __shfl_xor(kq, o);
  }
  if (lane == 0) {
    sred[0][w] = kk;
    sred[1][w] = kq;
  }
  __syncthreads();
  float nk = 0.f, dkq = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    nk += sred[0][i];
    dkq += sred[1][i];
  }
  const float alpha = expf(log_alpha[nh]);
  const float denom = nk + eps;
  const float beta = direct ? eta[nh] : denom != 0.f ? eta[nh] / denom : 0.f;
  const float ab = alpha * beta;

  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  int half = 0;  // the partial-sum buffers of the next bucket

  // One bucket: s holds its state at t-1 (this thread's tile). Applies the transition, writes
  // the result to slot `dest` and adds the bucket's output term with weight lambda^(dest).
  auto finish_bucket = [&](float4 (&s)[NP], int dest) __attribute__((always_inline)) {
    float4 pa = make_float4(0.f, 0.f, 0.f, 0.f), pb = pa;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float kr = sk[rg + p * RPP], qr = sq[rg + p * RPP];
      pa.x += s[p].x * kr; pa.y += s[p].y * kr; pa.z += s[p].z * kr; pa.w += s[p].w * kr;
      pb.x += s[p].x * qr; pb.y += s[p].y * qr; pb.z += s[p].z * qr; pb.w += s[p].w * qr;
    }
    spa[half][rg][c4] = pa;
    spb[half][rg][c4] = pb;
    lds_barrier();
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f), Bq = A;
#pragma unroll
    for (int g = 0; g < RPP; ++g) {
      const float4 x = spa[half][g][c4], y = spb[half][g][c4];
      A.x += x.x; A.y += x.y; A.z += x.z; A.w += x.w;
      Bq.x += y.x; Bq.y += y.y; Bq.z += y.z; Bq.w += y.w;
    }
    // the next bucket writes the other half; the one after it writes this half again only
    // after the next bucket's barrier, which every thread reaches after these reads
    half ^= 1;
    const float lw_d = lw[dest];
    const float bq = beta * dkq;
    o.x += lw_d * alpha * (Bq.x - bq * A.x); o.y += lw_d * alpha * (Bq.y - bq * A.y);
    o.z += lw_d * alpha * (Bq.z - bq * A.z); o.w += lw_d * alpha * (Bq.w - bq * A.w);
    float* D = slot(dest);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float bk = ab * sk[rg + p * RPP];
      float4 x = s[p];
      x.x = alpha * x.x - bk * A.x; x.y = alpha * x.y - bk * A.y;
      x.z = alpha * x.z - bk * A.z; x.w = alpha * x.w - bk * A.w;
      __builtin_nontemporal_store(f32x4{x.x, x.y, x.z, x.w}, reinterpret_cast<f32x4*>(D + static_cast<size_t>(rg + p * RPP) * DV + 4 * c4));
    }
  };
  auto load_set = [&](float4 (&s)[NP], int l) __attribute__((always_inline)) {
    const float* Sl = slot(l);
#pragma unroll
    for (int p = 0; p < NP; ++p)
    {
      const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sl + static_cast<size_t>(rg + p * RPP) * DV + 4 * c4));
      s[p] = make_float4(x[0], x[1], x[2], x[3]);
    }
  };
  auto load_add = [&](float4 (&s)[NP], int l) __attribute__((always_inline)) {
    const float* Sl = slot(l);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sl + static_cast<size_t>(rg + p * RPP) * DV + 4 * c4));
      s[p].x += x[0]; s[p].y += x[1]; s[p].z += x[2]; s[p].w += x[3];
    }
  };

  if (t > 0) {
    // Levels 0..j of t-1 join into level j+1; then the higher occupied levels (the set bits of t
    // above bit j) are transformed in place, one bucket per pass. The next bucket's loads are
    // issued before the current one's reductions, whose barriers wait for LDS only, so a
    // workgroup keeps a bucket of reads in flight while it finishes the previous one.
    const int j = __builtin_ctz(static_cast<unsigned>(t));
    float4 cur[NP], nxt[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) cur[p] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int l = 0; l <= j; ++l) load_add(cur, l);
    int dest = j + 1;
    while (true) {
      const unsigned rest = static_cast<unsigned>(t) >> dest;             // bits of t above bit dest - 1
      const int next = rest ? dest + __builtin_ctz(rest) + 1 : -1;          // level of the lowest of them
      if (next > 0) load_set(nxt, next);  // consumed only after this bucket's barriers
      finish_bucket(cur, dest);
      if (next < 0) break;
      for (int p = 0; p < NP; ++p) cur[p] = nxt[p];  // register renaming once unrolled
      dest = next;
    }
  }

  // the new token opens level 0: S^(0) = beta k v^T, read out as beta (k . q) v
  float vv[4];
#pragma unroll
  for (int jx = 0; jx < 4; ++jx) vv[jx] = TR::to_f32(v[nh * DV + 4 * c4 + jx]);
  float* D0 = slot(0);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const float bk = beta * sk[rg + p * RPP];
    __builtin_nontemporal_store(f32x4{bk * vv[0], bk * vv[1], bk * vv[2], bk * vv[3]},
                                reinterpret_cast<f32x4*>(D0 + static_cast<size_t>(rg + p * RPP) * DV + 4 * c4));
  }
  const float w0 = lw[0] * beta * dkq;
  o.x += w0 * vv[0]; o.y += w0 * vv[1]; o.z += w0 * vv[2]; o.w += w0 * vv[3];
  if (rg == 0) *reinterpret_cast<float4*>(out + nh * DV + 4 * c4) = o;
}

// ---------------------------------------------------------------------------
// Log-linear prefill, levels 0..6: the pairs of tokens inside one 64-token chunk.
//
// From a zero start, the chunk algebra of the KLA prefill gives the chunk's outputs as
// O = P T' V (P and T' from the chunk record), so W = P T' holds the token-pair weights
// W_ts = beta_s q_t^T A_t ... A_{s+1} k_s of the token-pair definition. Two tokens of one
// chunk differ only in their low six bits, so their bucket is level 0 (s = t) or the index of
// their highest differing bit plus one, at most 6:
//   out_t = sum_{s <= t in the chunk} lambda_t^(level(t,s)) W_ts v_s          (written, not added)
// One workgroup per (batch, head, chunk), fp32 on the vector ALU: W = P T' (8 pairs per
// thread), then the weighted W times the chunk's values.
constexpr int INTRA_THREADS = 512;

template <int MODE, int DV>
__global__ __launch_bounds__(INTRA_THREADS) void loglinear_intra_kernel(const uint8_t* __restrict__ rec,
                                                              const typename Tr<MODE>::in_t* __restrict__ v,
                                                              const float* __restrict__ lam, float* __restrict__ out,
                                                              int T, int H, int nc, int L) {
  using TR = Tr<MODE>;
  constexpr int NT = INTRA_THREADS;
  constexpr int SPT = CHUNK * CHUNK / NT;  // pairs of W per thread (8)
  constexpr int G = NT / DV;         // row groups
  constexpr int NR = CHUNK / G;      // rows per thread in the product with V
  constexpr int PT = CHUNK + 4;      // row pitch: 16-byte aligned rows, read four values at a time
  __shared__ __align__(16) float sT[CHUNK][PT];
  __shared__ __align__(16) float sW[CHUNK][PT];  // P, then the weighted W
  __shared__ __align__(16) float sV[CHUNK][DV + 4];

  const int tid = threadIdx.x;
  const int id = blockIdx.x;
  const int bh = id / nc, c = id - bh * nc;
  const int b = bh / H, h = bh - b * H;
  const int t0 = c * CHUNK;
  const uint8_t* R = rec + static_cast<size_t>(id) * REC_BYTES;
  // T' and P rows in 16-byte pieces: a thread takes (row, block of 8 columns) and, in bf16 mode,
  // the hi and the lo piece of that block (pieces are swizzled within their row)
#pragma unroll
  for (int u = 0; u < 512 / NT; ++u) {
    const int e = tid + NT * u;  // 512 (row, block) pairs
    const int r = e >> 3, cb = e & 7;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint8_t* base = R + (m == 0 ? REC_T_OFF : REC_P_OFF);
      float* dst = m == 0 ? &sT[r][8 * cb] : &sW[r][8 * cb];
      if constexpr (MODE == MODE_BF16) {
        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + swz_off<256>(r, 16 * cb));
        const u32x4 lo = *reinterpret_cast<const u32x4*>(base + swz_off<256>(r, 16 * (cb + 8)));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dst[2 * j] = __uint_as_float(hi[j] << 16) + __uint_as_float(lo[j] << 16);
          dst[2 * j + 1] = __uint_as_float(hi[j] & 0xFFFF0000u) + __uint_as_float(lo[j] & 0xFFFF0000u);
        }
      } else {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(base + swz_off<256>(r, 32 * cb));
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(base + swz_off<256>(r, 32 * cb + 16));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dst[j] = x0[j];
          dst[4 + j] = x1[j];
        }
      }
    }
  }
  // the chunk's value rows in 16-byte pieces
  constexpr int VE = 16 / static_cast<int>(sizeof(typename TR::in_t));  // values per piece
  constexpr int VP = DV / VE;                                            // pieces per row
  for (int e = tid; e < CHUNK * VP; e += NT) {
    const int sr = e / VP, pc = e - sr * VP;
    const int t = t0 + sr;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (t < T) x = *reinterpret_cast<const u32x4*>(v + (static_cast<size_t>(b) * T + t) * H * DV + h * DV + VE * pc);
    if constexpr (MODE == MODE_BF16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sV[sr][8 * pc + 2 * j] = __uint_as_float(x[j] << 16);
        sV[sr][8 * pc + 2 * j + 1] = __uint_as_float(x[j] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) sV[sr][4 * pc + j] = __uint_as_float(x[j]);
    }
  }
  __syncthreads();

  // W_ts = sum_r P_tr T'_rs for row t and columns s0 .. s0 + SPT - 1 (both factors are lower triangular)
  const int t = tid / (CHUNK / SPT), s0 = (tid % (CHUNK / SPT)) * SPT;
  float w[SPT];
#pragma unroll
  for (int j = 0; j < SPT; ++j) w[j] = 0.f;
  for (int r = 0; r < CHUNK; ++r) {
    const float p = sW[t][r];
#pragma unroll
    for (int j4 = 0; j4 < SPT / 4; ++j4) {
      const float4 tr = *reinterpret_cast<const float4*>(&sT[r][s0 + 4 * j4]);
      w[4 * j4] += p * tr.x;
      w[4 * j4 + 1] += p * tr.y;
      w[4 * j4 + 2] += p * tr.z;
      w[4 * j4 + 3] += p * tr.w;
    }
  }
  const bool live = t0 + t < T;
  const float* lw = lam + ((static_cast<size_t>(b) * T + t0 + t) * H + h) * L;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    const int s = s0 + j;
    const int lev = s == t ? 0 : 32 - __clz(static_cast<unsigned>(t ^ s));
    w[j] = (live && s <= t) ? w[j] * lw[lev] : 0.f;
  }
  __syncthreads();  // every read of P is done
#pragma unroll
  for (int j = 0; j < SPT; ++j) sW[t][s0 + j] = w[j];
  __syncthreads();

  // out_t = sum_s W_ts v_s for this thread's column cc and rows g, g + G, ...
  const int g = tid / DV, cc = tid - g * DV;
  float acc[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i] = 0.f;
  // full unrolling of this loop hoists every row's LDS reads at DV = 64 (and spills), so unroll it
  // only where that keeps the registers low
  constexpr int UNR = DV >= 128 ? 4 : 2;
#pragma unroll UNR
  for (int s = 0; s < CHUNK; s += 4) {
    const float v0 = sV[s][cc], v1 = sV[s + 1][cc], v2 = sV[s + 2][cc], v3 = sV[s + 3][cc];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float4 wr = *reinterpret_cast<const float4*>(&sW[g + G * i][s]);
      acc[i] += wr.x * v0 + wr.y * v1 + wr.z * v2 + wr.w * v3;
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int tt = t0 + g + G * i;
    if (tt < T) out[(static_cast<size_t>(b) * T + tt) * H * DV + h * DV + cc] = acc[i];
  }
}

// The same for bf16 inputs on the bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation), one
// workgroup per (batch, head, chunk), eight waves:
//   W = P T' from the record's hi and lo halves, three passes (hi hi, hi lo, lo hi), wave w on row
//   tile w % 4 and column tiles w / 4 + {0, 2}; W is lower triangular, so tiles above the
//   diagonal are zero and the contraction runs only over the tokens between the two tiles;
//   the weighted W (row t, column s scaled by lambda_t^(level(t,s)), zero above the diagonal and
//   past T) into LDS in fp32;
//   out = W V with W as hi + lo bf16 pairs and V exact, two passes.
// P's rows enter straight from the record as A operands (eight consecutive columns per lane);
// T'^T and V^T are staged transposed in LDS, so each B operand is one 16-byte read.
template <int DV>
__global__ __launch_bounds__(INTRA_THREADS) void loglinear_intra_mfma_kernel(const uint8_t* __restrict__ rec,
                                                                   const uint16_t* __restrict__ v,
                                                                   const float* __restrict__ lam,
                                                                   float* __restrict__ out, int T, int H, int nc,
                                                                   int L) {
  constexpr int BP = CHUNK + 8;  // bf16 pitch of the transposed rows (16-byte aligned)
  constexpr int WP = CHUNK + 4;  // fp32 pitch of W
  __shared__ __align__(16) uint16_t sTh[CHUNK][BP];  // T'^T, hi and lo
  __shared__ __align__(16) uint16_t sTl[CHUNK][BP];
  __shared__ __align__(16) uint16_t sVt[DV][BP];     // V^T
  __shared__ __align__(16) float sW[CHUNK][WP];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, gq = lane >> 4, ln = lane & 15;
  const int id = blockIdx.x;
  const int bh = id / nc, c = id - bh * nc;
  const int b = bh / H, h = bh - b * H;
  const int t0 = c * CHUNK;
  const uint8_t* R = rec + static_cast<size_t>(id) * REC_BYTES;
  const int mt = wv & 3;

  // P's rows for this wave's row tile (A operands), loaded first: row 16 mt + ln, columns
  // 32 kb + 8 gq + 0..7, hi and lo
  u32x4 ph[2], pl[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    ph[kb] = *reinterpret_cast<const u32x4*>(R + REC_P_OFF + swz_off<256>(16 * mt + ln, 16 * (4 * kb + gq)));
    pl[kb] = *reinterpret_cast<const u32x4*>(R + REC_P_OFF + swz_off<256>(16 * mt + ln, 16 * (4 * kb + gq + 8)));
  }
  // T' transposed: consecutive lanes take consecutive rows r, so the transposed writes hit
  // consecutive halves of LDS words
  {
    const int r = tid & 63, cb = tid >> 6;  // 64 rows x 8 blocks of 8 columns
    const u32x4 hi = *reinterpret_cast<const u32x4*>(R + REC_T_OFF + swz_off<256>(r, 16 * cb));
    const u32x4 lo = *reinterpret_cast<const u32x4*>(R + REC_T_OFF + swz_off<256>(r, 16 * (cb + 8)));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sTh[8 * cb + j][r] = static_cast<uint16_t>((j & 1) ? hi[j >> 1] >> 16 : hi[j >> 1] & 0xFFFFu);
      sTl[8 * cb + j][r] = static_cast<uint16_t>((j & 1) ? lo[j >> 1] >> 16 : lo[j >> 1] & 0xFFFFu);
    }
  }
  // V transposed, zero past T
#pragma unroll
  for (int u = 0; u < CHUNK * DV / 8 / INTRA_THREADS; ++u) {
    const int e = tid + INTRA_THREADS * u, tt = e & 63, pc = e >> 6;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (t0 + tt < T) x = *reinterpret_cast<const u32x4*>(v + (static_cast<size_t>(b) * T + t0 + tt) * H * DV + h * DV + 8 * pc);
#pragma unroll
    for (int j = 0; j < 8; ++j) sVt[8 * pc + j][tt] = static_cast<uint16_t>((j & 1) ? x[j >> 1] >> 16 : x[j >> 1] & 0xFFFFu);
  }
  __syncthreads();

  // W = P T' on tiles (mt, nt), nt = wv / 4 + 2 u; the contraction over r needs only
  // 16 nt <= r <= 16 mt + 15
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int nt = (wv >> 2) + 2 * u;
    f32x4 acc = zero4();
    if (nt <= mt) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (32 * kb > 16 * mt + 15 || 32 * kb + 31 < 16 * nt) continue;
        const bf16x8 th = *reinterpret_cast<const bf16x8*>(&sTh[16 * nt + ln][32 * kb + 8 * gq]);
        const bf16x8 tl = *reinterpret_cast<const bf16x8*>(&sTl[16 * nt + ln][32 * kb + 8 * gq]);
        const bf16x8 a_h = __builtin_bit_cast(bf16x8, ph[kb]), a_l = __builtin_bit_cast(bf16x8, pl[kb]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_h, th, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_h, tl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_l, th, acc, 0, 0, 0);
      }
    }
    // weights: row t = 16 mt + 4 gq + e, column s = 16 nt + ln
    const int s = 16 * nt + ln;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * mt + 4 * gq + e;
      float wgt = 0.f;
      if (s <= t && t0 + t < T) {
        const int lev = s == t ? 0 : 32 - __clz(static_cast<unsigned>(t ^ s));
        wgt = acc[e] * lam[((static_cast<size_t>(b) * T + t0 + t) * H + h) * L + lev];
      }
      sW[t][s] = wgt;
    }
  }
  __syncthreads();

  // out = W V on tiles (mt, nt), nt = wv / 4 + 2 u; W is zero for s > t, so row tiles 0 and 1
  // need only the first 32 tokens
#pragma unroll
  for (int u = 0; u < DV / 32; ++u) {
    const int nt = (wv >> 2) + 2 * u;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb == 1 && mt < 2) continue;
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&sW[16 * mt + ln][32 * kb + 8 * gq]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&sW[16 * mt + ln][32 * kb + 8 * gq + 4]);
      F8 wf;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wf.v[j] = w0[j];
        wf.v[4 + j] = w1[j];
      }
      const S8 ws = split8(wf);
      const bf16x8 vb = *reinterpret_cast<const bf16x8*>(&sVt[16 * nt + ln][32 * kb + 8 * gq]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ws.h, vb, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ws.l, vb, acc, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tt = t0 + 16 * mt + 4 * gq + e;
      if (tt < T) out[(static_cast<size_t>(b) * T + tt) * H * DV + h * DV + 16 * nt + ln] = acc[e];
    }
  }
}

// The same on the compact record (T' without its zero quadrant, and the gates), which the walks
// read anyway, so that no full record is prepared. A persistent, DMA-fed kernel: each workgroup
// takes chunks blockIdx.x, blockIdx.x + gridDim.x, ... of all heads; a copy wave brings chunk
// n + 1's rows of Q, K and V, its record and its weights into the other half of a
// double-buffered LDS area (buffer_load ... lds, rows in the swizzled layout of kla_device.h)
// while four compute waves work on chunk n, in three steps between workgroup barriers:
//  1. P = tril(e^{g_t - g_r} Q K^T) on the bf16 MFMA (exact products), three 16 x 16 tiles per
//     wave, split hi + lo into LDS in the record's layout (as the walk's output waves do);
//  2. W = P T' on the 12 tiles on or below the diagonal (four tile-contractions per wave), computed
//     transposed, W^T = T'^T P^T: T'^T from the record by transposed LDS reads
//     (ds_read_b64_tr_b16), P^T as P's row fragments, P and T' both split (three passes); each
//     pair weighted in place by lambda_t^(lev(t, s)) less lambda_t^(7 + lowest set bit of c) on
//     chunk c >= 1 (lev = bit length of t xor s within the chunk; see the scale walks of
//     state_walk_kernel, whose outputs on chunk c carry the chunk-local term with that weight),
//     then split hi + lo into LDS, rows t;
//  3. out = W V, written transposed as the walks' outputs are (16 columns x 16 tokens per tile,
//     one 16-byte store per lane and tile): V^T from V's rows by transposed reads, W as row
//     fragments; two passes (V is exact). Each wave takes DV / 64 column slices of 16.
// Rows t of every 64-row tile are in the permuted order tok(m, r) of the walks, so that the
// accumulator pair and fragment conventions are the same.
namespace {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

__device__ __forceinline__ int tok_r(int m, int r) { return 32 * (m >> 1) + 8 * (r >> 2) + 4 * (m & 1) + (r & 3); }

__device__ __forceinline__ void dma16_l(rsrc_t r, void* lds_dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4_l(rsrc_t r, void* lds_dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_dst, 4, voff, 0, 0, 0);
}

}  // namespace

constexpr int INTRA_DMA_THREADS = 320;  // four compute waves and the copy wave

template <int DK, int DV>
__global__ __launch_bounds__(INTRA_DMA_THREADS) void loglinear_intra_compact_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint8_t* __restrict__ crec,
    const uint16_t* __restrict__ v, const float* __restrict__ lam, float* __restrict__ out, int T, int H, int nc,
    int L, int nchunk_all) {
  using TR = Tr<MODE_BF16>;
  constexpr int KRB = DK * 2, VRB = DV * 2;            // bytes of a key/query row and a value row
  constexpr int KBYTES = CHUNK * KRB, VBYTES = CHUNK * VRB;
  constexpr int K_OFF = 0, Q_OFF = KBYTES, V_OFF = 2 * KBYTES, R_OFF = V_OFF + VBYTES;
  constexpr int L_OFF = R_OFF + CREC_BYTES;            // weights [8][64] fp32: levels 0..6, the subtracted one
  constexpr int BUF = L_OFF + 8 * CHUNK * 4;
  constexpr int KPR = KRB / 16, KRPB = 1024 / KRB, VPR = VRB / 16, VRPB = 1024 / VRB;
  constexpr int NSL = DV / 64;                         // 16-column slices per compute wave
  static_assert(BUF % 256 == 0 && R_OFF % 256 == 0, "buffers and records on the 256-byte bank period");
  __shared__ __align__(256) uint8_t lds0[BUF];
  __shared__ __align__(256) uint8_t lds1[BUF];
  __shared__ __align__(256) uint8_t ldsP[CREC_EG_OFF];  // P, hi and lo, in the record's layout
  __shared__ __align__(256) uint8_t ldsW[CREC_EG_OFF];  // weighted W, likewise

  const int tid = threadIdx.x, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, ln = lane & 15;
  const int first = blockIdx.x, step = gridDim.x;
  const int nmine = first < nchunk_all ? (nchunk_all - 1 - first) / step + 1 : 0;

  if (wu == 4) {  // the copy wave
    auto copy_chunk = [&](int n, uint8_t* B) __attribute__((always_inline)) {
      const int bh = n / nc, c = n - bh * nc;
      const int b = bh / H, h = bh - b * H;
      const int t0 = c * CHUNK;
      const rsrc_t rr = make_rsrc_wu(crec + static_cast<size_t>(n) * CREC_BYTES, CREC_BYTES);
#pragma unroll
      for (int m = 0; m < CREC_BYTES / 1024; ++m) dma16_l(rr, B + R_OFF + 1024 * m, 1024 * m + 16 * lane);
      if (lane < (CREC_BYTES % 1024) / 16)
        dma16_l(rr, B + R_OFF + (CREC_BYTES / 1024) * 1024, (CREC_BYTES / 1024) * 1024 + 16 * lane);
      const size_t row0 = (static_cast<size_t>(b) * T + t0) * H + h;  // token-head row of token t0
      const long long left = T - t0;
      const rsrc_t rk = make_rsrc_wu(k + row0 * DK, left * H * KRB - static_cast<long long>(h) * KRB);
      const rsrc_t rq = make_rsrc_wu(q + row0 * DK, left * H * KRB - static_cast<long long>(h) * KRB);
      const rsrc_t rv = make_rsrc_wu(v + row0 * DV, left * H * VRB - static_cast<long long>(h) * VRB);
#pragma unroll
      for (int blk = 0; blk < KBYTES / 1024; ++blk) {
        const int row = blk * KRPB + lane / KPR;
        const int off = row * H * KRB + 16 * ((lane % KPR) ^ swz<KRB>(row));
        dma16_l(rk, B + K_OFF + 1024 * blk, off);
        dma16_l(rq, B + Q_OFF + 1024 * blk, off);
      }
#pragma unroll
      for (int blk = 0; blk < VBYTES / 1024; ++blk) {
        const int row = blk * VRPB + lane / VPR;
        dma16_l(rv, B + V_OFF + 1024 * blk, row * H * VRB + 16 * ((lane % VPR) ^ swz<VRB>(row)));
      }
      // weights of levels 0..6 and of 7 + (lowest set bit of c), one dword per lane and level
      const int HL = H * L;
      const rsrc_t rl = make_rsrc_wu(lam + row0 * L, (left - 1) * HL * 4 + static_cast<long long>(L) * 4);
      const int low = c > 0 ? 7 + __builtin_ctz(static_cast<unsigned>(c)) : 0;
#pragma unroll
      for (int l = 0; l < 7; ++l) dma4_l(rl, B + L_OFF + 256 * l, (lane * HL + l) * 4);
      dma4_l(rl, B + L_OFF + 256 * 7, (lane * HL + low) * 4);
    };
    if (nmine > 0) copy_chunk(first, lds0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    for (int j = 0; j < nmine; ++j) {
      if (j + 1 < nmine) copy_chunk(first + (j + 1) * step, ((j + 1) & 1) ? lds1 : lds0);
      asm volatile("s_barrier\n\ts_barrier" ::: "memory");  // the P and the W barriers
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    return;
  }

  // compute waves 0..3
  const int w = wu;
  int oK[DK / 32], oRt[2], oRb[2][2];
#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb) oK[kb] = swz_off<KRB>(tok_r(0, ln), 64 * kb + 16 * gq);
#pragma unroll
  for (int hl = 0; hl < 2; ++hl) {
    oRt[hl] = CREC_TOP_OFF + swz_off<128>(tok_r(0, ln), 64 * hl + 16 * gq);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) oRb[kb][hl] = CREC_BOT_OFF + swz_off<256>(tok_r(0, ln), 128 * hl + 64 * kb + 16 * gq);
  }
  auto mrow = [](int m) { return 32 * (m >> 1) + 4 * (m & 1); };
  auto fragK = [&](const uint8_t* X, int m, int kb) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(X + oK[kb] + mrow(m) * KRB));
  };
  // hi and lo of row tok(m, ln) of a lower-triangular matrix in the record's layout, columns
  // 32 kb + 8 gq + 0..7 (kb = 0 when m < 2)
  auto fragR = [&](const uint8_t* X, int m, int kb) __attribute__((always_inline)) {
    const uint8_t* p = m < 2 ? X + oRt[0] + 4 * (m & 1) * 128 : X + oRb[kb][0] + 4 * (m & 1) * 256;
    const int lo = m < 2 ? oRt[1] - oRt[0] : oRb[kb][1] - oRb[kb][0];
    S8 r;
    r.h = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
    r.l = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p + lo));
    return r;
  };
  // T'^T operand: lane (gq, ln) receives T'[32 kb + 8 gq + j][16 nt + ln], j = 0..7, hi and lo
  // (ds_read_b64_tr_b16: it supplies the 8-byte block of row 32 kb + 8 gq + 4 hf + (ln >> 2),
  // columns 16 nt + 4 (ln & 3) + 0..3; kb = 0 only with nt < 2, the top rows' columns)
  auto fragTT = [&](const uint8_t* X, int nt, int kb) __attribute__((always_inline)) {
    const int cb = 2 * (16 * nt + 4 * (ln & 3));
    i16x4 hv[2], lv[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int row = 32 * kb + 8 * gq + 4 * hf + (ln >> 2);
      const int oh = kb == 0 ? CREC_TOP_OFF + swz_off<128>(row, cb) : CREC_BOT_OFF + swz_off<256>(row - 32, cb);
      const int ol = kb == 0 ? CREC_TOP_OFF + swz_off<128>(row, 64 + cb) : CREC_BOT_OFF + swz_off<256>(row - 32, 128 + cb);
      hv[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(X + oh));
      lv[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(X + ol));
    }
    S8 r;
    r.h = __builtin_bit_cast(bf16x8, __builtin_shufflevector(hv[0], hv[1], 0, 1, 2, 3, 4, 5, 6, 7));
    r.l = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lv[0], lv[1], 0, 1, 2, 3, 4, 5, 6, 7));
    return r;
  };
  // V^T operand: lane (gq, ln) receives V[32 a + 8 gq + j][16 cs + ln], j = 0..7
  auto fragVT = [&](const uint8_t* X, int cs, int a) __attribute__((always_inline)) {
    const uint8_t* p = X + swz_off<VRB>(8 * gq + (ln >> 2), 2 * (16 * cs + 4 * (ln & 3))) + 32 * a * VRB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * VRB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // this wave's W tiles (m_t, nt): four tile-contractions each
  constexpr int WT[4][4][2] = {{{2, 0}, {2, 1}, {-1, 0}, {-1, 0}},
                               {{3, 0}, {3, 1}, {-1, 0}, {-1, 0}},
                               {{0, 0}, {0, 1}, {2, 2}, {2, 3}},
                               {{1, 0}, {1, 1}, {3, 2}, {3, 3}}};

  asm volatile("s_barrier" ::: "memory");  // the first chunk has landed
  for (int j = 0; j < nmine; ++j) {
    const int n = first + j * step;
    const int bh = n / nc, c = n - bh * nc;
    const int b = bh / H, h = bh - b * H;
    const int t0 = c * CHUNK;
    const uint8_t* B = (j & 1) ? lds1 : lds0;
    const uint8_t* sK = B + K_OFF;
    const uint8_t* sQ = B + Q_OFF;
    const uint8_t* sV = B + V_OFF;
    const uint8_t* sR = B + R_OFF;
    const float* sL = reinterpret_cast<const float*>(B + L_OFF);
    const float* sG = reinterpret_cast<const float*>(sR + CREC_G_OFF);
    // 1. this wave's three P tiles (rows r of tile mj, columns i of tile mi, i <= r)
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) {
      const int mi = (w >> 1) + (jj == 2 ? 2 : 0), mj = (w & 1) + (jj >= 1 ? 2 : 0);
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) acc = mfma_bf16(fragK(sK, mi, kb), fragK(sQ, mj, kb), acc);
      const int r = tok_r(mj, ln), i0 = tok_r(mi, 4 * gq);
      const float gr = sG[r];
      const f32x4 gi = *reinterpret_cast<const f32x4*>(sG + i0);
      f32x4 pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = __expf(gr - gi[e]) * acc[e];
        pv[e] = (jj == 1 || i0 + e <= r) ? x : 0.f;
      }
      const u32x2 hw = __builtin_bit_cast(u32x2, __builtin_convertvector(pv, bf16x4));
      f32x4 hf;
      hf[0] = __uint_as_float(hw[0] << 16);
      hf[1] = __uint_as_float(hw[0] & 0xFFFF0000u);
      hf[2] = __uint_as_float(hw[1] << 16);
      hf[3] = __uint_as_float(hw[1] & 0xFFFF0000u);
      const u32x2 lw = __builtin_bit_cast(u32x2, __builtin_convertvector(pv - hf, bf16x4));
      const int oh = jj == 0 ? CREC_TOP_OFF + swz_off<128>(r, 2 * i0) : CREC_BOT_OFF + swz_off<256>(r - 32, 2 * i0);
      const int ol = jj == 0 ? CREC_TOP_OFF + swz_off<128>(r, 64 + 2 * i0)
                             : CREC_BOT_OFF + swz_off<256>(r - 32, 128 + 2 * i0);
      *reinterpret_cast<u32x2*>(ldsP + oh) = hw;
      *reinterpret_cast<u32x2*>(ldsP + ol) = lw;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // 2. W^T tiles: rows s = 16 nt + 4 gq + e, columns t = tok(m_t, ln); contraction over
    // i in [s, t]: i < 32 when s < 32, i >= 32 when t >= 32
    const float sub_on = c > 0 ? 1.f : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int mt = WT[w][u][0], nt = WT[w][u][1];
      if (mt < 0) continue;
      f32x4 x = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if ((kb == 0 && nt >= 2) || (kb == 1 && mt < 2)) continue;
        x = TR::mma_dd(x, fragTT(sR, nt, kb), fragR(ldsP, mt, kb));
      }
      const int t = tok_r(mt, ln);
      const float sub = sub_on * sL[7 * CHUNK + t];
      f32x4 xw;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 16 * nt + 4 * gq + e;
        const int lev = 32 - __clz(t ^ s);  // 0 when s == t
        xw[e] = s <= t ? x[e] * (sL[(lev > 6 ? 6 : lev) * CHUNK + t] - sub) : 0.f;
      }
      const u32x2 hw = __builtin_bit_cast(u32x2, __builtin_convertvector(xw, bf16x4));
      f32x4 hf;
      hf[0] = __uint_as_float(hw[0] << 16);
      hf[1] = __uint_as_float(hw[0] & 0xFFFF0000u);
      hf[2] = __uint_as_float(hw[1] << 16);
      hf[3] = __uint_as_float(hw[1] & 0xFFFF0000u);
      const u32x2 lw = __builtin_bit_cast(u32x2, __builtin_convertvector(xw - hf, bf16x4));
      const int col = 2 * (16 * nt + 4 * gq);
      const int oh = t < 32 ? CREC_TOP_OFF + swz_off<128>(t, col) : CREC_BOT_OFF + swz_off<256>(t - 32, col);
      const int ol = t < 32 ? CREC_TOP_OFF + swz_off<128>(t, 64 + col) : CREC_BOT_OFF + swz_off<256>(t - 32, 128 + col);
      *reinterpret_cast<u32x2*>(ldsW + oh) = hw;
      *reinterpret_cast<u32x2*>(ldsW + ol) = lw;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // 3. out = W V on this wave's column slices, stored transposed (rows: 4 columns per lane)
    const rsrc_t ro = make_rsrc_wu(out + ((static_cast<size_t>(b) * T + t0) * H + h) * DV,
                                   (static_cast<long long>(T - t0) * H - h) * DV * 4);
#pragma unroll
    for (int u = 0; u < NSL; ++u) {
      const int cs = w * NSL + u;
      const bf16x8 va0 = fragVT(sV, cs, 0);
      const bf16x8 va1 = fragVT(sV, cs, 1);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc = TR::mma_xd(zero4(), va0, fragR(ldsW, mt, 0));
        if (mt >= 2) acc = TR::mma_xd(acc, va1, fragR(ldsW, mt, 1));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), ro,
                                               (tok_r(mt, ln) * H * DV + 16 * cs + 4 * gq) * 4, 0, 0);
      }
    }
    // past the end barrier, P and W may be overwritten, and the next chunk has landed
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

hipError_t launch_loglinear_intra_compact(const Dims& d, const void* q, const void* k, const uint8_t* crec,
                                          const void* v, const float* lam, int L, float* out, hipStream_t stream) {
  const int nchunk = d.B * d.H * d.nc;
  if (nchunk == 0) return hipSuccess;
  const dim3 grid(nchunk < 256 ? nchunk : 256), block(INTRA_DMA_THREADS);
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kb = static_cast<const uint16_t*>(k);
  const auto* vb = static_cast<const uint16_t*>(v);
#define KLA_LLI_CASE(DKV, DVV)                                                                                   \
  if (d.dk == DKV && d.dv == DVV)                                                                                \
    return launch_kernel(loglinear_intra_compact_kernel<DKV, DVV>, grid, block, stream, qb, kb, crec, vb, lam, out, \
                         d.T, d.H, d.nc, L, nchunk);
  KLA_LLI_CASE(64, 64)
  KLA_LLI_CASE(64, 128)
  KLA_LLI_CASE(128, 64)
  KLA_LLI_CASE(128, 128)
#undef KLA_LLI_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_loglinear_intra(int mode, const Dims& d, const uint8_t* rec, const void* v, const float* lam,
                                  int L, float* out, hipStream_t stream) {
  const dim3 grid(d.B * d.H * d.nc);
  if (mode == MODE_BF16) {
    const auto* vb = static_cast<const uint16_t*>(v);
    if (d.dv == 64) return launch_kernel(loglinear_intra_mfma_kernel<64>, grid, dim3(INTRA_THREADS), stream, rec, vb, lam, out, d.T, d.H, d.nc, L);
    if (d.dv == 128) return launch_kernel(loglinear_intra_mfma_kernel<128>, grid, dim3(INTRA_THREADS), stream, rec, vb, lam, out, d.T, d.H, d.nc, L);
  } else {
    const auto* vf = static_cast<const Tr<MODE_F32>::in_t*>(v);
    if (d.dv == 64) return launch_kernel(loglinear_intra_kernel<MODE_F32, 64>, grid, dim3(INTRA_THREADS), stream, rec, vf, lam, out, d.T, d.H, d.nc, L);
    if (d.dv == 128) return launch_kernel(loglinear_intra_kernel<MODE_F32, 128>, grid, dim3(INTRA_THREADS), stream, rec, vf, lam, out, d.T, d.H, d.nc, L);
  }
  return hipErrorInvalidValue;
}

template <int MODE, int DK, int DV>
static hipError_t launch_ll_t(int N, int H, const void* q, const void* k, const void* v, const float* la,
                              const float* eta, const float* lam, float eps, int direct, float* states, float* out,
                              int L, int t, hipStream_t stream) {
  using in_t = typename Tr<MODE>::in_t;
  return launch_kernel(loglinear_decode_kernel<MODE, DK, DV>, dim3(N * H), dim3(ll_threads<DK, DV>()), stream,
                       static_cast<const in_t*>(q), static_cast<const in_t*>(k), static_cast<const in_t*>(v), la, eta,
                       lam, eps, direct, states, out, L, t);
}

template <int MODE>
static hipError_t dispatch_ll(int N, int H, int dk, int dv, const void* q, const void* k, const void* v,
                              const float* la, const float* eta, const float* lam, float eps, int direct,
                              float* states, float* out, int L, int t, hipStream_t stream) {
#define KLA_LL_CASE(DKV, DVV)                                                                              \
  if (dk == DKV && dv == DVV)                                                                              \
    return launch_ll_t<MODE, DKV, DVV>(N, H, q, k, v, la, eta, lam, eps, direct, states, out, L, t, stream);
  KLA_LL_CASE(64, 64)
  KLA_LL_CASE(64, 128)
  KLA_LL_CASE(128, 64)
  KLA_LL_CASE(128, 128)
  KLA_LL_CASE(256, 64)
  KLA_LL_CASE(256, 128)
#undef KLA_LL_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_loglinear_decode(int mode, int N, int H, int dk, int dv, const void* q, const void* k,
                                   const void* v, const float* log_alpha, const float* eta, const float* lam,
                                   float eps, int direct, float* states, float* out, int L, int t,
                                   hipStream_t stream) {
  if (mode == MODE_BF16)
    return dispatch_ll<MODE_BF16>(N, H, dk, dv, q, k, v, log_alpha, eta, lam, eps, direct, states, out, L, t, stream);
  return dispatch_ll<MODE_F32>(N, H, dk, dv, q, k, v, log_alpha, eta, lam, eps, direct, states, out, L, t, stream);
}

}  // namespace kla
