// Chunkwise backward of the KLA prefill (gradients for training) in fp32 arithmetic: the fp32
// MFMA (v_mfma_f32_16x16x4_f32, full fp32 products and accumulation) and the vector ALU. For
// bf16 inputs, products whose one operand is a bf16 input run on the bf16 MFMA: exactly when
// both operands are inputs (Q K^T, K K^T), and with the fp32 operand as a hi + lo bf16 pair
// (about 2^-17 of its size kept) in the gradients kernel's K S0, K dS1 and Q S0.
//
// The forward of one 64-token chunk with start state S0 (UT form of the delta rule, the
// chunkwise parallel algorithm that the KLA page trains with; KLA page, "Implementation"):
//   g  = cumsum(log_alpha) inside the chunk,  Dl[r][i] = e^{g_r - g_i},  w = e^{g_C - g}
//   A  = strict_lower(beta_r Dl[r][i] (k_r . k_i)),  Minv = (I + A)^-1,  T' = Minv diag(beta)
//   X  = V - e^g . (K S0),   U = T' X,   P = tril_incl(Dl . Q K^T)
//   O  = e^g . (Q S0) + P U,   S1 = e^{g_C} S0 + K^T (w . U)
// Reverse mode through these products runs in five kernels:
//   prep     per chunk: g, beta, ||k||^2 + eps, Minv, and P with K K^T in one matrix
//   states   forward walk over chunks per 16-column block of the state: every chunk-start S0
//   dprep    per chunk: the terms of the reverse walk that do not depend on the carried
//            gradient, P^T dO and Q^T (e^g . dO)
//   dstates  reverse walk per 16-column block: every chunk-end gradient dS1, from
//              dS0 = e^{g_C} dS1 + Q^T (e^g . dO) - K^T (e^g . dX),
//              dX  = diag(beta) Minv^T dU,  dU = w . (K dS1) + P^T dO
//   grads    per chunk, from S0 and dS1: dq, dk, dv, dlog_alpha, deta (the chunk-local
//            products of the reverse pass, then a reverse cumulative sum of dg inside the chunk)
// The columns of the state (the dv index) are independent in both walks, so a walk
// workgroup owns 16 columns. Walk and grads workgroups have 512 threads, 8 per chunk row. A
// ragged last chunk is padded with identity steps (k = q = v = 0, log_alpha = 0, eta = 0),
// which changes neither outputs nor gradients.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kla_launch.h"

namespace kla {
namespace {

constexpr int BC = 64;    // chunk length
constexpr int BT = 256;   // threads of a prep workgroup
constexpr int NT = 512;   // threads of a walk or grads workgroup: 8 per chunk row
constexpr int TPRW = NT / 64, CPT = 16 / TPRW, IPT = 64 / TPRW;  // per row: threads, columns, row entries
constexpr int MP = 65;    // LDS pitch of 64 x 64 matrices
constexpr int NJ = 16;    // state columns per walk workgroup / per grads column block
// chunk record: Minv [64][64], PG [64][64] (lower incl: P; strict upper: K K^T), g, beta, den
constexpr int REC_M = 0, REC_PG = BC * BC, REC_G = 2 * BC * BC, REC_B = REC_G + BC, REC_D = REC_B + BC;
constexpr int RECF = REC_D + 2 * BC;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Eight fp32 values that are bf16 numbers (bf16 inputs widened in LDS) as a bf16 MFMA operand:
// the upper halves, exactly.
__device__ __forceinline__ bf16x8_t bf16_exact8(const float* p) {
  const v4f a = *reinterpret_cast<const v4f*>(p), b = *reinterpret_cast<const v4f*>(p + 4);
  u32x4_t w;
  w[0] = (__float_as_uint(a[1]) & 0xFFFF0000u) | (__float_as_uint(a[0]) >> 16);
  w[1] = (__float_as_uint(a[3]) & 0xFFFF0000u) | (__float_as_uint(a[2]) >> 16);
  w[2] = (__float_as_uint(b[1]) & 0xFFFF0000u) | (__float_as_uint(b[0]) >> 16);
  w[3] = (__float_as_uint(b[3]) & 0xFFFF0000u) | (__float_as_uint(b[2]) >> 16);
  return __builtin_bit_cast(bf16x8_t, w);
}

// Eight fp32 values as hi + lo bf16 operands: hi rounded to nearest even, lo the same rounding of
// the exact residual x - hi, so hi + lo carries x to about 2^-17 of its size.
__device__ __forceinline__ void bf16_split8(const v4f& a, const v4f& b, bf16x8_t& hi, bf16x8_t& lo) {
  const f32x8_t x = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  hi = __builtin_convertvector(x, bf16x8_t);
  const u32x4_t hw = __builtin_bit_cast(u32x4_t, hi);
  f32x8_t hf;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    hf[2 * m] = __uint_as_float(hw[m] << 16);
    hf[2 * m + 1] = __uint_as_float(hw[m] & 0xFFFF0000u);
  }
  lo = __builtin_convertvector(x - hf, bf16x8_t);
}
__device__ __forceinline__ void bf16_split8(const float* p, bf16x8_t& hi, bf16x8_t& lo) {
  bf16_split8(*reinterpret_cast<const v4f*>(p), *reinterpret_cast<const v4f*>(p + 4), hi, lo);
}

// A bf16 MFMA operand from two runs of four bf16 values 16 elements apart (k = 0..3 and 4..7).
__device__ __forceinline__ bf16x8_t bf16_pair4(const uint16_t* p) {
  const uint2 u0 = *reinterpret_cast<const uint2*>(p), u1 = *reinterpret_cast<const uint2*>(p + 16);
  return __builtin_bit_cast(bf16x8_t, u32x4_t{u0.x, u0.y, u1.x, u1.y});
}

__device__ __forceinline__ v4f mfma_bf16(const bf16x8_t& a, const bf16x8_t& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int MODE>
__device__ __forceinline__ float ldin(const void* p, size_t i) {
  if constexpr (MODE == 0) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  else return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ size_t tok(int b, int t, int T, int H, int h) {
  return (static_cast<size_t>(b) * T + t) * H + h;
}


// Query and key rows in LDS keep the input's type: bf16 inputs stay bf16 (exact), which halves
// their footprint.
template <int MODE> struct LdsIn { using type = float; };
template <> struct LdsIn<0> { using type = uint16_t; };
__device__ __forceinline__ float lds_f(float x) { return x; }
__device__ __forceinline__ float lds_f(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

// Eight consecutive row elements from a 16-byte aligned LDS address, as fp32.
__device__ __forceinline__ void row8(const uint16_t* p, float f[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void row8(const float* p, float f[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Rows of a [B,T,H,D] input (in its own element type) for the 64 tokens of chunk c into s[64][P],
// in 16-byte pieces, zeros past T; rows of s must start on 16-byte boundaries.
template <int MODE, int D, int P, class E>
__device__ __forceinline__ void load_rows_vec(E (*s)[P], const void* x, int b, int h, int c, int T, int H) {
  constexpr int EV = 16 / sizeof(E), KV = D / EV;
  static_assert((P * sizeof(E)) % 16 == 0, "16-byte rows");
  for (int e = threadIdx.x; e < BC * KV; e += blockDim.x) {
    const int rr = e / KV, pe = e % KV, t = c * BC + rr;
    uint4 u = {0u, 0u, 0u, 0u};
    if (t < T) u = reinterpret_cast<const uint4*>(static_cast<const E*>(x) + tok(b, t, T, H, h) * D)[pe];
    *reinterpret_cast<uint4*>(&s[rr][pe * EV]) = u;
  }
}


template <int MODE, int DK>
__global__ __launch_bounds__(BT) void bwd_prep_kernel(const void* q, const void* k, const float* log_alpha,
                                                      const float* eta, float eps, int direct, int T, int H, int nc,
                                                      float* rec) {
  constexpr int AP = 68;  // pitch of A: 16-byte rows for vector reads
  const int c = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, tid = threadIdx.x;
  using E = typename LdsIn<MODE>::type;  // bf16 inputs stay bf16 in LDS (exact): three workgroups per CU
  constexpr int EP = MODE == 0 ? DK + 8 : DK + 4;  // 16-byte rows
  __shared__ __align__(16) E sQ[BC][EP];
  __shared__ __align__(16) E sK[BC][EP];
  __shared__ __align__(16) float sA[BC * AP];
  __shared__ float sla[BC], sg[BC], sb[BC];
  load_rows_vec<MODE, DK, EP, E>(sQ, q, b, h, c, T, H);
  load_rows_vec<MODE, DK, EP, E>(sK, k, b, h, c, T, H);
  float* R = rec + (static_cast<size_t>(bh) * nc + c) * RECF;
  const int t = c * BC + tid;
  if (tid < BC) sla[tid] = t < T ? log_alpha[tok(b, t, T, H, h)] : 0.f;
  __syncthreads();
  if constexpr (MODE == 0) {
    // bf16 inputs: Q K^T and K K^T on the bf16 MFMA (exact products, fp32 accumulation), wave w
    // on row tile w and all four column tiles (lane l supplies row l % 16, columns
    // 32 kb + 8 (l / 16) + 0..7 of both operands; the result's rows 4 (l / 16) + e, column l % 16
    // sit in lane l's acc[e]); ||k||^2 is the diagonal of K K^T.
    const int lane = tid & 63, wv = tid >> 6, gq = lane >> 4, ln = lane & 15;
    v4f qk[4], kk[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) qk[nt] = kk[nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
      const bf16x8_t aq = *reinterpret_cast<const bf16x8_t*>(&sQ[16 * wv + ln][32 * kb + 8 * gq]);
      const bf16x8_t ak = *reinterpret_cast<const bf16x8_t*>(&sK[16 * wv + ln][32 * kb + 8 * gq]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const bf16x8_t bk = *reinterpret_cast<const bf16x8_t*>(&sK[16 * nt + ln][32 * kb + 8 * gq]);
        qk[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bk, qk[nt], 0, 0, 0);
        kk[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bk, kk[nt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * gq + e == ln) sb[16 * wv + ln] = kk[wv][e];  // ||k_r||^2, until beta replaces it
    __syncthreads();
    if (tid < BC) {  // wave 0, lane r = token r: g by an inclusive scan over the wave
      float gs = sla[tid];
#pragma unroll
      for (int o = 1; o < BC; o <<= 1) {
        const float y = __shfl_up(gs, o);
        if (lane >= o) gs += y;
      }
      const float et = t < T ? eta[tok(b, t, T, H, h)] : 0.f;
      const float den = sb[tid] + eps;
      const float beta = direct ? et : (den != 0.f ? et / den : 0.f);
      sg[tid] = gs;
      sb[tid] = beta;
      R[REC_G + tid] = gs;
      R[REC_B + tid] = beta;
      R[REC_D + tid] = den;
    }
    __syncthreads();
    // lower triangle incl. the diagonal: P = Dl . Q K^T; strict upper: K K^T; A = strict lower
    // beta_r Dl G
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * wv + 4 * gq + e, i = 16 * nt + ln;
        const float dl = i <= r ? expf(sg[r] - sg[i]) : 0.f;
        R[REC_PG + r * BC + i] = i <= r ? dl * qk[nt][e] : kk[nt][e];
        sA[r * AP + i] = i < r ? sb[r] * dl * kk[nt][e] : 0.f;
      }
  } else {  // fp32 inputs: the vector ALU in 4 x 4 register tiles
    if (tid < BC) {
      float gs = 0.f;
      for (int i = 0; i <= tid; ++i) gs += sla[i];
      float n = 0.f;
      for (int d = 0; d < DK; ++d) n = fmaf(lds_f(sK[tid][d]), lds_f(sK[tid][d]), n);
      const float et = t < T ? eta[tok(b, t, T, H, h)] : 0.f;
      const float den = n + eps;
      const float beta = direct ? et : (den != 0.f ? et / den : 0.f);
      sg[tid] = gs;
      sb[tid] = beta;
      R[REC_G + tid] = gs;
      R[REC_B + tid] = beta;
      R[REC_D + tid] = den;
    }
    __syncthreads();
    // Q K^T and K K^T in 4 x 4 tiles (rows r0 + 4a, columns i0 + 4b... strided by 16 so that a
    // wave's reads of K rows spread over banks). Lower triangle incl. the diagonal: P = Dl . Q K^T;
    // strict upper: K K^T (symmetric, so entry [r][i], i > r, is also G[i][r]);
    // A = strict lower beta_r Dl G.
    {
      const int r0 = tid >> 4, i0 = tid & 15;
      float qk[4][4] = {}, kk[4][4] = {};
      for (int d = 0; d < DK; ++d) {
        float qa[4], ka[4], kb[4];
        for (int a = 0; a < 4; ++a) {
          qa[a] = lds_f(sQ[r0 + 16 * a][d]);
          ka[a] = lds_f(sK[r0 + 16 * a][d]);
          kb[a] = lds_f(sK[i0 + 16 * a][d]);
        }
        for (int a = 0; a < 4; ++a)
          for (int e = 0; e < 4; ++e) {
            qk[a][e] = fmaf(qa[a], kb[e], qk[a][e]);
            kk[a][e] = fmaf(ka[a], kb[e], kk[a][e]);
          }
      }
      for (int a = 0; a < 4; ++a)
        for (int e = 0; e < 4; ++e) {
          const int r = r0 + 16 * a, i = i0 + 16 * e;
          const float dl = i <= r ? expf(sg[r] - sg[i]) : 0.f;
          R[REC_PG + r * BC + i] = i <= r ? dl * qk[a][e] : kk[a][e];
          sA[r * AP + i] = i < r ? sb[r] * dl * kk[a][e] : 0.f;
        }
    }
  }
  __syncthreads();
  // (I + A)^-1 is unit lower triangular. Forward substitution with one column per lane held in
  // registers: row r of the inverse is e_r - A[r][:] m over the rows already found (m[i] = 0
  // for i above the column), and every lane reads the same A row (an LDS broadcast).
  if (tid < BC) {
    const int col = tid;
    float m[BC];
#pragma unroll
    for (int r = 0; r < BC; ++r) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int i = 0; i + 4 <= r; i += 4) {
        const float4 a4 = *reinterpret_cast<const float4*>(&sA[r * AP + i]);
        s0 = fmaf(a4.x, m[i], s0);
        s1 = fmaf(a4.y, m[i + 1], s1);
        s0 = fmaf(a4.z, m[i + 2], s0);
        s1 = fmaf(a4.w, m[i + 3], s1);
      }
#pragma unroll
      for (int i = r & ~3; i < r; ++i) s0 = fmaf(sA[r * AP + i], m[i], s0);
      m[r] = r == col ? 1.f : -(s0 + s1);
    }
#pragma unroll
    for (int r = 0; r < BC; ++r) R[REC_M + r * BC + col] = m[r];
  }
}


// One fp32 MFMA step (16 x 16 tile, K = 4, full fp32 products): lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16]; the tile's rows 4 (l / 16) + i, column l % 16, sit in lane l's acc[i].
__device__ __forceinline__ v4f mfma4(float a, float b, v4f acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Element j of a 16-byte piece of E values, taken from the piece's words (no address of the
// register piece is taken, so it stays in registers).
template <class E>
__device__ __forceinline__ E piece_elem(const uint4& u, int j) {
  const uint32_t wd = j / (4 / sizeof(E)) == 0 ? u.x : j / (4 / sizeof(E)) == 1 ? u.y : j / (4 / sizeof(E)) == 2 ? u.z : u.w;
  if constexpr (sizeof(E) == 2) return static_cast<E>((j & 1) ? wd >> 16 : wd & 0xFFFFu);
  else return __uint_as_float(wd);
}

// Chunk-local terms of the reverse walk, all chunks in parallel on the fp32 MFMA:
//   V~ = P^T dO (64 x dv) into vt, and Q^T (e^g . dO) (dk x dv) into the chunk's slot of dstates,
// which the reverse walk reads and then overwrites with the chunk-end state gradient.
// One workgroup per (b, h, chunk), one wave per 16 columns of dO. A wave loads its columns of
// dO straight into the accumulator layout of a 64 x 16 tile set (lane l: tokens 16 t + 4 (l/16)
// + e, column l % 16), which is the B operand of the K = 4 steps over the chunk's tokens; the A
// operands (P^T and Q^T, staged transposed in LDS) are one 16- or 8-byte read per four steps.
template <int MODE, int DK>
__global__ __launch_bounds__(NT) void bwd_dprep_kernel(const void* q, const float* dout, const float* rec, int T, int H,
                                                       int DV, int nc, float* vt, float* cq) {
  using E = typename LdsIn<MODE>::type;
  constexpr int EV = 16 / sizeof(E), KV = DK / EV;  // elements per 16-byte piece, pieces per query row
  constexpr int QTP = BC + EV;                     // pitch of Q^T [DK][QTP] (16-byte rows)
  constexpr int PTP = BC + 4;                      // pitch of P^T [BC][PTP]
  __shared__ __align__(16) E sQt[DK][QTP];
  __shared__ __align__(16) float sPt[BC][PTP];
  __shared__ __align__(16) float seg[BC];
  const int c = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, tid = threadIdx.x;
  const int nthr = static_cast<int>(blockDim.x);
  const int lane = tid & 63, wv = tid >> 6, gq = lane >> 4, ln = lane & 15;
  const float* R = rec + (static_cast<size_t>(bh) * nc + c) * RECF;
  const size_t cidx = static_cast<size_t>(bh) * nc + c;
  const int col = 16 * wv + ln;
  // this wave's columns of dO in the accumulator layout (zero past T)
  float o[4][4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = c * BC + 16 * tt + 4 * gq + e;
      o[tt][e] = t < T ? dout[tok(b, t, T, H, h) * DV + col] : 0.f;
    }
  // Q^T and P^T (P's lower triangle incl. the diagonal) into LDS; consecutive lanes take
  // consecutive tokens, so the transposed writes hit consecutive words
  for (int e = tid; e < BC * KV; e += nthr) {
    const int rr = e % BC, pe = e / BC, t = c * BC + rr;
    uint4 u = {0u, 0u, 0u, 0u};
    if (t < T) u = *(reinterpret_cast<const uint4*>(static_cast<const E*>(q) + tok(b, t, T, H, h) * DK) + pe);
#pragma unroll
    for (int j = 0; j < EV; ++j) sQt[pe * EV + j][rr] = piece_elem<E>(u, j);
  }
  for (int e = tid; e < BC * BC / 4; e += nthr) {
    const int rr = e % BC, pc = e / BC;  // token rr, columns 4 pc .. 4 pc + 3 of its row of P
    const v4f x = reinterpret_cast<const v4f*>(R + REC_PG)[rr * (BC / 4) + pc];
#pragma unroll
    for (int j = 0; j < 4; ++j) sPt[4 * pc + j][rr] = 4 * pc + j <= rr ? x[j] : 0.f;
  }
  if (tid < BC) seg[tid] = expf(R[REC_G + tid]);
  __syncthreads();
  v4f P4[4], C4[DK / 16];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) P4[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dt = 0; dt < DK / 16; ++dt) C4[dt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const v4f eg = *reinterpret_cast<const v4f*>(&seg[16 * tt + 4 * gq]);
    v4f ap[4];
#pragma unroll
    for (int mt = 0; mt <= tt; ++mt) ap[mt] = *reinterpret_cast<const v4f*>(&sPt[16 * mt + ln][16 * tt + 4 * gq]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int mt = 0; mt <= tt; ++mt) P4[mt] = mfma4(ap[mt][e], o[tt][e], P4[mt]);  // P^T[row][token] = 0 below
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      const E* pq = &sQt[16 * dt + ln][16 * tt + 4 * gq];
      float aq[4];
      if constexpr (MODE == 0) {
        const uint2 w2 = *reinterpret_cast<const uint2*>(pq);
        aq[0] = __uint_as_float(w2.x << 16);
        aq[1] = __uint_as_float(w2.x & 0xFFFF0000u);
        aq[2] = __uint_as_float(w2.y << 16);
        aq[3] = __uint_as_float(w2.y & 0xFFFF0000u);
      } else {
        const v4f w4 = *reinterpret_cast<const v4f*>(pq);
        aq[0] = w4[0]; aq[1] = w4[1]; aq[2] = w4[2]; aq[3] = w4[3];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) C4[dt] = mfma4(aq[e], eg[e] * o[tt][e], C4[dt]);
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) vt[(cidx * BC + 16 * mt + 4 * gq + e) * DV + col] = P4[mt][e];
#pragma unroll
  for (int dt = 0; dt < DK / 16; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) cq[(cidx * DK + 16 * dt + 4 * gq + e) * DV + col] = C4[dt][e];
}

// The two walks on the fp32 MFMA, one kernel: one workgroup per (b, h, 64 state columns), four
// waves of 16 columns, each wave's 16 columns of the carried matrix in MFMA accumulators for the
// whole walk. Every product has a chunk's 64 tokens or the state's dk rows as its contraction;
// the carried matrix enters as the B operand straight from the accumulators (a 16 x 16 tile's
// lane l holds rows 4 (l / 16) + i, i = 0..3, of column l % 16, which is the B operand of four
// K = 4 steps whose contraction slots are those rows), so only the A operands come from LDS:
//   forward (REV = false), S = chunk-start state, stored for every chunk:
//     R = K S,  X = beta . (V - e^g . R),  U = Minv X,  S <- e^{g_C} S + K^T (w . U)
//   reverse (REV = true), dS = chunk-end gradient dS1, stored for every chunk over the chunk's
//   slot of Q^T (e^g . dO) after reading it, the start state's gradient at the end:
//     dU = w . (K dS1) + V~,  dX = diag(beta) Minv^T dU,
//     dS0 = e^{g_C} dS1 + Q^T (e^g . dO) - K^T (e^g . dX)
// Key rows are staged in LDS twice (row-major for K, transposed for K^T) in the input's type
// (bf16 stays exact), the inverse row-major (forward) or transposed (reverse), the values (or
// V~) transposed in fp32, so that every A operand of a K = 4 step is one 8- or 16-byte read.
// The next chunk's rows are loaded into registers while the current chunk is computed.
// A walk workgroup has NW waves of 16 state columns: four (64 columns) when that gives every CU
// a workgroup, fewer otherwise (few heads: dk = 256 workloads, long single sequences), at least
// two at dk = 256, where one wave's registers cannot hold a chunk's prefetched rows.

// The LDS of one chunk of a walk: key rows, transposed key rows, the inverse (or its
// transpose), the transposed values (or V~), and the chunk's per-token factors e^g, beta,
// w = e^{g_C - g}, e^g beta and e^{g_C}.
template <class E, int DK, int WC>
struct WalkChunkLds {
  static constexpr int EV = 16 / sizeof(E);
  static constexpr int KP = DK + EV, TP = BC + EV;  // pitches of K [BC][KP] and K^T [DK][TP] (16-byte rows)
  static constexpr int MPP = BC + 4, VP = BC + 4;   // pitches of the inverse and of the transposed values
  E sK[BC][KP];
  E sKt[DK][TP];
  float sM[BC][MPP];
  float sV[WC][VP];
  float sEG[BC], sB[BC], sW[BC], sEB[BC];
  float sGam;
};

// A launch walks segments seg0 .. seg0 + nseg - 1 of seg_chunks chunks each (one segment of nc
// chunks for the whole sequence), workgroup row blockIdx.y = bh * nseg + (segment - seg0). A
// segment starts from sin's slot (bh, segment) of sin_segs per head (zero if sin is null),
// stores every chunk's carried matrix if dump is set, and leaves its final carried matrix in
// slast's slot (bh, segment) when segment < slast_segs.
template <int MODE, int DK, bool REV, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_walk_kernel(const void* k, const void* vin, const float* rec,
                                                      const float* sin, int T, int H, int DV, int nc, float* sdump,
                                                      float* slast, int seg_chunks, int nseg, int seg0, int sin_segs,
                                                      int slast_segs, int dump) {
  using E = typename LdsIn<MODE>::type;
  constexpr int WT = 64 * NW, WCOL = 16 * NW;     // threads, state columns
  using L = WalkChunkLds<E, DK, WCOL>;
  constexpr int EV = L::EV;
  constexpr int KV = DK / EV, KPT = BC * KV / WT;   // key pieces per row, per thread
  constexpr int MPT = BC * BC / 4 / WT;             // float4s of the inverse per thread
  using VE = typename std::conditional<REV, float, E>::type;  // element type of the value rows
  constexpr int VEV = 16 / sizeof(VE), VV = WCOL / VEV, VPT = BC * VV / WT;  // value pieces
  constexpr int NDT = DK / 16;                      // 16-row tiles of the carried matrix
  // bf16 rows at dk <= 128 leave room for two chunks' LDS: the next chunk is staged while this
  // one is computed, with one workgroup barrier per chunk. fp32 rows and dk = 256 stage between
  // two barriers.
  constexpr bool DB = MODE == 0 && DK <= 128;
  static_assert(KPT * WT == BC * KV && MPT * WT * 4 == BC * BC && VPT * WT == BC * VV, "walk tiling");
  __shared__ __align__(16) L lds0;
  __shared__ __align__(16) L lds1_[1];  // referenced (and allocated) only when DB
  L& lds1 = DB ? lds1_[0] : lds0;
  // per-wave 16 x 16 transpose tile: the accumulator layout to and from rows of 16-byte pieces
  __shared__ __align__(16) float sTr[NW][16][20];
  const int bh = blockIdx.y / nseg, seg = seg0 + blockIdx.y % nseg;
  const int jb = blockIdx.x * WCOL, b = bh / H, h = bh % H, tid = threadIdx.x;
  const int cb = seg * seg_chunks, ncount = min(nc, cb + seg_chunks) - cb;  // this segment's chunks
  const int lane = tid & 63, w = tid >> 6, gq = lane >> 4, ln = lane & 15;
  const int col = jb + 16 * w + ln;  // this lane's column of the carried matrix

  // ---- a later chunk's rows in registers ----
  uint4 pk[KPT];
  v4f pm[MPT];
  uint4 pv[VPT];
  float pg = 0.f, pb = 0.f;
  v4f pc[REV ? NDT : 1];
  // a lane's 16-byte piece of a 16 x 16 tile of the carried matrix: row lane / 4, columns 4 (lane % 4) + 0..3
  const int prow = lane >> 2, pcol = jb + 16 * w + 4 * (lane & 3);
  auto fetch_rows = [&](int c) __attribute__((always_inline)) {
    const size_t cidx = static_cast<size_t>(bh) * nc + c;
    const float* R = rec + cidx * RECF;
#pragma unroll
    for (int x = 0; x < KPT; ++x) {
      const int e = tid + x * WT, rr = e % BC, pe = e / BC, t = c * BC + rr;
      pk[x] = t < T ? *(reinterpret_cast<const uint4*>(static_cast<const E*>(k) + tok(b, t, T, H, h) * DK) + pe)
                    : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int x = 0; x < MPT; ++x) {
      // forward: row-major pieces (coalesced); reverse: consecutive lanes take consecutive rows
      const int e = tid + x * WT;
      pm[x] = reinterpret_cast<const v4f*>(R + REC_M)[REV ? (e % BC) * (BC / 4) + e / BC : e];
    }
#pragma unroll
    for (int x = 0; x < VPT; ++x) {
      const int e = tid + x * WT, rr = e % BC, pe = e / BC, t = c * BC + rr;
      if constexpr (REV) {  // V~ = P^T dO of the chunk, fp32 [BC][DV] (zero rows past T already)
        pv[x] = *reinterpret_cast<const uint4*>(static_cast<const float*>(vin) + (cidx * BC + rr) * DV + jb + VEV * pe);
      } else {
        pv[x] = t < T ? *reinterpret_cast<const uint4*>(static_cast<const E*>(vin) + tok(b, t, T, H, h) * DV + jb + VEV * pe)
                      : uint4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < BC) {
      pg = R[REC_G + tid];
      pb = R[REC_B + tid];
    }
  };
  // reverse walk: this wave's columns of Q^T (e^g . dO), the chunk's slot of dstates
  auto fetch_c = [&](int c) __attribute__((always_inline)) {
    if constexpr (REV) {
      const float* C = sdump + (static_cast<size_t>(bh) * nc + c) * DK * DV;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) pc[dt] = *reinterpret_cast<const v4f*>(C + (16 * dt + prow) * DV + pcol);
    }
  };
  auto stage = [&](L& Q) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < KPT; ++x) {
      const int e = tid + x * WT, rr = e % BC, pe = e / BC;
      *reinterpret_cast<uint4*>(&Q.sK[rr][pe * EV]) = pk[x];
#pragma unroll
      for (int j = 0; j < EV; ++j) Q.sKt[pe * EV + j][rr] = piece_elem<E>(pk[x], j);
    }
#pragma unroll
    for (int x = 0; x < MPT; ++x) {
      const int e = tid + x * WT;
      if constexpr (REV) {
        const int rr = e % BC, cc = 4 * (e / BC);
#pragma unroll
        for (int j = 0; j < 4; ++j) Q.sM[cc + j][rr] = pm[x][j];
      } else {
        const int rr = (4 * e) / BC, cc = (4 * e) % BC;
        *reinterpret_cast<v4f*>(&Q.sM[rr][cc]) = pm[x];
      }
    }
#pragma unroll
    for (int x = 0; x < VPT; ++x) {
      const int e = tid + x * WT, rr = e % BC, pe = e / BC;
#pragma unroll
      for (int j = 0; j < VEV; ++j) Q.sV[VEV * pe + j][rr] = lds_f(piece_elem<VE>(pv[x], j));
    }
    if (tid < BC) {  // wave 0: one token per lane
      const float gC = __shfl(pg, BC - 1);
      const float eg = expf(pg);
      Q.sEG[tid] = eg;
      Q.sB[tid] = pb;
      Q.sW[tid] = expf(gC - pg);
      Q.sEB[tid] = eg * pb;
      if (tid == 0) Q.sGam = expf(gC);
    }
  };
  // four consecutive elements of an LDS row as fp32 (an A operand of four K = 4 steps)
  auto rd4 = [](const E* p) __attribute__((always_inline)) {
    float f[4];
    if constexpr (MODE == 0) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      f[0] = __uint_as_float(u.x << 16);
      f[1] = __uint_as_float(u.x & 0xFFFF0000u);
      f[2] = __uint_as_float(u.y << 16);
      f[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
      const float4 u = *reinterpret_cast<const float4*>(p);
      f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
    }
    return float4{f[0], f[1], f[2], f[3]};
  };
  auto el4 = [](const float4& x, int i) __attribute__((always_inline)) {
    return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
  };

  // ---- the carried matrix ----
  v4f S[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[dt][i] = sin ? sin[((static_cast<size_t>(bh) * sin_segs + seg) * DK + 16 * dt + 4 * gq + i) * DV + col] : 0.f;

  // The start of chunk c: the reverse walk's Q^T (e^g . dO) of the chunk into the accumulator
  // layout, then the carried matrix out to the chunk's slot in 16-byte pieces, per 16-row tile
  // through the wave's transpose tile (LDS operations of a wave run in order). Every load of the
  // slot has returned before it is overwritten (the caller waits for vmcnt(0)).
  float cterm[REV ? NDT * 4 : 1];
  auto chunk_start = [&](int c) __attribute__((always_inline)) {
    float* D = sdump + (static_cast<size_t>(bh) * nc + c) * DK * DV;
    float (*tr)[20] = sTr[w];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if constexpr (REV) {
        *reinterpret_cast<v4f*>(&tr[prow][4 * (lane & 3)]) = pc[dt];
#pragma unroll
        for (int i = 0; i < 4; ++i) cterm[4 * dt + i] = tr[4 * gq + i][ln];
      }
      if (dump) {
#pragma unroll
        for (int i = 0; i < 4; ++i) tr[4 * gq + i][ln] = S[dt][i];
        *reinterpret_cast<v4f*>(D + (16 * dt + prow) * DV + pcol) = *reinterpret_cast<const v4f*>(&tr[prow][4 * (lane & 3)]);
      }
    }
  };
  // bf16 inputs: the same products on the bf16 MFMA (16 x 16 x 32). Keys are exact in bf16; the
  // fp32 operands (the carried matrix, X or dU, Y and the inverse) enter as hi + lo pairs: two
  // passes where the other operand is a key, three (hi hi, hi lo, lo hi) for the inverse. The
  // contraction index of a 32-wide step is ordered so that a lane's B operand is its accumulator
  // values of two adjacent 16-row tiles: k = 8 (l / 16) + j is row 4 (l / 16) + j of the first
  // tile for j < 4 and of the second for j >= 4; the A operands follow the same order.
  auto compute_bf16 = [&](const L& Q, auto&& mid) __attribute__((always_inline)) {
    if constexpr (MODE == 0) {
      // R = K S (token tiles mt), over 32-row slabs of S
      v4f R[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) R[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < NDT / 2; ++sl) {
        bf16x8_t bh, bl;
        bf16_split8(S[2 * sl], S[2 * sl + 1], bh, bl);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const bf16x8_t a = bf16_pair4(&Q.sK[16 * mt + ln][32 * sl + 4 * gq]);
          R[mt] = mfma_bf16(a, bl, mfma_bf16(a, bh, R[mt]));
        }
      }
      mid();
      // forward: X = beta . (V - e^g . R); reverse: dU = w . R + V~
      v4f X[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const v4f vv = *reinterpret_cast<const v4f*>(&Q.sV[16 * w + ln][16 * mt + 4 * gq]);
        const v4f eg = *reinterpret_cast<const v4f*>(&Q.sEG[16 * mt + 4 * gq]);
        const v4f bb = *reinterpret_cast<const v4f*>(&Q.sB[16 * mt + 4 * gq]);
        const v4f ww = *reinterpret_cast<const v4f*>(&Q.sW[16 * mt + 4 * gq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (REV) X[mt][i] = fmaf(ww[i], R[mt][i], vv[i]);
          else X[mt][i] = bb[i] * (vv[i] - eg[i] * R[mt][i]);
        }
      }
      // forward: U = Minv X (token slabs at or below the row tile); reverse: Minv^T dU (at or above)
      v4f U[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) U[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        bf16x8_t xh, xl;
        bf16_split8(X[2 * sl], X[2 * sl + 1], xh, xl);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (REV ? 2 * sl + 1 < mt : 2 * sl > mt) continue;
          const float* m = &Q.sM[16 * mt + ln][32 * sl + 4 * gq];
          bf16x8_t ah, al;
          bf16_split8(*reinterpret_cast<const v4f*>(m), *reinterpret_cast<const v4f*>(m + 16), ah, al);
          U[mt] = mfma_bf16(al, xh, mfma_bf16(ah, xl, mfma_bf16(ah, xh, U[mt])));
        }
      }
      // forward: Y = w . U, S <- e^{g_C} S + K^T Y;  reverse: Y = -e^g . beta . (Minv^T dU),
      // dS <- e^{g_C} dS + Q^T (e^g . dO) + K^T Y
      v4f Y[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const v4f eb = *reinterpret_cast<const v4f*>(&Q.sEB[16 * mt + 4 * gq]);
        const v4f ww = *reinterpret_cast<const v4f*>(&Q.sW[16 * mt + 4 * gq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (REV) Y[mt][i] = -eb[i] * U[mt][i];
          else Y[mt][i] = ww[i] * U[mt][i];
        }
      }
      const float gam = Q.sGam;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (REV) S[dt][i] = fmaf(gam, S[dt][i], cterm[4 * dt + i]);
          else S[dt][i] = gam * S[dt][i];
        }
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        bf16x8_t yh, yl;
        bf16_split8(Y[2 * sl], Y[2 * sl + 1], yh, yl);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8_t a = bf16_pair4(&Q.sKt[16 * dt + ln][32 * sl + 4 * gq]);
          S[dt] = mfma_bf16(a, yl, mfma_bf16(a, yh, S[dt]));
        }
      }
    }
  };
  // One chunk's products from the staged chunk Q. `mid` runs after the first product has been
  // issued (the next chunk's staging, in the double-buffered walk).
  auto compute = [&](const L& Q, auto&& mid) __attribute__((always_inline)) {
    if constexpr (MODE == 0) {
      compute_bf16(Q, mid);
      return;
    }
    // R = K S (token tiles mt)
    v4f R[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) R[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      float4 a[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) a[mt] = rd4(&Q.sK[16 * mt + ln][16 * dt + 4 * gq]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) R[mt] = mfma4(el4(a[mt], i), S[dt][i], R[mt]);
    }
    mid();
    // forward: X = beta . (V - e^g . R); reverse: dU = w . R + V~
    v4f X[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float4 vv = *reinterpret_cast<const float4*>(&Q.sV[16 * w + ln][16 * mt + 4 * gq]);
      const float4 eg = *reinterpret_cast<const float4*>(&Q.sEG[16 * mt + 4 * gq]);
      const float4 bb = *reinterpret_cast<const float4*>(&Q.sB[16 * mt + 4 * gq]);
      const float4 ww = *reinterpret_cast<const float4*>(&Q.sW[16 * mt + 4 * gq]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (REV) X[mt][i] = fmaf(el4(ww, i), R[mt][i], el4(vv, i));
        else X[mt][i] = el4(bb, i) * (el4(vv, i) - el4(eg, i) * R[mt][i]);
      }
    }
    // forward: U = Minv X (lower triangular blocks kt <= mt); reverse: Minv^T dU (kt >= mt)
    v4f U[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) U[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float4 a[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        if (REV ? kt >= mt : kt <= mt) a[mt] = *reinterpret_cast<const float4*>(&Q.sM[16 * mt + ln][16 * kt + 4 * gq]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          if (REV ? kt >= mt : kt <= mt) U[mt] = mfma4(el4(a[mt], i), X[kt][i], U[mt]);
    }
    // forward: Y = w . U, S <- e^{g_C} S + K^T Y;  reverse: Y = -e^g . beta . (Minv^T dU),
    // dS <- e^{g_C} dS + Q^T (e^g . dO) + K^T Y
    v4f Y[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float4 eb = *reinterpret_cast<const float4*>(&Q.sEB[16 * mt + 4 * gq]);
      const float4 ww = *reinterpret_cast<const float4*>(&Q.sW[16 * mt + 4 * gq]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (REV) Y[mt][i] = -el4(eb, i) * U[mt][i];
        else Y[mt][i] = el4(ww, i) * U[mt][i];
      }
    }
    const float gam = Q.sGam;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (REV) S[dt][i] = fmaf(gam, S[dt][i], cterm[4 * dt + i]);
        else S[dt][i] = gam * S[dt][i];
      }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float4 a[NDT];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) a[dt] = rd4(&Q.sKt[16 * dt + ln][16 * kt + 4 * gq]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) S[dt] = mfma4(el4(a[dt], i), Y[kt][i], S[dt]);
    }
  };

  const int c_first = REV ? cb + ncount - 1 : cb, c_step = REV ? -1 : 1;
  if constexpr (DB) {
    // chunk n is computed from lds[n % 2] while chunk n + 1 is staged into the other; the rows of
    // chunk n + 2 are loaded into registers meanwhile, the reverse walk's Q^T (e^g . dO) of chunk
    // n + 1 after chunk n's slot is written
    fetch_rows(c_first);
    fetch_c(c_first);
    stage(lds0);
    if (ncount > 1) fetch_rows(c_first + c_step);
    __syncthreads();
    auto step = [&](int n, L& cur, L& nxt) __attribute__((always_inline)) {
      const int c = c_first + n * c_step;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      chunk_start(c);
      if (n + 1 < ncount) fetch_c(c + c_step);
      compute(cur, [&]() __attribute__((always_inline)) {
        if (n + 1 < ncount) {
          stage(nxt);
          if (n + 2 < ncount) fetch_rows(c + 2 * c_step);
        }
      });
      __syncthreads();  // the next chunk is staged; every read of this one is done
    };
    for (int n = 0; n < ncount; n += 2) {
      step(n, lds0, lds1);
      if (n + 1 < ncount) step(n + 1, lds1, lds0);
    }
  } else {
    fetch_rows(c_first);
    fetch_c(c_first);
    for (int n = 0; n < ncount; ++n) {
      const int c = c_first + n * c_step;
      __syncthreads();  // every wave's reads of the previous chunk's rows are done
      stage(lds0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      chunk_start(c);
      if (n + 1 < ncount) {
        fetch_rows(c + c_step);
        fetch_c(c + c_step);
      }
      __syncthreads();
      compute(lds0, []() __attribute__((always_inline)) {});
    }
  }
  if (slast && seg < slast_segs) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        slast[((static_cast<size_t>(bh) * slast_segs + seg) * DK + 16 * dt + 4 * gq + i) * DV + col] = S[dt][i];
  }
}

// Sum over the TPRW adjacent lanes that share a chunk row.
__device__ __forceinline__ float quad_sum(float x) {
  for (int m = 1; m < TPRW; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Per-chunk gradients from the chunk-start state S0 and the chunk-end gradient dS1. The state
// columns are taken in blocks of NJG: 32 for bf16 inputs, whose query and key rows stay bf16 in
// LDS (exact), 16 for fp32 inputs, whose rows take twice the room.
template <int MODE, int DK>
__global__ __launch_bounds__(NT) void bwd_grads_kernel(const void* q, const void* k, const void* v, const float* eta,
                                                       const float* dout, const float* rec, const float* states,
                                                       const float* dstates, int direct, int T, int H, int DV, int nc,
                                                       float* dq, float* dk, float* dv, float* dla, float* deta) {
  // bf16 inputs with dk <= 128: 32-column blocks, one 16 x 16 tile of every product per wave
  // (FUSED); otherwise (fp32 rows, or dk = 256, where the LDS holds only 16-column blocks)
  // 16-column blocks, split over the waves by product
  constexpr bool FUSED = MODE == 0 && DK <= 128;
  constexpr int NJG = FUSED ? 32 : 16, CPTG = NJG / TPRW;
  constexpr int EPT = DK * NJG / NT, TPR = NJG / EPT;
  constexpr int SP = DK + 4, RP = BC + 4;  // pitches of the column-major blocks (16-byte rows)
  constexpr int WCOL = 2 * NJG * SP + 5 * NJG * RP, WMAT = 2 * BC * MP;
  constexpr int WN = WCOL > WMAT ? WCOL : WMAT;
  const int c = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H, tid = threadIdx.x;
  // Query and key rows in their input type, 16-byte rows; the bf16 pitch (DK + 16 halves) puts
  // the four rows of an MFMA K step on disjoint banks
  using QE = typename LdsIn<MODE>::type;
  constexpr int QP = MODE == 0 ? DK + 16 : DK + 4;
  __shared__ __align__(16) QE sQ[BC][QP], sK[BC][QP];
  __shared__ float sM[BC][MP], sPG[BC][MP];
  __shared__ __align__(16) float sW[WN];
  __shared__ float sg[BC], sb[BC], sden[BC], sdb[BC], srow[BC], sdeg[BC], sdw[BC], skc[BC];
  __shared__ float seg[BC], sww[BC];  // e^{g}, e^{g_C - g}
  __shared__ float sgp[BC];  // per-row parts of <dS1, S0>
  __shared__ float sdw2[FUSED ? BC : 1], sdeg2[FUSED ? BC : 1];  // second column-tile halves
  // column-block phase: 16 columns of each operand, stored column by column so that a
  // thread's run of rows (or of state rows) is one 16-byte read
  float* cS = sW;              // S0 [NJG][SP]
  float* cD = cS + NJG * SP;   // dS1 [NJG][SP]
  float* cX = cD + NJG * SP;   // V, then X [NJG][RP]
  float* cO = cX + NJG * RP;   // dO
  float* cU = cO + NJG * RP;   // U
  float* cDU = cU + NJG * RP;
  float* cDX = cDU + NJG * RP;
  // matrix phase
  float* m1 = sW;
  float* m2 = sW + BC * MP;

  const float* R = rec + (static_cast<size_t>(bh) * nc + c) * RECF;
  const float* S0 = states + (static_cast<size_t>(bh) * nc + c) * DK * DV;
  const float* D1 = dstates + (static_cast<size_t>(bh) * nc + c) * DK * DV;
  // query and key rows and the record's two matrices, in 16-byte loads
  {
    using E = typename LdsIn<MODE>::type;
    constexpr int EV = 16 / sizeof(E), KV = DK / EV;  // elements per piece, pieces per row
#pragma unroll
    for (int x = 0; x < BC * KV / NT; ++x) {
      const int e = tid + x * NT, rr = e / KV, pe = e % KV, t = c * BC + rr;
      uint4 uq = {0u, 0u, 0u, 0u}, uk = {0u, 0u, 0u, 0u};
      if (t < T) {
        const size_t o = tok(b, t, T, H, h) * DK;
        uq = reinterpret_cast<const uint4*>(static_cast<const E*>(q) + o)[pe];
        uk = reinterpret_cast<const uint4*>(static_cast<const E*>(k) + o)[pe];
      }
      *reinterpret_cast<uint4*>(&sQ[rr][pe * EV]) = uq;
      *reinterpret_cast<uint4*>(&sK[rr][pe * EV]) = uk;
    }
#pragma unroll
    for (int x = 0; x < BC * BC / 4 / NT; ++x) {
      const int e = tid + x * NT, rr = (4 * e) / BC, cc = (4 * e) % BC;
      const float4 m = reinterpret_cast<const float4*>(R + REC_M)[e];
      const float4 pg = reinterpret_cast<const float4*>(R + REC_PG)[e];
      sM[rr][cc] = m.x; sM[rr][cc + 1] = m.y; sM[rr][cc + 2] = m.z; sM[rr][cc + 3] = m.w;
      sPG[rr][cc] = pg.x; sPG[rr][cc + 1] = pg.y; sPG[rr][cc + 2] = pg.z; sPG[rr][cc + 3] = pg.w;
    }
  }
  if (tid < BC) {
    sg[tid] = R[REC_G + tid];
    sb[tid] = R[REC_B + tid];
    sden[tid] = R[REC_D + tid];
  }
  const int r = tid / TPRW, qd = tid % TPRW, j0 = qd * CPTG, i0 = qd * IPT;
  const int sd = tid / TPR, sj = (tid % TPR) * EPT;
  // Rank-16 updates on the fp32 MFMA: wave w owns row tile mt of the chunk and column tiles
  // nt = w / 4 + 2u of dP, dT' (64 x 64) and of dQ, dK (64 x DK).
  constexpr int NTW = DK / 32;
  const int lane = tid & 63, wv = tid >> 6, gq = lane >> 4, ln = lane & 15, mt = wv & 3, nt0 = wv >> 2;
  v4f mP[2], mT[2], mQ[NTW], mK[NTW];
  for (int u = 0; u < 2; ++u) mP[u] = mT[u] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int u = 0; u < NTW; ++u) mQ[u] = mK[u] = v4f{0.f, 0.f, 0.f, 0.f};
  float dwp = 0.f, degp = 0.f, gamp = 0.f;
  float dwp4[4] = {0.f, 0.f, 0.f, 0.f}, degp4[4] = {0.f, 0.f, 0.f, 0.f};  // bf16 inputs: rows 4 gq + e
  __syncthreads();
  const float gC = sg[BC - 1];
  const float egr = expf(sg[r]), wr = expf(gC - sg[r]);
  if (tid < BC) {
    seg[tid] = expf(sg[tid]);
    sww[tid] = expf(gC - sg[tid]);
  }

  // the next column block's S0, dS1, V and dO are loaded into registers while this one is
  // computed
  constexpr int VPT = BC * NJG / NT;
  // V and dO are fetched without a branch (a clamped token past T, zeroed when staged): a load
  // inside a conditional is waited for inside it, which would serialize the prefetch
  using VE = typename LdsIn<MODE>::type;
  float pS[EPT], pD[EPT], pO[VPT];
  VE pV[VPT];
  auto fetch = [&](int jb) {
    if constexpr (EPT % 4 == 0) {
#pragma unroll
      for (int e = 0; e < EPT; e += 4) {
        const v4f xs = *reinterpret_cast<const v4f*>(S0 + sd * DV + jb + sj + e);
        const v4f xd = *reinterpret_cast<const v4f*>(D1 + sd * DV + jb + sj + e);
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          pS[e + z] = xs[z];
          pD[e + z] = xd[z];
        }
      }
    } else {
      for (int e = 0; e < EPT; ++e) {
        pS[e] = S0[sd * DV + jb + sj + e];
        pD[e] = D1[sd * DV + jb + sj + e];
      }
    }
    for (int x = 0; x < VPT; ++x) {
      const int e = tid + x * NT, rr = e / NJG, j = e % NJG, t = c * BC + rr;
      const size_t o = tok(b, t < T ? t : T - 1, T, H, h) * DV + jb + j;
      pV[x] = static_cast<const VE*>(v)[o];
      pO[x] = dout[o];
    }
  };
  fetch(0);
  for (int jb = 0; jb < DV; jb += NJG) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      cS[(sj + e) * SP + sd] = pS[e];
      cD[(sj + e) * SP + sd] = pD[e];
    }
    for (int x = 0; x < VPT; ++x) {
      const int e = tid + x * NT, rr = e / NJG, j = e % NJG;
      const bool in = c * BC + rr < T;
      cX[j * RP + rr] = in ? lds_f(pV[x]) : 0.f;
      cO[j * RP + rr] = in ? pO[x] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) gamp = fmaf(pS[e], pD[e], gamp);
    if (jb + NJG < DV) fetch(jb + NJG);
    __syncthreads();
    if constexpr (FUSED) {
      // Wave wv owns tile (row tile mt, column tile nt0) of the block in every product below:
      // lane l holds rows 16 mt + 4 (l / 16) + e of block column jc = 16 nt0 + l % 16, so the
      // elementwise steps and the per-row sums run in the MFMA epilogues.
      const int row = 16 * mt + ln, jc = 16 * nt0 + ln;
      // K S0, K dS1, Q S0 on the bf16 MFMA: k and q are exact in bf16, the fp32 state columns
      // enter as hi + lo bf16 pairs (two passes per product)
      v4f aks = {0.f, 0.f, 0.f, 0.f}, akd = aks, aqs = aks;
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const int dd = 32 * kb + 8 * gq;
        const bf16x8_t ak = *reinterpret_cast<const bf16x8_t*>(&sK[row][dd]);
        const bf16x8_t aq = *reinterpret_cast<const bf16x8_t*>(&sQ[row][dd]);
        bf16x8_t h8, l8;
        bf16_split8(&cS[jc * SP + dd], h8, l8);
        aks = mfma_bf16(ak, l8, mfma_bf16(ak, h8, aks));
        aqs = mfma_bf16(aq, l8, mfma_bf16(aq, h8, aqs));
        bf16_split8(&cD[jc * SP + dd], h8, l8);
        akd = mfma_bf16(ak, l8, mfma_bf16(ak, h8, akd));
      }
      // X = V - e^g . (K S0) in place; dO . (Q S0) into the row sums of dg
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int x = jc * RP + 16 * mt + 4 * gq + e;
        cX[x] = fmaf(-seg[16 * mt + 4 * gq + e], aks[e], cX[x]);
        degp4[e] = fmaf(cO[x], aqs[e], degp4[e]);
      }
      __syncthreads();
      // U = Minv (beta . X) and P^T dO on the fp32 MFMA; dU = w . (K dS1) + P^T dO
      v4f au = {0.f, 0.f, 0.f, 0.f}, ap = au;
#pragma unroll 4
      for (int kk = 0; kk < BC / 4; ++kk) {
        const int i = 4 * kk + gq;
        au = mfma4(sM[row][i] * sb[i], cX[jc * RP + i], au);
        ap = mfma4(i >= row ? sPG[i][row] : 0.f, cO[jc * RP + i], ap);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = 16 * mt + 4 * gq + e;
        cU[jc * RP + rr] = au[e];
        cDU[jc * RP + rr] = fmaf(sww[rr], akd[e], ap[e]);
        dwp4[e] = fmaf(au[e], akd[e], dwp4[e]);
      }
      __syncthreads();
      // dX = diag(beta) Minv^T dU, which is also dV
      v4f ax = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int kk = 0; kk < BC / 4; ++kk) {
        const int i = 4 * kk + gq;
        ax = mfma4(sM[i][row], cDU[jc * RP + i], ax);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = 16 * mt + 4 * gq + e, t = c * BC + rr;
        const float dx = sb[rr] * ax[e];
        cDX[jc * RP + rr] = dx;
        degp4[e] = fmaf(-dx, aks[e], degp4[e]);
        if (t < T) dv[tok(b, t, T, H, h) * DV + jb + jc] = dx;
      }
      __syncthreads();
    } else {
      // one column tile: K S0, K dS1 (waves 0-3) and Q S0 (waves 4-7) for row tile mt on the fp32
      // MFMA, parked in the U, dU and dX blocks, which this column block has not written yet; the
      // elementwise steps by each element's owner thread
      const int row = 16 * mt + ln;
      if (wv < 4) {
        v4f aks = {0.f, 0.f, 0.f, 0.f}, akd = aks;
#pragma unroll 8
        for (int kk = 0; kk < DK / 4; ++kk) {
          const int d = 4 * kk + gq;
          const float a = lds_f(sK[row][d]);
          aks = mfma4(a, cS[ln * SP + d], aks);
          akd = mfma4(a, cD[ln * SP + d], akd);
        }
        for (int e = 0; e < 4; ++e) {
          cU[ln * RP + 16 * mt + 4 * gq + e] = aks[e];
          cDU[ln * RP + 16 * mt + 4 * gq + e] = akd[e];
        }
      } else {
        v4f aqs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int kk = 0; kk < DK / 4; ++kk) {
          const int d = 4 * kk + gq;
          aqs = mfma4(lds_f(sQ[row][d]), cS[ln * SP + d], aqs);
        }
        for (int e = 0; e < 4; ++e) cDX[ln * RP + 16 * mt + 4 * gq + e] = aqs[e];
      }
      __syncthreads();
      float ks[CPTG], kd[CPTG];
      for (int jj = 0; jj < CPTG; ++jj) {
        ks[jj] = cU[(j0 + jj) * RP + r];
        kd[jj] = cDU[(j0 + jj) * RP + r];
        degp = fmaf(cO[(j0 + jj) * RP + r], cDX[(j0 + jj) * RP + r], degp);
      }
      for (int jj = 0; jj < CPTG; ++jj) cX[(j0 + jj) * RP + r] -= egr * ks[jj];  // X
      __syncthreads();
      // U = Minv (beta . X) (waves 0-3) and P^T dO (waves 4-7) for row tile mt
      {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        if (wv < 4) {
#pragma unroll 4
          for (int kk = 0; kk < BC / 4; ++kk) {
            const int i = 4 * kk + gq;
            acc = mfma4(sM[row][i] * sb[i], cX[ln * RP + i], acc);
          }
          for (int e = 0; e < 4; ++e) cU[ln * RP + 16 * mt + 4 * gq + e] = acc[e];
        } else {
#pragma unroll 4
          for (int kk = 0; kk < BC / 4; ++kk) {
            const int i = 4 * kk + gq;
            acc = mfma4(i >= row ? sPG[i][row] : 0.f, cO[ln * RP + i], acc);
          }
          for (int e = 0; e < 4; ++e) cDU[ln * RP + 16 * mt + 4 * gq + e] = acc[e];
        }
      }
      __syncthreads();
      // dU = w . (K dS1) + P^T dO
      for (int jj = 0; jj < CPTG; ++jj) {
        const float u = cU[(j0 + jj) * RP + r];
        cDU[(j0 + jj) * RP + r] = fmaf(wr, kd[jj], cDU[(j0 + jj) * RP + r]);
        dwp = fmaf(u, kd[jj], dwp);
      }
      __syncthreads();
      // dX = diag(beta) Minv^T dU (waves 0-3), which is also dV
      if (wv < 4) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int kk = 0; kk < BC / 4; ++kk) {
          const int i = 4 * kk + gq;
          acc = mfma4(sM[i][row], cDU[ln * RP + i], acc);
        }
        for (int e = 0; e < 4; ++e) {
          const int rr = 16 * mt + 4 * gq + e;
          cDX[ln * RP + rr] = sb[rr] * acc[e];
        }
      }
      __syncthreads();
      for (int jj = 0; jj < CPTG; ++jj) {
        const float dx = cDX[(j0 + jj) * RP + r];
        degp = fmaf(-dx, ks[jj], degp);
        const int t = c * BC + r;
        if (t < T) dv[tok(b, t, T, H, h) * DV + jb + j0 + jj] = dx;
      }
    }
    // dP += dO U^T, dT' += dU X^T, dQ += e^g . (dO S0^T), dK += w . (U dS1^T) - e^g . (dX S0^T)
    {
      const int row = 16 * mt + ln;
      const float eg_row = seg[row], w_row = sww[row];
#pragma unroll
      for (int kk = 0; kk < NJG / 4; ++kk) {
        const int jk = 4 * kk + gq;
        const float o = cO[jk * RP + row], du = cDU[jk * RP + row];
        const float ao = eg_row * o, au = w_row * cU[jk * RP + row], ax = -eg_row * cDX[jk * RP + row];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int col = 16 * (nt0 + 2 * u) + ln;
          mP[u] = mfma4(o, cU[jk * RP + col], mP[u]);
          mT[u] = mfma4(du, cX[jk * RP + col], mT[u]);
        }
#pragma unroll
        for (int u = 0; u < NTW; ++u) {
          const int col = 16 * (nt0 + 2 * u) + ln;
          const float s0 = cS[jk * SP + col];
          mQ[u] = mfma4(ao, s0, mQ[u]);
          mK[u] = mfma4(ax, s0, mfma4(au, cD[jk * SP + col], mK[u]));
        }
      }
    }
    __syncthreads();
  }

  if constexpr (FUSED) {
    // row sums: over the 16 lanes of a row group, then (in the per-token step) over the two
    // column-tile waves of the row tile
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = dwp4[e], y = degp4[e];
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        x += __shfl_xor(x, m);
        y += __shfl_xor(y, m);
      }
      if (ln == 0) {
        const int rr = 16 * mt + 4 * gq + e;
        (nt0 == 0 ? sdw : sdw2)[rr] = x;
        (nt0 == 0 ? sdeg : sdeg2)[rr] = y;
      }
    }
  } else {
    const float dw = quad_sum(dwp), deg = quad_sum(degp);
    if (qd == 0) {
      sdw[r] = dw;
      sdeg[r] = deg;
    }
  }
  gamp = quad_sum(gamp);
  if (qd == 0) sgp[r] = gamp;
  // dP into m1 and dT' into m2 from the MFMA tiles
  for (int u = 0; u < 2; ++u)
    for (int e = 0; e < 4; ++e) {
      const int rr = 16 * mt + 4 * gq + e, col = 16 * (nt0 + 2 * u) + ln;
      m1[rr * MP + col] = mP[u][e];
      m2[rr * MP + col] = mT[u][e];
    }
  __syncthreads();
  // dQK = tril_incl(dP) . Dl;  dDl . Dl collects dP . P (and below dA . A)
  float ddl[IPT], dqk[IPT];
  for (int ii = 0; ii < IPT; ++ii) {
    const int i = i0 + ii;
    const bool low = i <= r;
    const float dp = m1[r * MP + i];
    dqk[ii] = low ? dp * expf(sg[r] - sg[i]) : 0.f;
    ddl[ii] = low ? dp * sPG[r][i] : 0.f;
  }
  __syncthreads();
  for (int ii = 0; ii < IPT; ++ii) m1[r * MP + i0 + ii] = dqk[ii];
  __syncthreads();
  // The 64 x 64 products below run on the fp32 MFMA, wave wv on row tile mt and column tiles
  // nt0 + 2u (a K = 4 step: lane l supplies A[row 16 mt + l % 16][k = 4 s + l / 16] and
  // B[k][col]; the result's rows 16 mt + 4 (l / 16) + e, column col sit in lane l's acc[e]).
  const int arow = 16 * mt + ln;
  // dQ += dQK K and dK += dQK^T Q, into the dQ and dK tiles
#pragma unroll 4
  for (int s4 = 0; s4 < BC / 4; ++s4) {
    const int kk = 4 * s4 + gq;
    const float a = m1[arow * MP + kk], at = m1[kk * MP + arow];
#pragma unroll
    for (int u = 0; u < NTW; ++u) {
      const int col = 16 * (nt0 + 2 * u) + ln;
      mQ[u] = mfma4(a, lds_f(sK[kk][col]), mQ[u]);
      mK[u] = mfma4(at, lds_f(sQ[kk][col]), mK[u]);
    }
  }
  // W1 = Minv^T dT' diag(beta): Minv^T[row][k] = Minv[k][row] is zero for k < row, so the
  // contraction starts at this row tile. dbeta_i (T' = Minv diag(beta)) is the diagonal of
  // Minv^T dT' before the scaling.
  v4f w1t[2];
  for (int u = 0; u < 2; ++u) w1t[u] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s4 = 4 * mt; s4 < BC / 4; ++s4) {
    const int kk = 4 * s4 + gq;
    const float a = sM[kk][arow];
#pragma unroll
    for (int u = 0; u < 2; ++u) w1t[u] = mfma4(a, m2[kk * MP + 16 * (nt0 + 2 * u) + ln], w1t[u]);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (nt0 + 2 * u == mt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * gq + e == ln) sdb[arow] = w1t[u][e];
  __syncthreads();  // every read of dQK (m1) and dT' (m2) is done
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int col = 16 * (nt0 + 2 * u) + ln;
#pragma unroll
    for (int e = 0; e < 4; ++e) m1[(16 * mt + 4 * gq + e) * MP + col] = w1t[u][e] * sb[col];
  }
  __syncthreads();
  // dA = -W1 Minv^T (used below on the strict lower triangle) into m2
  {
    v4f dat[2];
    for (int u = 0; u < 2; ++u) dat[u] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s4 = 0; s4 < BC / 4; ++s4) {
      const int kk = 4 * s4 + gq;
      const float a = m1[arow * MP + kk];
#pragma unroll
      for (int u = 0; u < 2; ++u) dat[u] = mfma4(a, sM[16 * (nt0 + 2 * u) + ln][kk], dat[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int col = 16 * (nt0 + 2 * u) + ln;
#pragma unroll
      for (int e = 0; e < 4; ++e) m2[(16 * mt + 4 * gq + e) * MP + col] = -dat[u][e];
    }
  }
  __syncthreads();
  // A = beta_r Dl G gives dbeta, dDl and dG
  float dbp = 0.f;
  float dG[IPT];
  for (int ii = 0; ii < IPT; ++ii) {
    const int i = i0 + ii;
    dG[ii] = 0.f;
    if (i < r) {
      const float da = m2[r * MP + i], dl = expf(sg[r] - sg[i]), G = sPG[i][r];
      dbp = fmaf(da * dl, G, dbp);
      ddl[ii] = fmaf(da * sb[r] * dl, G, ddl[ii]);
      dG[ii] = da * sb[r] * dl;
    }
  }
  dbp = quad_sum(dbp);
  __syncthreads();  // every thread's reads of dA (m2) are done
  for (int ii = 0; ii < IPT; ++ii) {
    m2[r * MP + i0 + ii] = dG[ii];
    m1[r * MP + i0 + ii] = ddl[ii];
  }
  float rs = 0.f;
  for (int ii = 0; ii < IPT; ++ii) rs += ddl[ii];
  rs = quad_sum(rs);
  if (qd == 0) {
    srow[r] = rs;
    sdb[r] += dbp;
  }
  __syncthreads();
  // dK += (dG + dG^T) K, into the dK tiles
#pragma unroll 4
  for (int s4 = 0; s4 < BC / 4; ++s4) {
    const int kk = 4 * s4 + gq;
    const float a = m2[arow * MP + kk] + m2[kk * MP + arow];
#pragma unroll
    for (int u = 0; u < NTW; ++u) mK[u] = mfma4(a, lds_f(sK[kk][16 * (nt0 + 2 * u) + ln]), mK[u]);
  }
  if (tid < BC) {  // one wave: lane i is token i of the chunk
    const int i = tid, t = c * BC + i;
    float cs = 0.f;
    for (int j = 0; j < BC; ++j) cs += m1[j * MP + i];
    const float sdwi = FUSED ? sdw[i] + sdw2[i] : sdw[i];
    const float sdegi = FUSED ? sdeg[i] + sdeg2[i] : sdeg[i];
    const float dww = sdwi * sww[i];
    float tot = dww;  // sum over the chunk of dw . w, across the wave
    for (int m = 1; m < BC; m <<= 1) tot += __shfl_xor(tot, m);
    float dg = srow[i] - cs + sdegi * seg[i] - dww;
    float gam = sgp[i];  // <dS1, S0>, summed across the wave in a fixed order
    for (int m = 1; m < BC; m <<= 1) gam += __shfl_xor(gam, m);
    if (i == BC - 1) dg += tot + gam * expf(gC);
    // dlog_alpha: the sum of dg over this token and the later ones in the chunk (a suffix scan)
    float sfx = dg;
    for (int m = 1; m < BC; m <<= 1) {
      const float o = __shfl_down(sfx, m);
      if (i + m < BC) sfx += o;
    }
    if (t < T) dla[tok(b, t, T, H, h)] = sfx;
    const float db = sdb[i], den = sden[i];
    const float et = t < T ? eta[tok(b, t, T, H, h)] : 0.f;
    float de = db, kc = 0.f;
    if (!direct) {
      de = den != 0.f ? db / den : 0.f;
      kc = den != 0.f ? -2.f * db * et / (den * den) : 0.f;
    }
    skc[i] = kc;
    if (t < T) deta[tok(b, t, T, H, h)] = de;
  }
  __syncthreads();
  // dQ and dK straight from the MFMA tiles: lane l holds rows 16 mt + 4 (l / 16) + e of column
  // 16 nt + l % 16, so each store covers 64 contiguous bytes of four rows
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int rr = 16 * mt + 4 * gq + e, t = c * BC + rr;
    if (t < T) {
      const size_t o = tok(b, t, T, H, h) * DK;
      const float kc = skc[rr];
#pragma unroll
      for (int u = 0; u < NTW; ++u) {
        const int col = 16 * (nt0 + 2 * u) + ln;
        dq[o + col] = mQ[u][e];
        dk[o + col] = fmaf(kc, lds_f(sK[rr][col]), mK[u][e]);
      }
    }
  }
}

// The reverse walk's fold over segments (the segmented backward of long sequences). The forward
// walk over segment s takes S to M_s S + N_s, so the gradient at its start is M_s^T G_s + D_s,
// with G_s the gradient at its end and D_s what the reverse walk over the segment gives from a
// zero end gradient. G of the last segment is the end state's gradient (zero if null); the fold
// writes G_s for every segment, last to first. maps holds [M_s | N_s] (dk x (dk + dv)) for
// segments 1 .. segs - 1, D holds D_s at slot (bh, s). One workgroup per (16 columns, head), the
// carried columns transposed in LDS, the products on the fp32 MFMA.
template <int DK>
__global__ __launch_bounds__(256) void bwd_rev_fold_kernel(const float* __restrict__ maps, const float* __restrict__ D,
                                                           const float* __restrict__ dfin, float* __restrict__ gend,
                                                           int DV, int segs) {
  constexpr int XP = DK + 4;  // padded pitch of X^T rows (floats)
  __shared__ __align__(16) float XT[2][16 * XP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, gq = lane >> 4, ln = lane & 15;
  const int c0 = blockIdx.x * 16, bh = blockIdx.y;
  const int LDM = DK + DV;
  for (int o = tid; o < DK * 16; o += 256) {
    const int r = o >> 4, j = o & 15;
    const float x = dfin ? dfin[static_cast<size_t>(bh) * DK * DV + r * DV + c0 + j] : 0.f;
    XT[(segs - 1) & 1][j * XP + r] = x;
    gend[(static_cast<size_t>(bh) * segs + segs - 1) * DK * DV + r * DV + c0 + j] = x;
  }
  __syncthreads();
  for (int s = segs - 1; s >= 1; --s) {
    const float* M = maps + (static_cast<size_t>(bh) * (segs - 1) + (s - 1)) * DK * LDM;
    const float* Ds = D + (static_cast<size_t>(bh) * segs + s) * DK * DV;
    const float* X = XT[s & 1];
    float* Xn = XT[(s - 1) & 1];
    float* out = gend + (static_cast<size_t>(bh) * segs + s - 1) * DK * DV;
#pragma unroll
    for (int u = 0; u < DK / 64; ++u) {
      const int mt = w + 4 * u;
      v4f acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = Ds[static_cast<size_t>(16 * mt + 4 * gq + i) * DV + c0 + ln];
#pragma unroll 4
      for (int kk = 0; kk < DK / 16; ++kk) {
        const v4f b4 = *reinterpret_cast<const v4f*>(X + ln * XP + 16 * kk + 4 * gq);
#pragma unroll
        for (int q = 0; q < 4; ++q)  // M^T[16 mt + ln][k] = M[k][16 mt + ln]
          acc = mfma4(M[static_cast<size_t>(16 * kk + 4 * gq + q) * LDM + 16 * mt + ln], b4[q], acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) out[static_cast<size_t>(16 * mt + 4 * gq + i) * DV + c0 + ln] = acc[i];
      *reinterpret_cast<v4f*>(Xn + ln * XP + 16 * mt + 4 * gq) = acc;
    }
    __syncthreads();
  }
}

// Waves per walk workgroup (one workgroup per head, segment and 16 x waves state columns): the
// count whose workgroups take the fewest rounds of one per CU, the smallest count on a tie (the
// chains are latency-bound, so more CUs with fewer waves each go faster); two at least for
// dk = 256, where one wave's registers cannot hold a chunk's prefetched rows.
int walk_waves(const BwdArgs& a, int nseg) {
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    ncu = 256;
  const long long units = static_cast<long long>(a.B) * a.H * nseg;
  int best = 4;
  long long best_rounds = -1;
  for (int nw = a.dk == 256 ? 2 : 1; nw <= 4; nw *= 2) {
    const long long rounds = ((a.dv / (16 * nw)) * units + ncu - 1) / ncu;
    if (best_rounds < 0 || rounds < best_rounds) {
      best = nw;
      best_rounds = rounds;
    }
  }
  return best;
}

template <int MODE, int DK, bool REV, int NW>
hipError_t launch_walk(const BwdArgs& a, const WalkSegs& g, hipStream_t stream) {
  const dim3 grid(a.dv / (16 * NW), a.B * a.H * g.nseg), blk(64 * NW);
  if constexpr (REV)
    return launch_kernel(bwd_walk_kernel<MODE, DK, true, NW>, grid, blk, stream, a.k, a.vt, a.rec, g.sin, a.T, a.H,
                         a.dv, a.nc, a.dstates, g.slast, g.seg_chunks, g.nseg, g.seg0, g.sin_segs, g.slast_segs,
                         g.dump);
  else
    return launch_kernel(bwd_walk_kernel<MODE, DK, false, NW>, grid, blk, stream, a.k, a.v, a.rec, g.sin, a.T, a.H,
                         a.dv, a.nc, a.states, g.slast, g.seg_chunks, g.nseg, g.seg0, g.sin_segs, g.slast_segs,
                         g.dump);
}

template <int MODE, int DK, bool REV>
hipError_t launch_walk_any(const BwdArgs& a, const WalkSegs& g, hipStream_t stream) {
  const int nw = walk_waves(a, g.nseg);
  if (nw == 4) return launch_walk<MODE, DK, REV, 4>(a, g, stream);
  if (nw == 2) return launch_walk<MODE, DK, REV, 2>(a, g, stream);
  if constexpr (DK == 256) return hipErrorInvalidValue;
  else return launch_walk<MODE, DK, REV, 1>(a, g, stream);
}

template <int MODE, int DK>
hipError_t launch_bwd_t(const BwdArgs& a, int stage, hipStream_t stream) {
  const dim3 blk(BT);
  const int bh = a.B * a.H;
  switch (stage) {
    case 0:
      return launch_kernel(bwd_prep_kernel<MODE, DK>, dim3(a.nc, bh), blk, stream, a.q, a.k, a.log_alpha, a.eta, a.eps,
                           a.direct, a.T, a.H, a.nc, a.rec);
    case 1:
      return launch_walk_any<MODE, DK, false>(a, WalkSegs{a.nc, 1, 0, a.init, 1, nullptr, 1, 1}, stream);
    case 2:
      return launch_kernel(bwd_dprep_kernel<MODE, DK>, dim3(a.nc, bh), dim3(64 * (a.dv / 16)), stream, a.q, a.dout, a.rec, a.T, a.H,
                           a.dv, a.nc, a.vt, a.dstates);
    case 3:
      return launch_walk_any<MODE, DK, true>(a, WalkSegs{a.nc, 1, 0, a.dfin, 1, a.ginit, 1, 1}, stream);
    default:
      return launch_kernel(bwd_grads_kernel<MODE, DK>, dim3(a.nc, bh), dim3(NT), stream, a.q, a.k, a.v, a.eta, a.dout,
                           a.rec, a.states, a.dstates, a.direct, a.T, a.H, a.dv, a.nc, a.gq, a.gk, a.gv, a.gla,
                           a.geta);
  }
}

}  // namespace

size_t bwd_record_floats() { return RECF; }

size_t bwd_workspace_bytes(int B, int T, int H, int dk, int dv) {
  const size_t nch = static_cast<size_t>(B) * H * ((T + BC - 1) / BC);
  return nch * (RECF + 2 * static_cast<size_t>(dk) * dv + static_cast<size_t>(BC) * dv) * sizeof(float);
}

hipError_t launch_bwd_walk_segs(int mode, const BwdArgs& a, bool rev, const WalkSegs& g, hipStream_t stream) {
  if (mode == 0) {
    if (a.dk == 64) return rev ? launch_walk_any<0, 64, true>(a, g, stream) : launch_walk_any<0, 64, false>(a, g, stream);
    if (a.dk == 128) return rev ? launch_walk_any<0, 128, true>(a, g, stream) : launch_walk_any<0, 128, false>(a, g, stream);
    if (a.dk == 256) return rev ? launch_walk_any<0, 256, true>(a, g, stream) : launch_walk_any<0, 256, false>(a, g, stream);
    return hipErrorInvalidValue;
  }
  if (a.dk == 64) return rev ? launch_walk_any<1, 64, true>(a, g, stream) : launch_walk_any<1, 64, false>(a, g, stream);
  if (a.dk == 128) return rev ? launch_walk_any<1, 128, true>(a, g, stream) : launch_walk_any<1, 128, false>(a, g, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_rev_fold(const BwdArgs& a, const float* maps, const float* D, float* gend, int segs,
                               hipStream_t stream) {
  const dim3 grid(a.dv / 16, a.B * a.H), blk(256);
  switch (a.dk) {
    case 64: return launch_kernel(bwd_rev_fold_kernel<64>, grid, blk, stream, maps, D, a.dfin, gend, a.dv, segs);
    case 128: return launch_kernel(bwd_rev_fold_kernel<128>, grid, blk, stream, maps, D, a.dfin, gend, a.dv, segs);
    case 256: return launch_kernel(bwd_rev_fold_kernel<256>, grid, blk, stream, maps, D, a.dfin, gend, a.dv, segs);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(int mode, const BwdArgs& a, int stage, hipStream_t stream) {
  if (mode == 0) {
    if (a.dk == 256) return launch_bwd_t<0, 256>(a, stage, stream);
    return a.dk == 64 ? launch_bwd_t<0, 64>(a, stage, stream) : launch_bwd_t<0, 128>(a, stage, stream);
  }
  return a.dk == 64 ? launch_bwd_t<1, 64>(a, stage, stream) : launch_bwd_t<1, 128>(a, stage, stream);
}

}  // namespace kla
