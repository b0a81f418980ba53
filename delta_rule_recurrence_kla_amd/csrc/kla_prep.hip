// Chunk prep kernel of the chunkwise KLA forward.
//
// For each 64-token chunk of one (batch, head) it computes, in this order:
//   n_r    = ||k_r||^2                            (fp32)
//   beta_r = eta_r / (n_r + eps)                  Kaczmarz step size: KLA page, "KLA update rule"
//   g_r    = sum_{j<=r} log_alpha_j               chunk-local decay exponents
//   A      = strict_lower(beta_r e^{g_r-g_i} (k_r . k_i))
//   T      = (I + A)^-1                           blocked fp32 inverse of a unit lower-triangular matrix
//   T'     = T diag(beta)
//   P      = (q_r . k_i) e^{g_r-g_i} for i <= r   (diagonal included: o_t reads S_t after the write)
// and stores T', P, e^{g_r} and e^{g_C-g_r} as the chunk's record.
//
// Why this is the chunk's whole job: writing u_i = beta_i e_i and unrolling the
// per-token update of the KLA page ("KLA update rule": S_t = S~ + beta_t k_t e_t^T,
// e_t = v_t - S~^T k_t, S~ = alpha_t S_{t-1}) inside a chunk that starts from S_0 gives
//   (I + A) U = diag(beta) (V - diag(e^g) K S_0),   so U = T' (V - diag(e^g) K S_0),
// the chunkwise solver that the KLA page ("Implementation") keeps from Gated DeltaNet
// with only B = Diag(beta_1..beta_C) changed. Everything above depends on the chunk's
// own inputs only, so all chunks of all heads run in parallel.
//
// Tokens past T in the last chunk enter as identity steps: k = q = 0, log_alpha = 0,
// eta = 0, so their rows and columns of T' and P are zero.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

template <int MODE, int DK>
__global__ __launch_bounds__(256) void prep_kernel(const typename Tr<MODE>::in_t* __restrict__ q,
                                                   const typename Tr<MODE>::in_t* __restrict__ k,
                                                   const float* __restrict__ log_alpha,
                                                   const float* __restrict__ eta, float eps,
                                                   uint8_t* __restrict__ rec, int T, int H, int nc) {
  using TR = Tr<MODE>;
  using in_t = typename TR::in_t;
  constexpr int VEC = 16 / static_cast<int>(sizeof(in_t));  // elements per 16-byte access
  constexpr int LD = DK + VEC;  // row pitch in elements: a 16-byte pad keeps rows 16-byte aligned
  constexpr int LPR = DK / VEC;                             // lanes per row
  constexpr int RPI = 256 / LPR;                            // rows per iteration
  static_assert(LPR <= 64 && 256 % LPR == 0 && CHUNK % RPI == 0, "load shape");

  __shared__ __align__(16) in_t sK[CHUNK * LD];
  __shared__ __align__(16) in_t sQ[CHUNK * LD];
  __shared__ float sA[CHUNK][CHUNK + 1];
  __shared__ float sT[CHUNK][CHUNK + 1];
  __shared__ float sY[3][16][17];
  __shared__ float sg[CHUNK], sbeta[CHUNK], snk[CHUNK];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gq = lane >> 4, ln = lane & 15;
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int t0 = c * CHUNK;
  uint8_t* R = rec + (static_cast<size_t>(bh) * nc + c) * REC_BYTES;

  // 1. chunk of K and Q into LDS (zero past T), and key norms
#pragma unroll
  for (int it = 0; it < CHUNK / RPI; ++it) {
    const int r = it * RPI + tid / LPR;
    const int cv = (tid % LPR) * VEC;
    const int t = t0 + r;
    uint4 kv = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
    if (t < T) {
      const size_t off = ((static_cast<size_t>(b) * T + t) * H + h) * DK + cv;
      kv = *reinterpret_cast<const uint4*>(k + off);
      qv = *reinterpret_cast<const uint4*>(q + off);
    }
    *reinterpret_cast<uint4*>(sK + r * LD + cv) = kv;
    *reinterpret_cast<uint4*>(sQ + r * LD + cv) = qv;
    const in_t* e = reinterpret_cast<const in_t*>(&kv);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const float x = TR::to_f32(e[j]);
      s += x * x;
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
    if (tid % LPR == 0) snk[r] = s;
  }
  __syncthreads();

  // 2. gates: lane = token of the chunk
  if (w == 0) {
    const int t = t0 + lane;
    float la = 0.f, et = 0.f;
    if (t < T) {
      const size_t gi = (static_cast<size_t>(b) * T + t) * H + h;
      la = log_alpha[gi];
      et = eta[gi];
    }
    float g = la;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(g, o);
      if (lane >= o) g += y;
    }
    const float denom = snk[lane] + eps;
    sg[lane] = g;
    sbeta[lane] = denom != 0.f ? et / denom : 0.f;
    const float gC = __shfl(g, 63);
    reinterpret_cast<float*>(R + REC_EG_OFF)[lane] = expf(g);
    reinterpret_cast<float*>(R + REC_EGC_OFF)[lane] = expf(gC - g);
  }
  __syncthreads();

  // 3. K K^T and Q K^T, one 16-row strip per wave, lower-triangular tiles only
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    f32x4 ag = zero4(), ap = zero4();
    if (nt <= w) {
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const auto xk = TR::ldx(sK, LD, 16 * w, 32 * kb, lane);
        const auto xq = TR::ldx(sQ, LD, 16 * w, 32 * kb, lane);
        const auto yk = TR::ldx(sK, LD, 16 * nt, 32 * kb, lane);
        ag = TR::mma_xx(ag, xk, yk);
        ap = TR::mma_xx(ap, xq, yk);
      }
    }
    const int cc = 16 * nt + ln;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * gq + i;
      const float dec = cc <= r ? expf(sg[r] - sg[cc]) : 0.f;
      sA[r][cc] = cc < r ? sbeta[r] * dec * ag[i] : 0.f;
      const float pv = dec * ap[i];
      if constexpr (MODE == MODE_BF16) {
        const __bf16 hi = static_cast<__bf16>(pv);
        const __bf16 lo = static_cast<__bf16>(pv - static_cast<float>(hi));
        __bf16* row = reinterpret_cast<__bf16*>(R + REC_P_OFF + r * 256);
        row[cc] = hi;
        row[64 + cc] = lo;
      } else {
        reinterpret_cast<float*>(R + REC_P_OFF + r * 256)[cc] = pv;
      }
    }
  }
  __syncthreads();

  // 4a. inverses of the four 16x16 diagonal blocks of I + A, by forward substitution;
  //     lane (blk, j) produces column j of block blk
  if (w == 0) {
    const int blk = lane >> 4, j = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = r == j ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) s -= sA[16 * blk + r][16 * blk + i] * x[i];
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[16 * blk + r][16 * blk + j] = x[r];
  }
  __syncthreads();

  // 4b. off-diagonal blocks by distance from the diagonal:
  //     T_IJ = -T_II * sum_{C=J}^{I-1} A_IC T_CJ
#pragma unroll
  for (int d = 1; d <= 3; ++d) {
    const int nblk = 4 - d;
    for (int o = tid; o < nblk * 256; o += 256) {
      const int bi = o >> 8, r = (o >> 4) & 15, s = o & 15;
      const int I = d + bi, J = bi;
      float y = 0.f;
      for (int C = J; C < I; ++C) {
#pragma unroll
        for (int u = 0; u < 16; ++u) y += sA[16 * I + r][16 * C + u] * sT[16 * C + u][16 * J + s];
      }
      sY[bi][r][s] = y;
    }
    __syncthreads();
    for (int o = tid; o < nblk * 256; o += 256) {
      const int bi = o >> 8, r = (o >> 4) & 15, s = o & 15;
      const int I = d + bi, J = bi;
      float t = 0.f;
      for (int u = 0; u <= r; ++u) t += sT[16 * I + r][16 * I + u] * sY[bi][u][s];
      sT[16 * I + r][16 * J + s] = -t;
    }
    __syncthreads();
  }

  // 5. T' = T diag(beta), lower triangle incl. diagonal; 16 columns per thread
  {
    const int r = tid >> 2, c0 = (tid & 3) * 16;
    float tv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int cc = c0 + j;
      tv[j] = cc <= r ? sT[r][cc] * sbeta[cc] : 0.f;
    }
    if constexpr (MODE == MODE_BF16) {
      union {
        uint4 u[2];
        __bf16 e[16];
      } hi, lo;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        hi.e[j] = static_cast<__bf16>(tv[j]);
        lo.e[j] = static_cast<__bf16>(tv[j] - static_cast<float>(hi.e[j]));
      }
      uint4* ph = reinterpret_cast<uint4*>(R + REC_T_OFF + r * 256 + 2 * c0);
      uint4* pl = reinterpret_cast<uint4*>(R + REC_T_OFF + r * 256 + 128 + 2 * c0);
      ph[0] = hi.u[0];
      ph[1] = hi.u[1];
      pl[0] = lo.u[0];
      pl[1] = lo.u[1];
    } else {
      float4* p = reinterpret_cast<float4*>(R + REC_T_OFF + r * 256 + 4 * c0);
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = make_float4(tv[4 * j], tv[4 * j + 1], tv[4 * j + 2], tv[4 * j + 3]);
    }
  }
}

template <int MODE, int DK>
static hipError_t launch_prep_t(const Dims& d, const void* q, const void* k, const float* la, const float* eta,
                                float eps, uint8_t* rec, hipStream_t stream) {
  using in_t = typename Tr<MODE>::in_t;
  dim3 grid(d.nc, d.B * d.H);
  hipLaunchKernelGGL((prep_kernel<MODE, DK>), grid, dim3(256), 0, stream, static_cast<const in_t*>(q),
                     static_cast<const in_t*>(k), la, eta, eps, rec, d.T, d.H, d.nc);
  return hipGetLastError();
}

hipError_t launch_prep(int mode, const Dims& d, const void* q, const void* k, const float* log_alpha,
                       const float* eta, float eps, uint8_t* rec, hipStream_t stream) {
  if (mode == MODE_BF16) {
    switch (d.dk) {
      case 64: return launch_prep_t<MODE_BF16, 64>(d, q, k, log_alpha, eta, eps, rec, stream);
      case 128: return launch_prep_t<MODE_BF16, 128>(d, q, k, log_alpha, eta, eps, rec, stream);
      case 256: return launch_prep_t<MODE_BF16, 256>(d, q, k, log_alpha, eta, eps, rec, stream);
    }
  } else {
    switch (d.dk) {
      case 64: return launch_prep_t<MODE_F32, 64>(d, q, k, log_alpha, eta, eps, rec, stream);
      case 128: return launch_prep_t<MODE_F32, 128>(d, q, k, log_alpha, eta, eps, rec, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kla
