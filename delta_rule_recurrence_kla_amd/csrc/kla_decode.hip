// Single-token decode step of KLA for N x H independent states, in place.
//
// Per state (KLA page, "KLA update rule"; the recurrent form keeps a constant-size
// state per head, KLA page "Key contributions" 4):
//   alpha = exp(log_alpha), beta = eta / (||k||^2 + eps)   (beta = 0 if the denominator is 0)
//   (with `direct` set, beta = eta: the learned write strength of the Gated DeltaNet rule the
//   KLA page sets itself against in its "Problem statement")
//   a = S^T k, b = S^T q                  (one pass over S)
//   e = v - alpha a                       residual against the decayed state
//   o = S_new^T q = alpha b + beta (k . q) e
//   S_new = alpha S + beta k e^T          (written back in the same pass)
// S is read once and written once; everything else is a few hundred bytes, so the
// kernel is bound by HBM bandwidth. One workgroup per state: 256 threads, each
// owning 4 adjacent columns (one 16-byte access) of DK / (1024 / DV) rows, so a
// wavefront reads and writes whole 512-byte rows.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

template <int MODE, int DK, int DV>
__global__ __launch_bounds__(256) void decode_kernel(const typename Tr<MODE>::in_t* __restrict__ q,
                                                     const typename Tr<MODE>::in_t* __restrict__ k,
                                                     const typename Tr<MODE>::in_t* __restrict__ v,
                                                     const float* __restrict__ log_alpha,
                                                     const float* __restrict__ eta, float eps, int direct,
                                                     float* __restrict__ state, float* __restrict__ out) {
  using TR = Tr<MODE>;
  constexpr int TPR = DV / 4;     // threads per state row
  constexpr int RPP = 256 / TPR;  // rows per pass
  constexpr int NP = DK / RPP;    // rows per thread
  static_assert(DK % RPP == 0 && DK <= 256, "shape");

  __shared__ float sq[DK], sk[DK];
  __shared__ float4 spa[RPP][TPR], spb[RPP][TPR];
  __shared__ float sred[2][4];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rg = tid / TPR, c4 = tid - rg * TPR;
  const size_t nh = blockIdx.x;
  float* S = state + nh * DK * DV;

  // the state tile of this thread: rows rg, rg + RPP, ...; columns 4*c4 .. 4*c4+3
  float4 s[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) s[p] = *reinterpret_cast<const float4*>(S + static_cast<size_t>(rg + p * RPP) * DV + 4 * c4);

  // q, k as fp32 in LDS, with ||k||^2 and k.q reduced per wave
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

  float4 pa = make_float4(0.f, 0.f, 0.f, 0.f), pb = pa;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const float kr = sk[rg + p * RPP], qr = sq[rg + p * RPP];
    pa.x += s[p].x * kr; pa.y += s[p].y * kr; pa.z += s[p].z * kr; pa.w += s[p].w * kr;
    pb.x += s[p].x * qr; pb.y += s[p].y * qr; pb.z += s[p].z * qr; pb.w += s[p].w * qr;
  }
  spa[rg][c4] = pa;
  spb[rg][c4] = pb;
  __syncthreads();

  float4 A = make_float4(0.f, 0.f, 0.f, 0.f), Bq = A;
#pragma unroll
  for (int g = 0; g < RPP; ++g) {
    const float4 x = spa[g][c4], y = spb[g][c4];
    A.x += x.x; A.y += x.y; A.z += x.z; A.w += x.w;
    Bq.x += y.x; Bq.y += y.y; Bq.z += y.z; Bq.w += y.w;
  }
  const float nk = sred[0][0] + sred[0][1] + sred[0][2] + sred[0][3];
  const float dkq = sred[1][0] + sred[1][1] + sred[1][2] + sred[1][3];
  const float alpha = expf(log_alpha[nh]);
  const float denom = nk + eps;
  const float beta = direct ? eta[nh] : denom != 0.f ? eta[nh] / denom : 0.f;

  float vv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vv[j] = TR::to_f32(v[nh * DV + 4 * c4 + j]);
  float4 e;
  e.x = vv[0] - alpha * A.x; e.y = vv[1] - alpha * A.y; e.z = vv[2] - alpha * A.z; e.w = vv[3] - alpha * A.w;
  if (rg == 0) {
    const float bq = beta * dkq;
    float4 o;
    o.x = alpha * Bq.x + bq * e.x; o.y = alpha * Bq.y + bq * e.y;
    o.z = alpha * Bq.z + bq * e.z; o.w = alpha * Bq.w + bq * e.w;
    *reinterpret_cast<float4*>(out + nh * DV + 4 * c4) = o;
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const float bk = beta * sk[rg + p * RPP];
    float4 x = s[p];
    x.x = alpha * x.x + bk * e.x; x.y = alpha * x.y + bk * e.y;
    x.z = alpha * x.z + bk * e.z; x.w = alpha * x.w + bk * e.w;
    *reinterpret_cast<float4*>(S + static_cast<size_t>(rg + p * RPP) * DV + 4 * c4) = x;
  }
}

template <int MODE, int DK, int DV>
static hipError_t launch_decode_t(int N, int H, const void* q, const void* k, const void* v, const float* la,
                                  const float* eta, float eps, int direct, float* state, float* out,
                                  hipStream_t stream) {
  using in_t = typename Tr<MODE>::in_t;
  return launch_kernel(decode_kernel<MODE, DK, DV>, dim3(N * H), dim3(256), stream, static_cast<const in_t*>(q),
                       static_cast<const in_t*>(k), static_cast<const in_t*>(v), la, eta, eps, direct, state, out);
}

template <int MODE>
static hipError_t dispatch_decode(int N, int H, int dk, int dv, const void* q, const void* k, const void* v,
                                  const float* la, const float* eta, float eps, int direct, float* state,
                                  float* out, hipStream_t stream) {
#define KLA_DEC_CASE(DKV, DVV)                                                                      \
  if (dk == DKV && dv == DVV)                                                                       \
    return launch_decode_t<MODE, DKV, DVV>(N, H, q, k, v, la, eta, eps, direct, state, out, stream);
  KLA_DEC_CASE(64, 64)
  KLA_DEC_CASE(64, 128)
  KLA_DEC_CASE(128, 64)
  KLA_DEC_CASE(128, 128)
  KLA_DEC_CASE(256, 64)
  KLA_DEC_CASE(256, 128)
#undef KLA_DEC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode(int mode, int N, int H, int dk, int dv, const void* q, const void* k, const void* v,
                         const float* log_alpha, const float* eta, float eps, int direct, float* state,
                         float* out, hipStream_t stream) {
  if (mode == MODE_BF16)
    return dispatch_decode<MODE_BF16>(N, H, dk, dv, q, k, v, log_alpha, eta, eps, direct, state, out, stream);
  return dispatch_decode<MODE_F32>(N, H, dk, dv, q, k, v, log_alpha, eta, eps, direct, state, out, stream);
}

}  // namespace kla
