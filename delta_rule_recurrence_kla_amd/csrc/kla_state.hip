// Inter-chunk state and output kernels of the chunkwise KLA forward.
//
// One workgroup owns a group of NCOLS = 16 * NW state columns of one (batch, head)
// and walks its chunks in order; each wave owns 16 columns. Columns of the state
// never mix: every product below contracts over keys or tokens only, so a
// column group evolves on its own. The state S (dk x 16 per wave, fp32) lives
// in registers as MFMA accumulator tiles for the whole walk.
//
// Per chunk, with the chunk's record from the prep kernel (T', P, e^{g}, e^{g_C-g}):
//   R  = V - diag(e^g) K S              residual of the chunk's tokens against the start state
//   U  = T' R                           the chunk's writes u_r = beta_r e_r
//   O  = diag(e^g) Q S + P U            o_t = S_t^T q_t for every token of the chunk
//   S <- e^{g_C} S + K^T diag(e^{g_C - g}) U
// This is the unrolled form of the KLA page's update ("KLA update rule") inside one
// chunk; the chunkwise solver itself is kept from Gated DeltaNet (KLA page,
// "Implementation"). In bf16 mode q, k, v enter the MFMA exactly; every other
// operand is fp32 carried as a hi + lo bf16 pair, and accumulation is fp32.
//
// The same kernel also serves the associative-scan path (KATA page, section 2.3;
// HLA page, section 4): a segment of chunks maps any start state affinely,
// S_end = M S_start + N. Running the walk on the augmented state [I | 0] with value
// columns zero in the identity part yields [M | N] (AUG = true). A short sequential
// pass composes the maps of all segments into each segment's true start state, and
// a final walk per segment produces the outputs.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

struct StateArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* rec;
  int T, H, DV, nc;
  int seg_chunks;        // chunks per segment (nc for the sequential path)
  const float* init;     // start states: init + (bh * init_segs + seg) * DK * DV; null = zero
  int init_segs;
  float* out;            // [B, T, H, DV]
  float* fin;            // end states: fin + (bh * fin_segs + slot) * DK * fin_ld
  int fin_ld;
  int fin_segs;
  int fin_last_only;     // write only from the last segment, into slot 0
};

template <int MODE, int DK, int NW, bool WITH_OUT, bool AUG>
__global__ __launch_bounds__(NW * 64) void state_kernel(StateArgs a) {
  using TR = Tr<MODE>;
  using in_t = typename TR::in_t;
  using DF = typename TR::DF;
  constexpr int NT = NW * 64;
  constexpr int NCOLS = NW * 16;
  constexpr int VEC = 16 / static_cast<int>(sizeof(in_t));
  constexpr int LDK = DK + VEC;      // [token][key] pitch
  constexpr int LDT = CHUNK + VEC;   // [key][token] pitch
  constexpr int LDV = NCOLS + VEC;   // [token][column] pitch
  static_assert(!AUG || DK % NCOLS == 0, "identity/value columns must not share a workgroup");

  __shared__ __align__(16) in_t sK[CHUNK * LDK];
  __shared__ __align__(16) in_t sKt[DK * LDT];
  __shared__ __align__(16) in_t sQ[WITH_OUT ? CHUNK * LDK : VEC];
  __shared__ __align__(16) in_t sV[CHUNK * LDV];
  __shared__ __align__(16) uint8_t sTP[CHUNK * DROW_BYTES];
  __shared__ __align__(16) uint8_t sPP[WITH_OUT ? CHUNK * DROW_BYTES : 16];
  __shared__ float sEG[CHUNK], sEGC[CHUNK];

  const in_t* __restrict__ gq_ = static_cast<const in_t*>(a.q);
  const in_t* __restrict__ gk_ = static_cast<const in_t*>(a.k);
  const in_t* __restrict__ gv_ = static_cast<const in_t*>(a.v);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gq = lane >> 4, ln = lane & 15;
  const int cg = blockIdx.x, seg = blockIdx.y, bh = blockIdx.z;
  const int H = a.H, T = a.T, DV = a.DV;
  const int b = bh / H, h = bh - b * H;
  const int col0 = cg * NCOLS;            // first (augmented) column of the workgroup
  const int col = col0 + 16 * w + ln;     // this lane's column
  const bool ident = AUG && col0 < DK;    // identity part of [M | N]
  const int vcol0 = AUG ? col0 - DK : col0;
  const int vcol = vcol0 + 16 * w + ln;
  const int c_begin = seg * a.seg_chunks;
  const int c_end = min(a.nc, c_begin + a.seg_chunks);

  // start state
  f32x4 S[DK / 16];
#pragma unroll
  for (int mt = 0; mt < DK / 16; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mt + 4 * gq + i;
      float s0 = 0.f;
      if constexpr (AUG) {
        s0 = (ident && r == col) ? 1.f : 0.f;
      } else {
        if (a.init) s0 = a.init[(static_cast<size_t>(bh) * a.init_segs + seg) * DK * DV + r * DV + col];
      }
      S[mt][i] = s0;
    }
  }

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * CHUNK;
    const uint8_t* R = a.rec + (static_cast<size_t>(bh) * a.nc + c) * REC_BYTES;

    // ---- chunk inputs into LDS ----
    for (int idx = tid; idx < CHUNK * DK / VEC; idx += NT) {
      const int r = idx / (DK / VEC), cv = (idx % (DK / VEC)) * VEC;
      const int t = t0 + r;
      uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
      if (t < T) {
        const size_t off = ((static_cast<size_t>(b) * T + t) * H + h) * DK + cv;
        x = *reinterpret_cast<const uint4*>(gk_ + off);
        if constexpr (WITH_OUT) y = *reinterpret_cast<const uint4*>(gq_ + off);
      }
      *reinterpret_cast<uint4*>(sK + r * LDK + cv) = x;
      if constexpr (WITH_OUT) *reinterpret_cast<uint4*>(sQ + r * LDK + cv) = y;
      const in_t* e = reinterpret_cast<const in_t*>(&x);
#pragma unroll
      for (int j = 0; j < VEC; ++j) sKt[(cv + j) * LDT + r] = e[j];
    }
    if (!ident) {
      for (int idx = tid; idx < CHUNK * NCOLS / VEC; idx += NT) {
        const int r = idx / (NCOLS / VEC), cv = (idx % (NCOLS / VEC)) * VEC;
        const int t = t0 + r;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (t < T) x = *reinterpret_cast<const uint4*>(gv_ + ((static_cast<size_t>(b) * T + t) * H + h) * DV + vcol0 + cv);
        *reinterpret_cast<uint4*>(sV + r * LDV + cv) = x;
      }
    }
    for (int idx = tid; idx < CHUNK * 16; idx += NT) {
      const int r = idx >> 4, j = idx & 15;
      *reinterpret_cast<uint4*>(sTP + r * DROW_BYTES + 16 * j) =
          *reinterpret_cast<const uint4*>(R + REC_T_OFF + r * 256 + 16 * j);
      if constexpr (WITH_OUT)
        *reinterpret_cast<uint4*>(sPP + r * DROW_BYTES + 16 * j) =
            *reinterpret_cast<const uint4*>(R + REC_P_OFF + r * 256 + 16 * j);
    }
    if (tid < CHUNK) {
      sEG[tid] = reinterpret_cast<const float*>(R + REC_EG_OFF)[tid];
      sEGC[tid] = reinterpret_cast<const float*>(R + REC_EGC_OFF)[tid];
    }
    __syncthreads();

    // ---- S as B operand (contraction over keys) ----
    DF Sb[DK / 32];
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) Sb[kb] = TR::mk(frag_from_acc(S[2 * kb], S[2 * kb + 1]));

    // ---- R = V - diag(e^g) K S ----
    f32x4 Rr[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) acc = TR::mma_xd(acc, TR::ldx(sK, LDK, 16 * mt, 32 * kb, lane), Sb[kb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * mt + 4 * gq + i;
        const float vv = ident ? 0.f : TR::to_f32(sV[tok * LDV + 16 * w + ln]);
        Rr[mt][i] = vv - sEG[tok] * acc[i];
      }
    }
    DF Rb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Rb[kb] = TR::mk(frag_from_acc(Rr[2 * kb], Rr[2 * kb + 1]));

    // ---- U = T' R ----
    f32x4 U[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      U[mt] = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) U[mt] = TR::mma_dd(U[mt], TR::ldd(sTP, 16 * mt, 32 * kb, lane), Rb[kb]);
    }

    // ---- O = diag(e^g) Q S + P U ----
    if constexpr (WITH_OUT) {
      DF Ub[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) Ub[kb] = TR::mk(frag_from_acc(U[2 * kb], U[2 * kb + 1]));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) acc = TR::mma_xd(acc, TR::ldx(sQ, LDK, 16 * mt, 32 * kb, lane), Sb[kb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= sEG[16 * mt + 4 * gq + i];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc = TR::mma_dd(acc, TR::ldd(sPP, 16 * mt, 32 * kb, lane), Ub[kb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 16 * mt + 4 * gq + i;
          if (t < T) a.out[((static_cast<size_t>(b) * T + t) * H + h) * DV + vcol] = acc[i];
        }
      }
    }

    // ---- S <- e^{g_C} S + K^T diag(e^{g_C - g}) U ----
    const float gC = sEG[CHUNK - 1];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) U[mt][i] *= sEGC[16 * mt + 4 * gq + i];
    }
    DF Ud[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Ud[kb] = TR::mk(frag_from_acc(U[2 * kb], U[2 * kb + 1]));
#pragma unroll
    for (int mt = 0; mt < DK / 16; ++mt) {
      S[mt] *= gC;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) S[mt] = TR::mma_xd(S[mt], TR::ldx(sKt, LDT, 16 * mt, 32 * kb, lane), Ud[kb]);
    }
    __syncthreads();
  }

  // end state
  if (a.fin && (!a.fin_last_only || seg == static_cast<int>(gridDim.y) - 1)) {
    float* F = a.fin + (static_cast<size_t>(bh) * a.fin_segs + (a.fin_last_only ? 0 : seg)) * DK * a.fin_ld;
#pragma unroll
    for (int mt = 0; mt < DK / 16; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) F[(16 * mt + 4 * gq + i) * a.fin_ld + col] = S[mt][i];
    }
  }
}

// Start state of every segment: X_0 = init (or 0), X_{s+1} = M_s X_s + N_s.
// One workgroup per (b, h, 16-column tile of dv); fp32 throughout.
template <int DK>
__global__ __launch_bounds__(256) void scan_starts_kernel(const float* __restrict__ maps,
                                                          const float* __restrict__ init,
                                                          float* __restrict__ starts, int DV, int segs) {
  __shared__ float X[DK][16];
  const int tid = threadIdx.x;
  const int ct = blockIdx.x, bh = blockIdx.y;
  const int c0 = ct * 16;
  const int LDM = DK + DV;
  for (int o = tid; o < DK * 16; o += 256) {
    const int r = o >> 4, j = o & 15;
    const float x = init ? init[static_cast<size_t>(bh) * DK * DV + r * DV + c0 + j] : 0.f;
    X[r][j] = x;
    starts[(static_cast<size_t>(bh) * segs) * DK * DV + r * DV + c0 + j] = x;
  }
  __syncthreads();
  for (int s = 0; s + 1 < segs; ++s) {
    const float* M = maps + (static_cast<size_t>(bh) * (segs - 1) + s) * DK * LDM;
    float y[DK * 16 / 256];
#pragma unroll
    for (int q = 0; q < DK * 16 / 256; ++q) {
      const int o = tid + 256 * q;
      const int r = o >> 4, j = o & 15;
      const float* Mr = M + static_cast<size_t>(r) * LDM;
      float acc = Mr[DK + c0 + j];
      for (int u = 0; u < DK; ++u) acc += Mr[u] * X[u][j];
      y[q] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < DK * 16 / 256; ++q) {
      const int o = tid + 256 * q;
      const int r = o >> 4, j = o & 15;
      X[r][j] = y[q];
      starts[(static_cast<size_t>(bh) * segs + s + 1) * DK * DV + r * DV + c0 + j] = y[q];
    }
    __syncthreads();
  }
}

__global__ void copy_or_zero_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------
constexpr int NW_STATE = 4;  // 4 waves = 64 columns per workgroup

template <int MODE, int DK, bool WITH_OUT, bool AUG>
static hipError_t launch_state_t(dim3 grid, const StateArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((state_kernel<MODE, DK, NW_STATE, WITH_OUT, AUG>), grid, dim3(NW_STATE * 64), 0, stream, a);
  return hipGetLastError();
}

template <bool WITH_OUT, bool AUG>
static hipError_t dispatch_state(int mode, int dk, dim3 grid, const StateArgs& a, hipStream_t stream) {
  if (mode == MODE_BF16) {
    switch (dk) {
      case 64: return launch_state_t<MODE_BF16, 64, WITH_OUT, AUG>(grid, a, stream);
      case 128: return launch_state_t<MODE_BF16, 128, WITH_OUT, AUG>(grid, a, stream);
      case 256: return launch_state_t<MODE_BF16, 256, WITH_OUT, AUG>(grid, a, stream);
    }
  } else {
    switch (dk) {
      case 64: return launch_state_t<MODE_F32, 64, WITH_OUT, AUG>(grid, a, stream);
      case 128: return launch_state_t<MODE_F32, 128, WITH_OUT, AUG>(grid, a, stream);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_state_seq(int mode, const Dims& d, const void* q, const void* k, const void* v,
                            const uint8_t* rec, const float* init, float* out, float* fin,
                            hipStream_t stream) {
  StateArgs a{q, k, v, rec, d.T, d.H, d.dv, d.nc, d.nc, init, 1, out, fin, d.dv, 1, 0};
  dim3 grid(d.dv / (16 * NW_STATE), 1, d.B * d.H);
  return dispatch_state<true, false>(mode, d.dk, grid, a, stream);
}

hipError_t launch_scan_maps(int mode, const Dims& d, const void* k, const void* v, const uint8_t* rec,
                            int seg_chunks, int segs, float* maps, hipStream_t stream) {
  StateArgs a{nullptr, k, v, rec, d.T, d.H, d.dv, d.nc, seg_chunks, nullptr, 1, nullptr, maps, d.dk + d.dv,
              segs - 1, 0};
  dim3 grid((d.dk + d.dv) / (16 * NW_STATE), segs - 1, d.B * d.H);
  return dispatch_state<false, true>(mode, d.dk, grid, a, stream);
}

hipError_t launch_scan_starts(const Dims& d, const float* maps, const float* init, int segs, float* starts,
                              hipStream_t stream) {
  dim3 grid(d.dv / 16, d.B * d.H);
  switch (d.dk) {
    case 64: hipLaunchKernelGGL(scan_starts_kernel<64>, grid, dim3(256), 0, stream, maps, init, starts, d.dv, segs); break;
    case 128: hipLaunchKernelGGL(scan_starts_kernel<128>, grid, dim3(256), 0, stream, maps, init, starts, d.dv, segs); break;
    case 256: hipLaunchKernelGGL(scan_starts_kernel<256>, grid, dim3(256), 0, stream, maps, init, starts, d.dv, segs); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_scan_apply(int mode, const Dims& d, const void* q, const void* k, const void* v,
                             const uint8_t* rec, int seg_chunks, int segs, const float* starts, float* out,
                             float* fin, hipStream_t stream) {
  StateArgs a{q, k, v, rec, d.T, d.H, d.dv, d.nc, seg_chunks, starts, segs, out, fin, d.dv, 1, 1};
  dim3 grid(d.dv / (16 * NW_STATE), segs, d.B * d.H);
  return dispatch_state<true, false>(mode, d.dk, grid, a, stream);
}

hipError_t launch_copy_or_zero(const float* src, float* dst, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                     stream, src, dst, n);
  return hipGetLastError();
}

}  // namespace kla
