// Chunk prep kernel of the chunkwise KLA forward.
//
// For each 64-token chunk of one (batch, head) it computes, in this order:
//   G      = K K^T, QK = Q K^T                     (MFMA; q, k enter exactly)
//   n_r    = ||k_r||^2 = G_rr
//   beta_r = eta_r / (n_r + eps)                   Kaczmarz step size: KLA page, "KLA update rule"
//   g_r    = sum_{j<=r} log_alpha_j                chunk-local decay exponents
//   P      = QK masked by e^{g_r-g_i} for i <= r   (diagonal included: o_t reads S_t after the write)
//   A      = strict_lower(beta_r e^{g_r-g_i} G)
//   T      = (I + A)^-1                            blocked inverse of a unit lower-triangular matrix
//   T'     = T diag(beta)
// and stores T', P, e^{g_r}, e^{g_C-g_r} and g_r as the chunk's record (matrix rows in the
// swizzled LDS layout of kla_device.h). The compact variant (COMPACT = true) is for the
// state kernel that forms P itself: it neither reads Q nor stores P, and stores T' without
// its zero upper-right quadrant.
//
// Why this is the chunk's whole job: writing u_i = beta_i e_i and unrolling the
// per-token update of the KLA page ("KLA update rule": S_t = S~ + beta_t k_t e_t^T,
// e_t = v_t - S~^T k_t, S~ = alpha_t S_{t-1}) inside a chunk that starts from S_0 gives
//   (I + A) U = diag(beta) (V - diag(e^g) K S_0),   so U = T' (V - diag(e^g) K S_0),
// and o_r = e^{g_r} S_0^T q_r + sum_{i<=r} P_ri u_i. This is the chunkwise solver that
// the KLA page ("Implementation") keeps from Gated DeltaNet with only
// B = Diag(beta_1..beta_C) changed. None of it depends on the state, so every chunk of
// every head is prepared in parallel.
//
// One wavefront prepares one chunk and never waits on another wave: K and Q enter
// MFMA straight from global memory in fragment layout, the inverse runs as MFMA
// products over 16x16 blocks, and LDS serves only as the wave's own staging area
// (to turn accumulator tiles into coalesced record rows and into A operands).
//
// The inverse, by block rows (D_I = (I + A_II)^-1, found by forward substitution):
//   T_II = D_I,   T_IJ = -D_I X_IJ,   X_IJ = sum_{C=J}^{I-1} A_IC T_CJ   (J < I).
//
// With LIFT = true, q and k arrive as the 16-wide vectors u of the KATA page's rank-one PSD
// feature (section 2.2) and each key/query fragment is formed from them as it is loaded:
// feature 16a + b is u_a u_b, rounded to bf16, so the products below see exactly the 256
// features the unfused path would read. Each feature passes through one lane exactly once, and
// that lane also stores it: prep writes the lifted query and key rows that the state walks read.
//
// Tokens past T in the last chunk enter as identity steps: k = q = 0, log_alpha = 0,
// eta = 0, so their rows and columns of T' and P are zero.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

static_assert(LIFT_P_HOST == LIFT_P, "host and kernels must agree on the lift width");

namespace {

constexpr int AP = 20;        // fp32 pitch of a packed 16 x 16 block of A (80-byte rows)
constexpr int ABLK = 16 * AP;  // floats per packed block
constexpr int DP = 17;        // fp32 pitch of a 16 x 16 diagonal-block inverse

__device__ __forceinline__ int tix(int mt, int nt) { return mt * (mt + 1) / 2 + nt; }  // lower tiles

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// 8 fp32 values of block row I of A in contraction-slot order: row ln of blocks (I, C0) and
// (I, C0 + 1), columns 4gq .. 4gq+3 of each. `second` = false zeroes slots 4..7.
__device__ __forceinline__ F8 a_frag(const float* sA, int I, int C0, int ln, int gq, bool second) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(sA + tix(I, C0) * ABLK + ln * AP + 4 * gq);
  f32x4 b = zero4();
  if (second) b = *reinterpret_cast<const f32x4*>(sA + tix(I, C0 + 1) * ABLK + ln * AP + 4 * gq);
  return frag_from_acc(a, b);
}

}  // namespace

template <int MODE, int DK, bool COMPACT, bool LIFT>
__global__ __launch_bounds__(64) void prep_kernel(const void* __restrict__ qv, const void* __restrict__ kv,
                                                   const float* __restrict__ log_alpha,
                                                   const float* __restrict__ eta, float eps, int direct,
                                                   uint8_t* __restrict__ rec, int T, int H, int nc, int nchunks,
                                                   void* __restrict__ fq, void* __restrict__ fk) {
  using TR = Tr<MODE>;
  using in_t = typename TR::in_t;
  using XF = typename TR::XF;
  using DF = typename TR::DF;
  constexpr int SZ = static_cast<int>(sizeof(in_t));
  static_assert(!LIFT || (MODE == MODE_BF16 && DK == LIFT_DK && !COMPACT), "the lift makes 256 bf16 features");
  constexpr int KIN = LIFT ? LIFT_P : DK;  // elements of a query/key row in memory

  // One wave per workgroup (17.3 KB of LDS), so that LDS, not the workgroup shape, sets how
  // many chunks a CU holds: nine, against eight as four-wave groups (about 6% faster).
  // The 10 lower 16x16 blocks of A; a 16-row staging strip (272-byte rows) that also holds
  // the diagonal-block inverses during the inverse; n (then beta) and g.
  __shared__ __align__(16) float sA[10 * ABLK];
  __shared__ __align__(16) float st[16 * 68];
  __shared__ __align__(16) float sVec[2][64];

  const int lane = threadIdx.x;
  const int gq = lane >> 4, ln = lane & 15;
  const int id = blockIdx.x;
  const int bh = id / nc, c = id - bh * nc;
  const int b = bh / H, h = bh - b * H;
  const int t0 = c * CHUNK;
  float* sDw = st;  // diagonal-block inverses D_I at I * 16 * DP
  float* sNB = sVec[0];
  float* sGv = sVec[1];

  // ---- G = K K^T and QK = Q K^T on the lower 10 tiles, operands straight from memory ----
  const int rowK = H * KIN * SZ;
  const size_t chunk_off = (static_cast<size_t>(b) * T + t0) * rowK;
  const long long avail = static_cast<long long>(T - t0) * rowK;
  const rsrc_t rk = make_rsrc_wu(static_cast<const uint8_t*>(kv) + chunk_off, avail);
  const rsrc_t rq = make_rsrc_wu(static_cast<const uint8_t*>(qv) + chunk_off, avail);
  // LIFT: the lifted query and key rows ([B, T, H, DK] bf16) that the state walks read
  const int rowF = H * DK * 2;
  const size_t fchunk_off = (static_cast<size_t>(b) * T + t0) * rowF;
  const long long favail = LIFT ? static_cast<long long>(T - t0) * rowF : 0;
  const rsrc_t wq = make_rsrc_wu(LIFT ? static_cast<uint8_t*>(fq) + fchunk_off : nullptr, favail);
  const rsrc_t wk = make_rsrc_wu(LIFT ? static_cast<uint8_t*>(fk) + fchunk_off : nullptr, favail);
  // gates first: their loads then overlap the key loads
  const int t = t0 + lane;
  float la = 0.f, et = 0.f;
  if (t < T) {
    const size_t gi = (static_cast<size_t>(b) * T + t) * H + h;
    la = log_alpha[gi];
    et = eta[gi];
  }
  f32x4 G[10], QK[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) G[i] = QK[i] = zero4();

  // Compact bf16 variant: every key fragment of the chunk is loaded before the first
  // product, so the wave waits for one memory round trip instead of one per 32 columns.
  constexpr bool PRELOAD = COMPACT && MODE == MODE_BF16 && DK <= 128;
  XF kall[PRELOAD ? DK / 32 : 1][4];
  if constexpr (PRELOAD) {
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        // eight consecutive key columns per lane, one 16-byte load: G = K K^T sums over the
        // columns in any order in which both operands agree
        const int off = (16 * x + ln) * rowK + h * DK * SZ + (32 * kb + 8 * gq) * SZ;
        kall[kb][x] = __builtin_bit_cast(bf16x8, bload16(rk, off));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the products
  }
  // Lifted rows: the chunk's u rows (32 bytes each, keys then queries) go to the staging
  // strip, which is free until the products are done; lane t loads token t's rows.
  uint8_t* sU = reinterpret_cast<uint8_t*>(st);
  if constexpr (LIFT) {
    static_assert(2 * CHUNK * LIFT_P * 2 <= static_cast<int>(sizeof(st)), "u rows fit the strip");
    const int off = lane * rowK + h * LIFT_P * 2;
    const u32x4 k0 = bload16(rk, off), k1 = bload16(rk, off + 16);
    const u32x4 q0 = bload16(rq, off), q1 = bload16(rq, off + 16);
    *reinterpret_cast<u32x4*>(sU + 32 * lane) = k0;
    *reinterpret_cast<u32x4*>(sU + 32 * lane + 16) = k1;
    *reinterpret_cast<u32x4*>(sU + 2048 + 32 * lane) = q0;
    *reinterpret_cast<u32x4*>(sU + 2048 + 32 * lane + 16) = q1;
    wave_sync();
  }

#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb) {
    XF kf[4], qf[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int off = (16 * x + ln) * rowK + h * DK * SZ + (32 * kb + 4 * gq) * SZ;
      if constexpr (PRELOAD) {
        kf[x] = kall[kb][x];
      } else if constexpr (LIFT) {
        // features 32kb + 8gq + 0..7 = 16a + b0 + 0..7 with a = 2kb + (gq >> 1), b0 = 8 (gq & 1):
        // u_a is half (gq >> 1) of word kb of the row, u_b0.. the row's half (gq & 1)
        const bool odd = (gq >> 1) != 0;
        const uint8_t* ukr = sU + 32 * (16 * x + ln);
        const uint8_t* uqr = ukr + 2048;
        const uint32_t kw = *reinterpret_cast<const uint32_t*>(ukr + 4 * kb);
        const uint32_t qw = *reinterpret_cast<const uint32_t*>(uqr + 4 * kb);
        const u32x4 kbv = *reinterpret_cast<const u32x4*>(ukr + 16 * (gq & 1));
        const u32x4 qbv = *reinterpret_cast<const u32x4*>(uqr + 16 * (gq & 1));
        const u32x4 kl = lift8(lift_pick(kw, odd), kbv), ql = lift8(lift_pick(qw, odd), qbv);
        kf[x] = __builtin_bit_cast(bf16x8, kl);
        qf[x] = __builtin_bit_cast(bf16x8, ql);
        // every feature of the chunk passes through exactly one lane here: store it for the walks
        // (rows past T fall outside the buffer range and are dropped)
        const int foff = (16 * x + ln) * rowF + (h * DK + 32 * kb + 8 * gq) * 2;
        __builtin_amdgcn_raw_buffer_store_b128(kl, wk, foff, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(ql, wq, foff, 0, 0);
      } else if constexpr (MODE == MODE_BF16) {
        const int off8 = (16 * x + ln) * rowK + h * DK * SZ + (32 * kb + 8 * gq) * SZ;  // as in the preload
        kf[x] = __builtin_bit_cast(bf16x8, bload16(rk, off8));
        if constexpr (!COMPACT) qf[x] = __builtin_bit_cast(bf16x8, bload16(rq, off8));
      } else {
        const f32x4 k0 = __builtin_bit_cast(f32x4, bload16(rk, off));
        const f32x4 k1 = __builtin_bit_cast(f32x4, bload16(rk, off + 16 * SZ));
        const f32x4 q0 = __builtin_bit_cast(f32x4, bload16(rq, off));
        const f32x4 q1 = __builtin_bit_cast(f32x4, bload16(rq, off + 16 * SZ));
        kf[x] = frag_from_acc(k0, k1);
        qf[x] = frag_from_acc(q0, q1);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int nt = 0; nt <= mt; ++nt) {
        G[tix(mt, nt)] = TR::mma_xx(G[tix(mt, nt)], kf[mt], kf[nt]);
        if constexpr (!COMPACT) QK[tix(mt, nt)] = TR::mma_xx(QK[tix(mt, nt)], qf[mt], kf[nt]);
      }
    }
  }

  // ---- key norms from the diagonal of G; gates; beta; decay exponents ----
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const f32x4 d = G[tix(x, x)];
    const int i = ln & 3;
    const float v = i == 0 ? d[0] : i == 1 ? d[1] : i == 2 ? d[2] : d[3];
    if ((ln >> 2) == gq) sNB[16 * x + ln] = v;  // G[16x+ln][16x+ln]
  }
  // inclusive cumsum over the 64 lanes: DPP row shifts by 1, 2, 4, 8 within rows of 16 lanes
  // (lanes shifted in from outside a row read 0), then lane 15 of each row added to the next
  // row (rows 1 and 3) and lane 31 to rows 2 and 3
  float g = la;
  auto dpp = [](float x, auto ctrl_c, auto rows_c, auto bound_c) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl_c)::value,
                                                      decltype(rows_c)::value, 0xf, decltype(bound_c)::value));
  };
  using shr1 = std::integral_constant<int, 0x111>;
  using shr2 = std::integral_constant<int, 0x112>;
  using shr4 = std::integral_constant<int, 0x114>;
  using shr8 = std::integral_constant<int, 0x118>;
  using bc15 = std::integral_constant<int, 0x142>;
  using bc31 = std::integral_constant<int, 0x143>;
  using all_rows = std::integral_constant<int, 0xf>;
  using rows13 = std::integral_constant<int, 0xa>;
  using rows23 = std::integral_constant<int, 0xc>;
  using zero_oob = std::integral_constant<bool, true>;
  using keep_oob = std::integral_constant<bool, false>;
  g += dpp(g, shr1{}, all_rows{}, zero_oob{});
  g += dpp(g, shr2{}, all_rows{}, zero_oob{});
  g += dpp(g, shr4{}, all_rows{}, zero_oob{});
  g += dpp(g, shr8{}, all_rows{}, zero_oob{});
  g += dpp(g, bc15{}, rows13{}, keep_oob{});
  g += dpp(g, bc31{}, rows23{}, keep_oob{});
  const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), 63));
  wave_sync();
  const float denom = sNB[lane] + eps;
  // the Kaczmarz step, or (direct) the learned write strength as given
  const float beta = direct ? et : denom != 0.f ? et / denom : 0.f;
  wave_sync();
  sNB[lane] = beta;
  sGv[lane] = g;
  constexpr int RB = COMPACT ? CREC_BYTES : REC_BYTES;
  uint8_t* R = rec + static_cast<size_t>(id) * RB;
  const rsrc_t rr = make_rsrc_wu(R, RB);
  bstore_f32(__expf(g), rr, (COMPACT ? CREC_EG_OFF : REC_EG_OFF) + 4 * lane);
  bstore_f32(__expf(gC - g), rr, (COMPACT ? CREC_EGC_OFF : REC_EGC_OFF) + 4 * lane);
  bstore_f32(g, rr, (COMPACT ? CREC_G_OFF : REC_G_OFF) + 4 * lane);
  wave_sync();

  // Copies the staged strip (16 rows of 256 bytes, pitch 272) to record rows 16*mt .. 16*mt+15 at byte dst.
  auto flush_strip = [&](int dst, int mt) __attribute__((always_inline)) {
    wave_sync();
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(st);
    if (COMPACT && mt < 2) {
      // rows 0..31 of the compact T': pieces 0..3 (hi of columns 0..31) and 8..11 (lo)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int p = lane + 64 * j;  // strip row p >> 3, compact piece p & 7
        const int cp = p & 7, sp = cp < 4 ? cp : cp + 4;
        const u32x4 x = *reinterpret_cast<const u32x4*>(sb + (p >> 3) * 272 + 16 * sp);
        const int row = 16 * mt + (p >> 3);
        __builtin_amdgcn_raw_buffer_store_b128(x, rr, CREC_TOP_OFF + swz_off<128>(row, 16 * cp), 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = lane + 64 * j;  // 16-byte piece: strip row p >> 4, column piece p & 15
        const u32x4 x = *reinterpret_cast<const u32x4*>(sb + (p >> 4) * 272 + 16 * (p & 15));
        const int row = 16 * mt + (p >> 4);
        if constexpr (COMPACT)
          __builtin_amdgcn_raw_buffer_store_b128(x, rr, CREC_BOT_OFF + swz_off<256>(row - 32, 16 * (p & 15)), 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b128(x, rr, dst + swz_off<256>(row, 16 * (p & 15)), 0, 0);
      }
    }
    wave_sync();
  };
  // Writes one element of a derived 64 x 64 matrix into the strip (row r of the strip).
  auto stage_put = [&](int r, int cc, float v) __attribute__((always_inline)) {
    uint8_t* row = reinterpret_cast<uint8_t*>(st) + r * 272;
    if constexpr (MODE == MODE_BF16) {
      const __bf16 hi = static_cast<__bf16>(v);
      reinterpret_cast<__bf16*>(row)[cc] = hi;
      reinterpret_cast<__bf16*>(row)[64 + cc] = static_cast<__bf16>(v - static_cast<float>(hi));
    } else {
      reinterpret_cast<float*>(row)[cc] = v;
    }
  };

  // ---- P = QK masked by the inclusive decay mask -> record ----
#pragma unroll
  for (int mt = 0; mt < (COMPACT ? 0 : 4); ++mt) {
    const f32x4 gr = *reinterpret_cast<const f32x4*>(sGv + 16 * mt + 4 * gq);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int cc = 16 * nt + ln;
      const float gc = sGv[cc];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * gq + i;
        float v = 0.f;
        if (nt <= mt) v = cc <= r ? __expf(gr[i] - gc) * QK[tix(mt, nt)][i] : 0.f;
        stage_put(4 * gq + i, cc, v);
      }
    }
    flush_strip(REC_P_OFF, mt);
  }

  // ---- A = strict_lower(beta_r e^{g_r - g_i} G) into the stage as fp32 ----
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const f32x4 gr = *reinterpret_cast<const f32x4*>(sGv + 16 * mt + 4 * gq);
    const f32x4 br = *reinterpret_cast<const f32x4*>(sNB + 16 * mt + 4 * gq);
#pragma unroll
    for (int nt = 0; nt <= mt; ++nt) {
      const int cc = 16 * nt + ln;
      const float gc = sGv[cc];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * gq + i;
        sA[tix(mt, nt) * ABLK + (4 * gq + i) * AP + ln] =
            cc < r ? br[i] * __expf(gr[i] - gc) * G[tix(mt, nt)][i] : 0.f;
      }
    }
  }
  wave_sync();

  // ---- diagonal blocks D_blk = (I + A_blk,blk)^-1; lane (gq, ln) = (block, column) ----
  // column-oriented forward substitution: once x_i is final, fold it into every later row
  {
    const int blk = gq, j = ln;
    const float* Ab = sA + tix(blk, blk) * ABLK;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = r == j ? 1.f : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
      for (int r = i + 1; r < 16; ++r) x[r] -= Ab[r * AP + i] * x[i];
    }
    wave_sync();  // the P strip flush has finished with the staging area
#pragma unroll
    for (int r = 0; r < 16; ++r) sDw[blk * 16 * DP + r * DP + j] = x[r];
  }
  wave_sync();

  // ---- off-diagonal blocks by block rows; tiles of T in accumulator layout ----
  f32x4 Tt[10];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
#pragma unroll
    for (int i = 0; i < 4; ++i) Tt[tix(I, I)][i] = sDw[I * 16 * DP + (4 * gq + i) * DP + ln];
  }
#pragma unroll
  for (int I = 1; I < 4; ++I) {
    // D_I as an A operand: row ln, contraction columns 4gq .. 4gq+3 (a 16-deep contraction)
    const float* dr = sDw + I * 16 * DP + ln * DP + 4 * gq;
    const f32x4 drow = {dr[0], dr[1], dr[2], dr[3]};
    const DF dI = TR::mk(frag_from_acc(drow, zero4()));
#pragma unroll
    for (int J = 0; J < I; ++J) {
      f32x4 X = zero4();
#pragma unroll
      for (int C0 = J; C0 < I; C0 += 2) {
        const bool two = C0 + 1 < I;
        const DF a = TR::mk(a_frag(sA, I, C0, ln, gq, two));
        const DF bb = TR::mk(frag_from_acc(Tt[tix(C0, J)], two ? Tt[tix(C0 + 1, J)] : zero4()));
        X = TR::mma_dd(X, a, bb);
      }
      const DF xb = TR::mk(frag_from_acc(X, zero4()));
      Tt[tix(I, J)] = -TR::mma_dd(zero4(), dI, xb);
    }
  }
  wave_sync();

  // ---- T' = T diag(beta) -> record ----
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int cc = 16 * nt + ln;
      const float bc = sNB[cc];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * gq + i;
        float v = 0.f;
        if (nt <= mt) v = cc <= r ? Tt[tix(mt, nt)][i] * bc : 0.f;
        stage_put(4 * gq + i, cc, v);
      }
    }
    flush_strip(REC_T_OFF, mt);
  }
}

template <int MODE, int DK, bool LIFT = false>
static hipError_t launch_prep_t(const Dims& d, const void* q, const void* k, const float* la, const float* eta,
                                float eps, int direct, uint8_t* rec, void* fq, void* fk, hipStream_t stream) {
  const int nchunks = d.B * d.H * d.nc;
  if (!LIFT && !d.full_rec && state_dma_supported(MODE, DK))
    return launch_kernel(prep_kernel<MODE, DK, true, false>, dim3(nchunks), dim3(64), stream, q, k, la, eta, eps,
                         direct, rec, d.T, d.H, d.nc, nchunks, fq, fk);
  return launch_kernel(prep_kernel<MODE, DK, false, LIFT>, dim3(nchunks), dim3(64), stream, q, k, la, eta, eps,
                       direct, rec, d.T, d.H, d.nc, nchunks, fq, fk);
}

int record_bytes(int mode, int dk) { return state_dma_supported(mode, dk) ? CREC_BYTES : REC_BYTES; }
int full_record_bytes() { return REC_BYTES; }

hipError_t launch_prep(int mode, const Dims& d, const void* q, const void* k, const float* log_alpha,
                       const float* eta, float eps, int direct, uint8_t* rec, hipStream_t stream, void* fq,
                       void* fk) {
  if (d.lift) {
    if (mode == MODE_BF16 && d.dk == LIFT_DK && fq && fk)
      return launch_prep_t<MODE_BF16, LIFT_DK, true>(d, q, k, log_alpha, eta, eps, direct, rec, fq, fk, stream);
    return hipErrorInvalidValue;
  }
  if (mode == MODE_BF16) {
    switch (d.dk) {
      case 64: return launch_prep_t<MODE_BF16, 64>(d, q, k, log_alpha, eta, eps, direct, rec, nullptr, nullptr, stream);
      case 128: return launch_prep_t<MODE_BF16, 128>(d, q, k, log_alpha, eta, eps, direct, rec, nullptr, nullptr, stream);
      case 256: return launch_prep_t<MODE_BF16, 256>(d, q, k, log_alpha, eta, eps, direct, rec, nullptr, nullptr, stream);
    }
  } else {
    switch (d.dk) {
      case 64: return launch_prep_t<MODE_F32, 64>(d, q, k, log_alpha, eta, eps, direct, rec, nullptr, nullptr, stream);
      case 128: return launch_prep_t<MODE_F32, 128>(d, q, k, log_alpha, eta, eps, direct, rec, nullptr, nullptr, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kla
