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
// a final walk per segment produces the outputs. From a zero start the first segment's
// start is known (X_1 = N_0), so its identity columns are not walked.
//
// The log-linear prefill (Log-Linear page, "Mathematical formalization") uses three more
// options: a segment stride (seg_mul, seg_add: every other half-block of a scale), walks
// with no values (v null: value loads go through a zero-size buffer range and read as
// zeros), and ACC = true, which adds lambda-weighted outputs to the ones already in `out`.
#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

constexpr int kMaxScales = 24;  // scales of 1, 2, 4, ... chunks: enough for any int T

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
  int ncg;               // column groups per (segment, head)
  int nseg;              // segments in the grid
  // Segment s of the grid walks chunks [(s * seg_mul + seg_add) * seg_chunks, + seg_chunks):
  // every segment (1, 0), or every other one (2, 0 / 2, 1) for the log-linear scales.
  int seg_mul = 1;
  int seg_add = 0;
  // ACC kernels: out[b, t, h, :] += lam[((b * T + t) * H + h) * lam_L + lam_level] * o_t
  const float* lam = nullptr;
  int lam_L = 0;
  int lam_level = 0;
  // Several scales in one grid (walks without outputs on the plain state only): scale i owns
  // workgroups [scale_wg[i], scale_wg[i + 1]), walks segments of scale_half[i] chunks with
  // stride 2, and writes its scale_nseg[i] end states per head at fin + scale_fin_off[i].
  int nscale = 0;
  int scale_wg[kMaxScales + 1] = {};
  int scale_half[kMaxScales] = {};
  int scale_nseg[kMaxScales] = {};
  long long scale_fin_off[kMaxScales] = {};
  // Map walks of a scan from a zero start: segment 0's identity columns are not walked (the
  // fold never reads M_0 then, since it multiplies a zero state), and their workgroups exit.
  int skip_ident0 = 0;
};

// Workgroup id -> (column group, unit), unit = bh * nseg + seg. The column groups of one
// unit read the same K, Q and T'; workgroup ids are dealt to the 8 XCDs round-robin, so
// ids that differ by a multiple of 8 share an L2. When the grid divides evenly, the
// groups of a unit get such ids.
__device__ __forceinline__ void decode_wg(int L, int ncg, int nunits, int& cg, int& unit) {
  if ((ncg * nunits) % (8 * ncg) == 0) {
    const int xcd = L & 7, slot = L >> 3;
    cg = slot % ncg;
    unit = (slot / ncg) * 8 + xcd;
  } else {
    cg = L % ncg;
    unit = L / ncg;
  }
}

// Packs 16-bit element `half` (0 = low, 1 = high) of words lo and hi into one word (lo first).
__device__ __forceinline__ uint32_t pack_halves(uint32_t lo, uint32_t hi, int half) {
  return __builtin_amdgcn_perm(hi, lo, half ? 0x07060302u : 0x05040100u);
}

template <int MODE, int DK, bool WITH_OUT, bool AUG, bool ACC>
// The bf16 map walk at dk = 256 (61 KB of LDS without a transposed copy of K) is held to the
// registers of two workgroups per CU: two map chains per SIMD, a few values spilled outside the
// chunk loop (map walk 389 -> 353 us on the PSD workload).
__global__ __launch_bounds__(256, (MODE == MODE_BF16 && DK == 256 && AUG) ? 2 : 1) void state_kernel(StateArgs a) {
  using TR = Tr<MODE>;
  using in_t = typename TR::in_t;
  using DF = typename TR::DF;
  constexpr int NT = 256;
  constexpr int NCOLS = 64;                    // 4 waves x 16 columns
  constexpr int SZ = static_cast<int>(sizeof(in_t));
  constexpr int VEC = 16 / SZ;                 // elements per 16-byte access
  constexpr int LDK = DK + VEC;                // [token][key] pitch (16-byte aligned rows)
  constexpr int LDT = CHUNK + 4;               // [key][token] and [column][token] pitch
  constexpr int KCB = DK / VEC;                // 16-byte column blocks of a key row
  constexpr int KBLK = 16 * KCB;               // (4 tokens x 16 bytes) blocks of a chunk's K
  constexpr int KPT = (KBLK + NT - 1) / NT;    // such blocks per thread
  constexpr int VCB = NCOLS / VEC;             // 16-byte column blocks of a value row
  constexpr int VBLK = 16 * VCB;               // (4 tokens x 16 bytes) blocks of a chunk's V
  constexpr int VPT = (VBLK + NT - 1) / NT;
  constexpr int TPT = CHUNK * 16 / NT;         // T' (and P) vectors per thread
  static_assert(!AUG || DK % NCOLS == 0, "identity/value columns must not share a workgroup");
  static_assert((KCB & (KCB - 1)) == 0 && (VCB & (VCB - 1)) == 0, "shape");

  __shared__ __align__(16) in_t sK[CHUNK * LDK];
  // K^T for the state update. bf16 features read K's rows transposed instead (ds_read_b64_tr_b16):
  // the map walk at dk = 256 then fits two workgroups per CU and the walks do fewer vector
  // transposes (PSD step 5% faster, 9% with the two workgroups).
  constexpr bool KT_TR = MODE == MODE_BF16;
  __shared__ __align__(16) in_t sKt[KT_TR ? VEC : DK * LDT];
  __shared__ __align__(16) in_t sQ[WITH_OUT ? CHUNK * LDK : VEC];
  __shared__ __align__(16) in_t sVt[NCOLS * LDT];
  __shared__ __align__(16) uint8_t sTP[CHUNK * DROW_BYTES];
  __shared__ __align__(16) uint8_t sPP[WITH_OUT ? CHUNK * DROW_BYTES : 16];
  __shared__ __align__(16) float sTail[3 * CHUNK];  // e^{g}, e^{g_C - g}, g
  const float* sEG = sTail;
  const float* sEGC = sTail + CHUNK;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gq = lane >> 4, ln = lane & 15;
  int cg, unit;
  // this workgroup's segment geometry (per scale when several scales share the grid)
  int wg = blockIdx.x, nwg_here = static_cast<int>(gridDim.x);
  int seg_chunks = a.seg_chunks, nseg = a.nseg, fin_segs = a.fin_segs;
  float* fin_base = a.fin;
  if constexpr (!WITH_OUT && !AUG) {
    if (a.nscale > 0) {
      int sc = 0;
      while (sc + 1 < a.nscale && wg >= a.scale_wg[sc + 1]) ++sc;
      wg -= a.scale_wg[sc];
      nwg_here = a.scale_wg[sc + 1] - a.scale_wg[sc];
      seg_chunks = a.scale_half[sc];
      nseg = fin_segs = a.scale_nseg[sc];
      fin_base = a.fin + a.scale_fin_off[sc];
    }
  }
  decode_wg(wg, a.ncg, nwg_here / a.ncg, cg, unit);
  const int bh = unit / nseg, seg = unit - bh * nseg;
  const int H = a.H, T = a.T, DV = a.DV;
  const int b = bh / H, h = bh - b * H;
  const int col0 = cg * NCOLS;            // first (augmented) column of the workgroup
  const int col = col0 + 16 * w + ln;     // this lane's column
  const bool ident = AUG && col0 < DK;    // identity part of [M | N]
  if (AUG && ident && seg == 0 && a.skip_ident0) return;  // uniform over the workgroup, before any barrier
  const int vcol0 = AUG ? col0 - DK : col0;
  const int vcol = vcol0 + 16 * w + ln;
  const int c_begin = (seg * a.seg_mul + a.seg_add) * seg_chunks;
  const int c_end = min(a.nc, c_begin + seg_chunks);

  // byte strides between consecutive tokens, and this batch's first rows
  const int rowK = H * DK * SZ, rowV = H * DV * SZ, rowO = H * DV * 4;
  const uint8_t* kb_ = static_cast<const uint8_t*>(a.k) + static_cast<size_t>(b) * T * rowK;
  const uint8_t* qb_ = static_cast<const uint8_t*>(a.q) + static_cast<size_t>(b) * T * rowK;
  const uint8_t* vb_ = static_cast<const uint8_t*>(a.v) + static_cast<size_t>(b) * T * rowV;
  uint8_t* ob_ = reinterpret_cast<uint8_t*>(a.out) + static_cast<size_t>(b) * T * rowO;

  // per-lane byte offsets inside a chunk (token 0 of the chunk = offset 0)
  auto kblk = [&](int blk, int& rb, int& cb) __attribute__((always_inline)) {
    rb = (blk & 3) | ((blk / (4 * KCB)) << 2);
    cb = (blk >> 2) & (KCB - 1);
  };
  auto vblk = [&](int blk, int& rb, int& cb) __attribute__((always_inline)) {
    rb = (blk & 3) | ((blk / (4 * VCB)) << 2);
    cb = (blk >> 2) & (VCB - 1);
  };

  // ---- prefetch registers: the next chunk's inputs, loaded while the current one is computed ----
  u32x4 pk[KPT][4];
  u32x4 pq[WITH_OUT ? KPT : 1][4];
  u32x4 pv[VPT][4];
  u32x4 pt[TPT];
  u32x4 pp[WITH_OUT ? TPT : 1];
  u32x4 ptail = {0u, 0u, 0u, 0u};

  auto issue_loads = [&](int c) __attribute__((always_inline)) {
    const int t0 = c * CHUNK;
    const long long rem = static_cast<long long>(T - t0);
    const rsrc_t rk = make_rsrc(kb_ + static_cast<size_t>(t0) * rowK, rem * rowK);
    const rsrc_t rq = make_rsrc(qb_ + static_cast<size_t>(t0) * rowK, WITH_OUT ? rem * rowK : 0);
    // no values (a.v null: the log-linear propagation walks) read as zeros, like the identity part
    const rsrc_t rv = make_rsrc(vb_ + static_cast<size_t>(t0) * rowV, ident || !a.v ? 0 : rem * rowV);
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int blk = tid + NT * u;
      int rb, cb;
      kblk(blk, rb, cb);
      const int off = blk < KBLK ? 4 * rb * rowK + h * DK * SZ + 16 * cb : BUF_OOB;
#pragma unroll
      for (int u4 = 0; u4 < 4; ++u4) {
        pk[u][u4] = bload16(rk, off + u4 * rowK);
        if constexpr (WITH_OUT) pq[u][u4] = bload16(rq, off + u4 * rowK);
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int blk = tid + NT * u;
      int rb, cb;
      vblk(blk, rb, cb);
      const int off = blk < VBLK ? 4 * rb * rowV + (h * DV + vcol0) * SZ + 16 * cb : BUF_OOB;
#pragma unroll
      for (int u4 = 0; u4 < 4; ++u4) pv[u][u4] = bload16(rv, off + u4 * rowV);
    }
    const uint8_t* R = a.rec + (static_cast<size_t>(bh) * a.nc + c) * REC_BYTES;
    const rsrc_t rr = make_rsrc(R, REC_BYTES);
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      pt[u] = bload16(rr, REC_T_OFF + 16 * (tid + NT * u));
      if constexpr (WITH_OUT) pp[u] = bload16(rr, REC_P_OFF + 16 * (tid + NT * u));
    }
    if (tid < 3 * CHUNK / 4) ptail = bload16(rr, REC_EG_OFF + 16 * tid);
  };

  // 4 tokens x VEC elements -> VEC rows of a transposed [element][token] LDS matrix
  auto store_transposed = [&](in_t* dst, const u32x4 (&blk4)[4], int row0, int tok0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      if constexpr (MODE == MODE_BF16) {
        const u32x2 pair = {pack_halves(blk4[0][j >> 1], blk4[1][j >> 1], j & 1),
                            pack_halves(blk4[2][j >> 1], blk4[3][j >> 1], j & 1)};
        *reinterpret_cast<u32x2*>(dst + (row0 + j) * LDT + tok0) = pair;
      } else {
        const u32x4 col4 = {blk4[0][j], blk4[1][j], blk4[2][j], blk4[3][j]};
        *reinterpret_cast<u32x4*>(dst + (row0 + j) * LDT + tok0) = col4;
      }
    }
  };

  auto store_lds = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int blk = tid + NT * u;
      if (blk < KBLK) {
        int rb, cb;
        kblk(blk, rb, cb);
#pragma unroll
        for (int u4 = 0; u4 < 4; ++u4) {
          *reinterpret_cast<u32x4*>(sK + (4 * rb + u4) * LDK + VEC * cb) = pk[u][u4];
          if constexpr (WITH_OUT) *reinterpret_cast<u32x4*>(sQ + (4 * rb + u4) * LDK + VEC * cb) = pq[u][u4];
        }
        if constexpr (!KT_TR) store_transposed(sKt, pk[u], VEC * cb, 4 * rb);
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int blk = tid + NT * u;
      if (blk < VBLK) {
        int rb, cb;
        vblk(blk, rb, cb);
        store_transposed(sVt, pv[u], VEC * cb, 4 * rb);
      }
    }
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int vid = tid + NT * u;
      const int row = vid >> 4, piece = (vid & 15) ^ swz<256>(vid >> 4);  // record rows are swizzled
      *reinterpret_cast<u32x4*>(sTP + row * DROW_BYTES + 16 * piece) = pt[u];
      if constexpr (WITH_OUT) *reinterpret_cast<u32x4*>(sPP + row * DROW_BYTES + 16 * piece) = pp[u];
    }
    if (tid < 3 * CHUNK / 4) reinterpret_cast<u32x4*>(sTail)[tid] = ptail;
  };

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

  if (c_begin < c_end) {
    issue_loads(c_begin);
    store_lds();
  }
  __syncthreads();

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * CHUNK;
    const bool more = c + 1 < c_end;
    if (more) issue_loads(c + 1);
    // ACC: the outputs already there and the weights of this chunk's rows, loaded now so that the
    // adds at the end of the chunk never wait on a memory round trip (a load issued after the
    // output stores would also wait for them: loads and stores share one in-order counter)
    float acc_old[ACC ? 16 : 1], acc_w[ACC ? 16 : 1];
    if constexpr (ACC) {
      const rsrc_t ra = make_rsrc(ob_ + static_cast<size_t>(t0) * rowO, static_cast<long long>(T - t0) * rowO);
      const int abase = 4 * gq * rowO + (h * DV + vcol) * 4;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 16 * mt + 4 * gq + i;
          acc_old[4 * mt + i] = __uint_as_float(bload4(ra, abase + (16 * mt + i) * rowO));
          acc_w[4 * mt + i] = t < T ? a.lam[((static_cast<size_t>(b) * T + t) * H + h) * a.lam_L + a.lam_level] : 0.f;
        }
      }
    }

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
      const f32x4 eg = *reinterpret_cast<const f32x4*>(sEG + 16 * mt + 4 * gq);
      float vv[4] = {0.f, 0.f, 0.f, 0.f};
      if (!ident) {
        const in_t* vp = sVt + (16 * w + ln) * LDT + 16 * mt + 4 * gq;
        if constexpr (MODE == MODE_BF16) {
          const u32x2 x = *reinterpret_cast<const u32x2*>(vp);
          vv[0] = __uint_as_float(x[0] << 16);
          vv[1] = __uint_as_float(x[0] & 0xFFFF0000u);
          vv[2] = __uint_as_float(x[1] << 16);
          vv[3] = __uint_as_float(x[1] & 0xFFFF0000u);
        } else {
          const f32x4 x = *reinterpret_cast<const f32x4*>(vp);
          vv[0] = x[0]; vv[1] = x[1]; vv[2] = x[2]; vv[3] = x[3];
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Rr[mt][i] = vv[i] - eg[i] * acc[i];
    }
    DF Rb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Rb[kb] = TR::mk(frag_from_acc(Rr[2 * kb], Rr[2 * kb + 1]));

    // ---- U = T' R  (T' is lower triangular: rows 0..31 need only tokens 0..31) ----
    f32x4 U[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      U[mt] = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb == 0 || mt >= 2) U[mt] = TR::mma_dd(U[mt], TR::ldd(sTP, 16 * mt, 32 * kb, lane), Rb[kb]);
    }

    // ---- O = diag(e^g) Q S + P U ----
    if constexpr (WITH_OUT) {
      f32x4 O[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) acc = TR::mma_xd(acc, TR::ldx(sQ, LDK, 16 * mt, 32 * kb, lane), Sb[kb]);
        O[mt] = acc * *reinterpret_cast<const f32x4*>(sEG + 16 * mt + 4 * gq);
      }

      DF Ub[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) Ub[kb] = TR::mk(frag_from_acc(U[2 * kb], U[2 * kb + 1]));
      const rsrc_t ro = make_rsrc(ob_ + static_cast<size_t>(t0) * rowO, static_cast<long long>(T - t0) * rowO);
      const int obase = 4 * gq * rowO + (h * DV + vcol) * 4;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if (kb == 0 || mt >= 2) O[mt] = TR::mma_dd(O[mt], TR::ldd(sPP, 16 * mt, 32 * kb, lane), Ub[kb]);
        if constexpr (ACC) {
#pragma unroll
          for (int i = 0; i < 4; ++i)  // rows past T: weight 0, and the store falls outside the buffer
            bstore_f32(acc_old[4 * mt + i] + acc_w[4 * mt + i] * O[mt][i], ro, obase + (16 * mt + i) * rowO);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) bstore_f32(O[mt][i], ro, obase + (16 * mt + i) * rowO);
        }
      }
    }

    // ---- S <- e^{g_C} S + K^T diag(e^{g_C - g}) U ----
    const float gC = sEG[CHUNK - 1];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) U[mt] *= *reinterpret_cast<const f32x4*>(sEGC + 16 * mt + 4 * gq);
    DF Ud[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Ud[kb] = TR::mk(frag_from_acc(U[2 * kb], U[2 * kb + 1]));
    // KT_TR: lane (gq, ln) takes K[32 kb + kslot(gq, j)][16 mt + ln], j = 0..7, from two transposed reads
    // of four consecutive token rows each: it supplies the 8-byte block of row 32 kb + 4 gq (+ 16) +
    // (ln >> 2), keys 16 mt + 4 (ln & 3) + 0..3
    auto ldKT = [&](int mt, int kb) __attribute__((always_inline)) {
      if constexpr (KT_TR) {
        typedef short i16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const in_t* p = sK + (32 * kb + 4 * gq + (ln >> 2)) * LDK + 16 * mt + 4 * (ln & 3);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 16 * LDK));
        return __builtin_bit_cast(typename TR::XF, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        return TR::ldx(sKt, LDT, 16 * mt, 32 * kb, lane);
      }
    };
#pragma unroll
    for (int mt = 0; mt < DK / 16; ++mt) {
      S[mt] *= gC;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) S[mt] = TR::mma_xd(S[mt], ldKT(mt, kb), Ud[kb]);
    }
    // Both barriers guard LDS only: the output stores and the next chunk's prefetch loads stay
    // in flight (store_lds waits for the loads it consumes, not for the stores issued after them).
    lds_barrier();  // every read of this chunk's LDS is done
    if (more) store_lds();
    lds_barrier();
  }

  // end state
  if (fin_base && (!a.fin_last_only || seg == nseg - 1)) {
    float* F = fin_base + (static_cast<size_t>(bh) * fin_segs + (a.fin_last_only ? 0 : seg)) * DK * a.fin_ld;
#pragma unroll
    for (int mt = 0; mt < DK / 16; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) F[(16 * mt + 4 * gq + i) * a.fin_ld + col] = S[mt][i];
    }
  }
}

// Start state of every segment: X_0 = init (or 0), X_{s+1} = M_s X_s + N_s (the fold of the
// segment maps; the associative scan of the KATA page, 2.3, and the HLA page, 4).
// One workgroup per (b, h, 16-column tile of dv), four waves, each owning DK/64 row tiles of
// 16 rows. The products run on the fp32 MFMA (v_mfma_f32_16x16x4_f32, full fp32 products).
// The contraction is taken in the order k = 16 kk + 4 gq + s (s = 0..3 over four MFMAs), so a
// lane's A operands for four MFMAs are one 16-byte load of a row of M and its B operands one
// 16-byte LDS read of X^T, kept in LDS with a padded row pitch. X^T is double-buffered: one
// barrier per segment step.
template <int DK>
__global__ __launch_bounds__(256) void scan_starts_kernel(const float* __restrict__ maps,
                                                          const float* __restrict__ init,
                                                          float* __restrict__ starts, int DV, int segs) {
  constexpr int XP = DK + 4;  // padded pitch of X^T rows (floats)
  __shared__ __align__(16) float XT[2][16 * XP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gq = lane >> 4, ln = lane & 15;
  const int c0 = blockIdx.x * 16, bh = blockIdx.y;
  const int LDM = DK + DV;
  for (int o = tid; o < DK * 16; o += 256) {
    const int r = o >> 4, j = o & 15;
    const float x = init ? init[static_cast<size_t>(bh) * DK * DV + r * DV + c0 + j] : 0.f;
    XT[0][j * XP + r] = x;
    starts[(static_cast<size_t>(bh) * segs) * DK * DV + r * DV + c0 + j] = x;
  }
  __syncthreads();
  for (int s = 0; s + 1 < segs; ++s) {
    const float* M = maps + (static_cast<size_t>(bh) * (segs - 1) + s) * DK * LDM;
    const float* X = XT[s & 1];
    float* Xn = XT[(s + 1) & 1];
    float* out = starts + (static_cast<size_t>(bh) * segs + s + 1) * DK * DV;
#pragma unroll
    for (int u = 0; u < DK / 64; ++u) {
      const int mt = w + 4 * u;
      f32x4 acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = M[static_cast<size_t>(16 * mt + 4 * gq + i) * LDM + DK + c0 + ln];  // N
      const float* Mrow = M + static_cast<size_t>(16 * mt + ln) * LDM + 4 * gq;
      const float* Xrow = X + ln * XP + 4 * gq;
      // from a zero start, X_1 = N_0: M_0 is never computed (the map walk skips it) or read
      if (init || s > 0) {
#pragma unroll 4
        for (int kk = 0; kk < DK / 16; ++kk) {
          const f32x4 a4 = *reinterpret_cast<const f32x4*>(Mrow + 16 * kk);
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(Xrow + 16 * kk);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[q], b4[q], acc, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) out[static_cast<size_t>(16 * mt + 4 * gq + i) * DV + c0 + ln] = acc[i];
      *reinterpret_cast<f32x4*>(Xn + ln * XP + 16 * mt + 4 * gq) = acc;  // X^T[col][rows 16mt + 4gq + 0..3]
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
constexpr int NCOLS_STATE = 64;  // state columns per workgroup (4 waves x 16)

template <int MODE, int DK, bool WITH_OUT, bool AUG, bool ACC = false>
static hipError_t launch_state_t(int nwg, const StateArgs& a, hipStream_t stream) {
  return launch_kernel(state_kernel<MODE, DK, WITH_OUT, AUG, ACC>, dim3(nwg), dim3(256), stream, a);
}

template <bool WITH_OUT, bool AUG>
static hipError_t dispatch_state(int mode, int dk, int nwg, const StateArgs& a, hipStream_t stream) {
  if (mode == MODE_BF16) {
    switch (dk) {
      case 64: return launch_state_t<MODE_BF16, 64, WITH_OUT, AUG>(nwg, a, stream);
      case 128: return launch_state_t<MODE_BF16, 128, WITH_OUT, AUG>(nwg, a, stream);
      case 256: return launch_state_t<MODE_BF16, 256, WITH_OUT, AUG>(nwg, a, stream);
    }
  } else {
    switch (dk) {
      case 64: return launch_state_t<MODE_F32, 64, WITH_OUT, AUG>(nwg, a, stream);
      case 128: return launch_state_t<MODE_F32, 128, WITH_OUT, AUG>(nwg, a, stream);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_state_seq(int mode, const Dims& d, const void* q, const void* k, const void* v,
                            const uint8_t* rec, const float* init, float* out, float* fin,
                            hipStream_t stream) {
  const int ncg = d.dv / NCOLS_STATE;
  if (state_dma_supported(mode, d.dk))
    return launch_state_dma(true, false, d.dk, ncg * d.B * d.H, q, k, v, rec, d.T, d.H, d.dv, d.nc, d.nc, init, 1, out,
                            fin, d.dv, 1, 0, ncg, 1, stream);
  StateArgs a{q, k, v, rec, d.T, d.H, d.dv, d.nc, d.nc, init, 1, out, fin, d.dv, 1, 0, ncg, 1};
  return dispatch_state<true, false>(mode, d.dk, ncg * d.B * d.H, a, stream);
}

hipError_t launch_scan_maps(int mode, const Dims& d, const void* k, const void* v, const uint8_t* rec,
                            int seg_chunks, int segs, float* maps, bool zero_start, hipStream_t stream) {
  const int ncg = (d.dk + d.dv) / NCOLS_STATE;
  if (state_dma_supported(mode, d.dk))
    return launch_state_dma(false, true, d.dk, ncg * (segs - 1) * d.B * d.H, nullptr, k, v, rec, d.T, d.H, d.dv, d.nc,
                            seg_chunks, nullptr, 1, nullptr, maps, d.dk + d.dv, segs - 1, 0, ncg, segs - 1, stream, 1, 0,
                            zero_start ? 1 : 0);
  StateArgs a{nullptr, k, v, rec, d.T, d.H, d.dv, d.nc, seg_chunks, nullptr, 1, nullptr, maps, d.dk + d.dv,
              segs - 1, 0, ncg, segs - 1};
  a.skip_ident0 = zero_start ? 1 : 0;
  return dispatch_state<false, true>(mode, d.dk, ncg * (segs - 1) * d.B * d.H, a, stream);
}

hipError_t launch_scan_starts(const Dims& d, const float* maps, const float* init, int segs, float* starts,
                              hipStream_t stream) {
  dim3 grid(d.dv / 16, d.B * d.H);
  switch (d.dk) {
    case 64: return launch_kernel(scan_starts_kernel<64>, grid, dim3(256), stream, maps, init, starts, d.dv, segs);
    case 128: return launch_kernel(scan_starts_kernel<128>, grid, dim3(256), stream, maps, init, starts, d.dv, segs);
    case 256: return launch_kernel(scan_starts_kernel<256>, grid, dim3(256), stream, maps, init, starts, d.dv, segs);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_apply(int mode, const Dims& d, const void* q, const void* k, const void* v,
                             const uint8_t* rec, int seg_chunks, int segs, const float* starts, float* out,
                             float* fin, hipStream_t stream) {
  const int ncg = d.dv / NCOLS_STATE;
  if (state_dma_supported(mode, d.dk))
    return launch_state_dma(true, false, d.dk, ncg * segs * d.B * d.H, q, k, v, rec, d.T, d.H, d.dv, d.nc, seg_chunks,
                            starts, segs, out, fin, d.dv, 1, 1, ncg, segs, stream);
  StateArgs a{q, k, v, rec, d.T, d.H, d.dv, d.nc, seg_chunks, starts, segs, out, fin, d.dv, 1, 1, ncg, segs};
  return dispatch_state<true, false>(mode, d.dk, ncg * segs * d.B * d.H, a, stream);
}

// Log-linear prefill, one scale: half-blocks of `half` chunks, left ones (even) and right ones (odd).
template <bool WITH_OUT, bool ACC>
static hipError_t dispatch_scale(int mode, int dk, int nwg, const StateArgs& a, hipStream_t stream) {
  if (mode == MODE_BF16) {
    switch (dk) {
      case 64: return launch_state_t<MODE_BF16, 64, WITH_OUT, false, ACC>(nwg, a, stream);
      case 128: return launch_state_t<MODE_BF16, 128, WITH_OUT, false, ACC>(nwg, a, stream);
      case 256: return launch_state_t<MODE_BF16, 256, WITH_OUT, false, ACC>(nwg, a, stream);
    }
  } else {
    switch (dk) {
      case 64: return launch_state_t<MODE_F32, 64, WITH_OUT, false, ACC>(nwg, a, stream);
      case 128: return launch_state_t<MODE_F32, 128, WITH_OUT, false, ACC>(nwg, a, stream);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_loglinear_left(int mode, const Dims& d, const void* k, const void* v, const uint8_t* rec,
                                 int nscale, const int* half, const int* nleft, const long long* ends_off,
                                 float* ends, hipStream_t stream) {
  if (nscale < 1 || nscale > kMaxScales) return hipErrorInvalidValue;
  const int ncg = d.dv / NCOLS_STATE;
  StateArgs a{nullptr, k, v, rec, d.T, d.H, d.dv, d.nc, half[0], nullptr, 1, nullptr, ends, d.dv, nleft[0], 0, ncg,
              nleft[0]};
  a.seg_mul = 2;
  a.seg_add = 0;
  a.nscale = nscale;
  int nwg = 0;
  for (int i = 0; i < nscale; ++i) {
    a.scale_wg[i] = nwg;
    a.scale_half[i] = half[i];
    a.scale_nseg[i] = nleft[i];
    a.scale_fin_off[i] = ends_off[i];
    nwg += ncg * nleft[i] * d.B * d.H;
  }
  a.scale_wg[nscale] = nwg;
  return dispatch_scale<false, false>(mode, d.dk, nwg, a, stream);
}

hipError_t launch_loglinear_right(int mode, const Dims& d, const void* q, const void* k, const uint8_t* rec, int half,
                                  int nright, const float* ends, int nleft, const float* lam, int L, int level,
                                  float* out, hipStream_t stream) {
  const int ncg = d.dv / NCOLS_STATE;
  StateArgs a{q, k, nullptr, rec, d.T, d.H, d.dv, d.nc, half, ends, nleft, out, nullptr, d.dv, 1, 0, ncg, nright};
  a.seg_mul = 2;
  a.seg_add = 1;
  a.lam = lam;
  a.lam_L = L;
  a.lam_level = level;
  return dispatch_scale<true, true>(mode, d.dk, ncg * nright * d.B * d.H, a, stream);
}

hipError_t launch_copy_or_zero(const float* src, float* dst, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  return launch_kernel(copy_or_zero_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256),
                       stream, src, dst, n);
}

}  // namespace kla
