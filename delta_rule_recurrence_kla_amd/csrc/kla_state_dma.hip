// Inter-chunk state kernels, bf16 inputs, dk in {64, 128}: the DMA-fed variants.
//
// Same mathematics as state_kernel in kla_state.hip (see there; KLA page, "KLA update
// rule" and "Implementation"):
//   R  = V - diag(e^g) K S,   U = T' R,   O = diag(e^g) Q S + P U,
// with one workgroup per (b, h, 64 state columns), 16 columns per wave, and the state held in
// MFMA accumulator registers for the whole walk over the chunks. Two kernels:
//  * state_map_kernel walks a segment without outputs and leaves its end state: on the
//    augmented state [I | 0] that is the segment's affine map [M | N] (the scan's first phase).
//    One compute wave per 16 columns and a copy wave;
//  * state_walk_kernel walks with outputs (the sequential path, the scan's walk from every
//    segment's start, and the scales of log-linear KLA): per 16 columns one wave runs the
//    recurrence and another the output products, with a copy wave (see the comment above it).
//
// What both share is how a chunk's operands reach LDS and registers:
//  * every input of chunk c+1 (rows of K, Q, V and the chunk record) is copied into LDS by
//    buffer_load ... lds while chunk c is computed (double-buffered), so no registers hold
//    prefetched data;
//  * a copy wave issues those copies. A wave cannot issue past a memory instruction that the
//    CU has not yet accepted, and in these kernels a 1 KB copy is accepted only every 50 or
//    so cycles: 53 copies per chunk held each compute wave for about a thousand cycles when
//    the compute waves shared them. The copy wave takes that wait instead, and the compute
//    waves issue no memory instructions but their 16-byte output stores (which they never
//    wait for);
//  * rows land in the swizzled layout of kla_device.h: the DMA picks, per lane, the
//    source piece that belongs at its fixed destination;
//  * K^T operands and the accumulator-layout view of V come from transposed LDS reads
//    (ds_read_b64_tr_b16) of the row-major rows, so no transposed copies are built;
//  * P = tril(e^{g_r - g_i} Q K^T) is formed from the Q and K rows already in LDS (twelve
//    16 x 16 tiles, three per slice, shared through LDS), so the chunk record carries only T'
//    (without its zero quadrant) and the gates: 12.75 KB instead of 33.5 KB per chunk, the
//    larger part of what the kernel streams in;
//  * rows of every 64-row tile (tokens, and state rows) are taken in the permuted order
//    tok(m, r) = 32(m >> 1) + 8(r >> 2) + 4(m & 1) + (r & 3) for MFMA tile m, tile row r.
//    An accumulator pair (tiles 2a, 2a + 1) then gives each lane eight consecutive
//    indices 32a + 8(lane >> 4) + 0..7 as the contraction slots of the next product, so
//    every row-major operand fragment is one contiguous 16-byte LDS read.
#include <algorithm>

#include "kla_device.h"
#include "kla_launch.h"

namespace kla {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

struct StateDmaArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* rec;
  int T, H, DV, nc;
  int seg_chunks;
  const float* init;
  int init_segs;
  float* out;
  float* fin;
  int fin_ld;
  int fin_segs;
  int fin_last_only;
  int ncg;
  int nseg;
  // Segment s walks chunks [(s * seg_mul + seg_add) * seg_chunks, + seg_chunks): every segment
  // (1, 0), or every other one (2, 1) for the right half-blocks of a log-linear scale.
  int seg_mul;
  int seg_add;
  // Log-linear scale walks only (see state_walk_kernel): weights lam [B, T, H, lam_L] of level
  // lam_level, and wg_segs consecutive segments per workgroup.
  const float* lam;
  int lam_L;
  int lam_level;
  int wg_segs;
  // Map walks of a scan from a zero start: the workgroups of segment 0's identity columns exit
  // (the fold never reads M_0 then).
  int skip_ident0;
};

namespace {

// Row of 64-row tile block m (16-row MFMA tile m of four) taken by tile row r.
__device__ __forceinline__ int tok(int m, int r) {
  return 32 * (m >> 1) + 8 * (r >> 2) + 4 * (m & 1) + (r & 3);
}

__device__ __forceinline__ void dma16(rsrc_t r, uint8_t* lds_dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_dst, 16, voff, 0, 0, 0);
}

// 4 bytes per lane; lane i's dword lands at lds_dst + 4 i
__device__ __forceinline__ void dma4(rsrc_t r, void* lds_dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_dst, 4, voff, 0, 0, 0);
}

__device__ __forceinline__ void decode_wg_dma(int L, int ncg, int nunits, int& cg, int& unit) {
  if ((ncg * nunits) % (8 * ncg) == 0) {
    const int xcd = L & 7, slot = L >> 3;
    cg = slot % ncg;
    unit = (slot / ncg) * 8 + xcd;
  } else {
    cg = L % ncg;
    unit = L / ncg;
  }
}

}  // namespace

constexpr int MAP_THREADS = 320;  // four compute waves and the copy wave

template <int DK, bool AUG>
__global__ __launch_bounds__(MAP_THREADS) void state_map_kernel(StateDmaArgs a) {
  using TR = Tr<MODE_BF16>;
  constexpr int NCOLS = 64;
  constexpr int KRB = DK * 2;                 // bytes of a key row
  constexpr int VRB = NCOLS * 2;              // bytes of a value row (this workgroup's columns)
  constexpr int KBYTES = CHUNK * KRB;
  constexpr int VBYTES = CHUNK * VRB;
  constexpr int RECB = 13 * 1024;             // compact record (13056 bytes) rounded up to whole DMA blocks
  constexpr int K_OFF = 0;
  constexpr int V_OFF = K_OFF + KBYTES;
  constexpr int R_OFF = V_OFF + VBYTES;
  constexpr int BUF = R_OFF + RECB;           // one buffer
  static_assert(KRB == 128 || KRB == 256, "dk must be 64 or 128");
  static_assert(!AUG || DK % NCOLS == 0, "identity/value columns must not share a workgroup");

  // Two separate buffers (not one array indexed by parity): the compiler must see that the
  // copies into one buffer cannot alias the reads of the other, or it waits for the copies
  // before the first read and the overlap is lost.
  __shared__ __align__(1024) uint8_t lds0[BUF];
  __shared__ __align__(1024) uint8_t lds1[BUF];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index as a scalar
  const int gq = lane >> 4, ln = lane & 15;
  const int seg_chunks = a.seg_chunks, nseg = a.nseg, fin_segs = a.fin_segs;
  float* fin = a.fin;
  int cg, unit;
  decode_wg_dma(blockIdx.x, a.ncg, static_cast<int>(gridDim.x) / a.ncg, cg, unit);
  const int bh = unit / nseg, seg = unit - bh * nseg;
  const int H = a.H, T = a.T, DV = a.DV;
  const int b = bh / H, h = bh - b * H;
  const int col0 = cg * NCOLS;
  const int col = col0 + 16 * w + ln;
  const bool ident = AUG && col0 < DK;  // identity columns (they carry M), else value columns (N)
  if (AUG && ident && seg == 0 && a.skip_ident0) return;  // uniform over the workgroup, before any barrier
  const int vcol0 = AUG ? col0 - DK : col0;
  const int c_begin = (seg * a.seg_mul + a.seg_add) * seg_chunks;
  const int c_end = min(a.nc, c_begin + seg_chunks);

  const int rowK = H * DK * 2, rowV = H * DV * 2;
  const uint8_t* kb_ = static_cast<const uint8_t*>(a.k) + static_cast<size_t>(b) * T * rowK;
  const uint8_t* vb_ = static_cast<const uint8_t*>(a.v) + static_cast<size_t>(b) * T * rowV;

  constexpr int KPR = KRB / 16, KRPB = 1024 / KRB;  // pieces per key row, key rows per 1 KB block
  constexpr int VPR = VRB / 16, VRPB = 1024 / VRB;

  if (wu == 4) {
    // The copy wave. Chunk c's rows of K, Q and V and its record go into buffer B, one
    // 1 KB block per instruction; each lane fetches the source piece that belongs at its
    // fixed destination in the swizzled layout. Out-of-range rows of a ragged last chunk
    // read as zeros. Chunk c + 1 is copied while chunk c is computed; the wave then meets
    // the compute waves at their barriers (the P barrier and the end of the chunk), having
    // waited for its copies before the second.
    auto copy_chunk = [&](int c, uint8_t* B) __attribute__((always_inline)) {
      const int t0 = c * CHUNK;
      const rsrc_t rr = make_rsrc_wu(a.rec + (static_cast<size_t>(bh) * a.nc + c) * CREC_BYTES, CREC_BYTES);
#pragma unroll
      for (int m = 0; m < RECB / 1024; ++m) dma16(rr, B + R_OFF + 1024 * m, 1024 * m + 16 * lane);
      const rsrc_t rk = make_rsrc_wu(kb_ + static_cast<size_t>(t0) * rowK, static_cast<long long>(T - t0) * rowK);
#pragma unroll
      for (int blk = 0; blk < KBYTES / 1024; ++blk) {
        const int row = blk * KRPB + lane / KPR;
        const int off = row * rowK + h * DK * 2 + 16 * ((lane % KPR) ^ swz<KRB>(row));
        dma16(rk, B + K_OFF + 1024 * blk, off);
      }
      if (!ident) {
        const rsrc_t rv = make_rsrc_wu(vb_ + static_cast<size_t>(t0) * rowV, static_cast<long long>(T - t0) * rowV);
#pragma unroll
        for (int blk = 0; blk < VBYTES / 1024; ++blk) {
          const int row = blk * VRPB + lane / VPR;
          dma16(rv, B + V_OFF + 1024 * blk, row * rowV + (h * DV + vcol0) * 2 + 16 * ((lane % VPR) ^ swz<VRB>(row)));
        }
      }
    };
    if (c_begin < c_end) copy_chunk(c_begin, lds0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    for (int c = c_begin; c < c_end; ++c) {
      if (c + 1 < c_end) copy_chunk(c + 1, ((c + 1 - c_begin) & 1) ? lds1 : lds0);
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    return;
  }

  // Per-lane LDS offsets of the operand reads. Both swizzles ignore row bits 2 and 5, the
  // bits that a tile index adds to a permuted row (tok(m, r) = tok(0, r) + 32(m >> 1) +
  // 4(m & 1)), so every read below is one of these lane offsets plus a constant.
  int oK[DK / 32], oT[DK / 32], oRt[2], oRb[2][2];
#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb) {
    oK[kb] = swz_off<KRB>(tok(0, ln), 64 * kb + 16 * gq);                   // K, Q rows
    oT[kb] = swz_off<KRB>(8 * gq + (ln >> 2), 2 * (32 * kb + 8 * (ln & 3)));  // K^T blocks
  }
#pragma unroll
  for (int hl = 0; hl < 2; ++hl) {
    oRt[hl] = CREC_TOP_OFF + swz_off<128>(tok(0, ln), 64 * hl + 16 * gq);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) oRb[kb][hl] = CREC_BOT_OFF + swz_off<256>(tok(0, ln), 128 * hl + 64 * kb + 16 * gq);
  }
  const int oV = swz_off<VRB>(8 * gq + (ln >> 2), 2 * (16 * w + 4 * (ln & 3)));
  auto mrow = [](int m) { return 32 * (m >> 1) + 4 * (m & 1); };

  // Operand fragments. ds_read_b64_tr_b16: lane (gq, ln) supplies the address of an 8-byte
  // block and receives, for j = 0..3, element (ln & 3) of the block of lane 4j + (ln >> 2)
  // of its 16-lane group.
  //  fragK:  row tok(m, ln) of K or Q, contraction columns 32 kb + 8 gq + 0..7 (one 16-byte read)
  //  fragKT: element [tok(m, ln)][32 kb + 8 gq + j] = K[32 kb + 8 gq + j][tok(m, ln)]
  //          (lane blocks: row 32 kb + 8 gq + (ln >> 2) (+4), columns 32(m >> 1) + 8(ln & 3) + 4(m & 1))
  //  fragR:  hi and lo halves of row tok(m, ln) of a lower-triangular matrix in the compact
  //          record layout (T', or P), columns 32 kb + 8 gq + 0..7 (kb = 0 when m < 2)
  //  trV:    lane (gq, ln) gets V[tok(m, 4 gq + j)][16 w + ln], j = 0..3 (accumulator layout)
  auto fragK = [&](const uint8_t* X, int m, int kb) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(X + oK[kb] + mrow(m) * KRB));
  };
  auto fragKT = [&](const uint8_t* X, int m, int kb) __attribute__((always_inline)) {
    const uint8_t* p = X + oT[m >> 1] + 32 * kb * KRB + 8 * (m & 1);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * KRB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto fragR = [&](const uint8_t* X, int m, int kb) __attribute__((always_inline)) {
    const uint8_t* p = m < 2 ? X + oRt[0] + 4 * (m & 1) * 128 : X + oRb[kb][0] + 4 * (m & 1) * 256;
    const int lo = m < 2 ? oRt[1] - oRt[0] : oRb[kb][1] - oRb[kb][0];
    S8 r;
    r.h = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
    r.l = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p + lo));
    return r;
  };
  auto trV = [&](const uint8_t* X, int m) __attribute__((always_inline)) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(X + oV + mrow(m) * VRB));
    return __builtin_bit_cast(u32x2, v);
  };

  // start state
  f32x4 S[DK / 16];
#pragma unroll
  for (int mt = 0; mt < DK / 16; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = tok(mt, 4 * gq + i);
      S[mt][i] = (ident && r == col) ? 1.f : 0.f;
    }
  }

  // one chunk computed from buffer B (while the copy wave fills the other buffer)
  auto chunk = [&](const uint8_t* B) __attribute__((always_inline)) {
    const uint8_t* sK = B + K_OFF;
    const uint8_t* sV = B + V_OFF;
    const uint8_t* sR = B + R_OFF;
    const float* sEG = reinterpret_cast<const float*>(sR + CREC_EG_OFF);
    const float* sEGC = reinterpret_cast<const float*>(sR + CREC_EGC_OFF);

    // ---- S as B operand ----
    S8 Sb[DK / 32];
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) Sb[kb] = split8(frag_from_acc(S[2 * kb], S[2 * kb + 1]));

    // ---- R = V - diag(e^g) K S ----
    f32x4 Rr[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) acc = TR::mma_xd(acc, fragK(sK, mt, kb), Sb[kb]);
      const f32x4 eg = *reinterpret_cast<const f32x4*>(sEG + tok(mt, 4 * gq));
      f32x4 vv = zero4();
      if (!ident) {
        const u32x2 x = trV(sV, mt);
        vv[0] = __uint_as_float(x[0] << 16);
        vv[1] = __uint_as_float(x[0] & 0xFFFF0000u);
        vv[2] = __uint_as_float(x[1] << 16);
        vv[3] = __uint_as_float(x[1] & 0xFFFF0000u);
      }
      Rr[mt] = vv - eg * acc;
    }
    S8 Rb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Rb[kb] = split8(frag_from_acc(Rr[2 * kb], Rr[2 * kb + 1]));

    // ---- U = T' R (lower triangular: rows 0..31 need only tokens 0..31) ----
    f32x4 U[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      U[mt] = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (kb == 0 || mt >= 2) U[mt] = TR::mma_dd(U[mt], fragR(sR, mt, kb), Rb[kb]);
    }

    // ---- S <- e^{g_C} S + K^T diag(e^{g_C - g}) U ----
    f32x4 Ue[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) Ue[mt] = U[mt] * *reinterpret_cast<const f32x4*>(sEGC + tok(mt, 4 * gq));
    S8 Ud[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) Ud[kb] = split8(frag_from_acc(Ue[2 * kb], Ue[2 * kb + 1]));
    const float gC = sEG[CHUNK - 1];
#pragma unroll
    for (int mt = 0; mt < DK / 16; ++mt) {
      S[mt] *= gC;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) S[mt] = TR::mma_xd(S[mt], fragKT(sK, mt, kb), Ud[kb]);
    }
    // end of chunk: this wave's reads of buffer B are done (lgkmcnt) and, past the barrier,
    // every wave's are, and the copy wave's copies of chunk c + 1 have landed
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  asm volatile("s_barrier" ::: "memory");  // the first chunk has landed
  for (int c = c_begin; c < c_end; c += 2) {
    chunk(lds0);
    if (c + 1 < c_end) chunk(lds1);
  }

  if (fin && (!a.fin_last_only || seg == nseg - 1)) {
    float* F = fin + (static_cast<size_t>(bh) * fin_segs + (a.fin_last_only ? 0 : seg)) * DK * a.fin_ld;
#pragma unroll
    for (int mt = 0; mt < DK / 16; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) F[(tok(mt, 4 * gq) + i) * a.fin_ld + col] = S[mt][i];
    }
  }
}

// ---------------------------------------------------------------------------
// The walk with outputs (sequential path, the scan's walk from each segment's start, and the
// scales of log-linear KLA).
//
// Per 16-column slice of the workgroup's 64 state columns the chunk's work splits into the
// recurrence chain, which carries the state from chunk to chunk,
//   R = V - diag(e^g) K S,  U = T' R,  S <- e^{g_C} S + K^T diag(e^{g_C - g}) U,
// and work off that chain, which only produces outputs: P = tril(e^{g_r - g_i} Q K^T), Q S and
// O = diag(e^g) Q S + P U. Each slice gets two waves on one SIMD, plus one copy wave for the
// workgroup:
//  * the recurrence wave (waves 0..3) runs the chain. It hands U, split hi/lo, to the output
//    wave through LDS, and at the end of each chunk the hi/lo split of the new S, which it
//    keeps in registers for its own next chunk;
//  * the output wave (waves 4..7) computes its three P tiles and reads that split of S while the
//    recurrence wave computes U, then Q S, P U, and stores its output tiles;
//  * the copy wave (wave 8) copies chunk c+1's rows of K and Q and its record into the other
//    half of a double-buffered LDS area while chunk c is computed. V rows are read only by the
//    recurrence wave, before the mid-chunk barrier, so they have one buffer, which the copy
//    wave refills after that barrier.
// Two barriers per chunk: the mid-chunk one publishes U and every output wave's P tiles (and
// tells the recurrence wave the output wave is done with the S split it may now overwrite);
// the end-of-chunk one follows the state update and the copies. The products are those of the
// single-wave walk, in the same order, so the results are the same bit for bit; split this way
// the walk takes about 3% less time on the LM-layer shape (the chain's latency dominates).
// LDS: 2 x 45,824 B (K, Q, record) + 8 KB (V) + 12 KB (P) + 16 KB (U split) + 32 KB (S split)
// = 161,280 B, so the record's last copy is cut to its 768 remaining bytes (the log-linear walks
// add 1 KB of output weights).
//
// LL: one chunk scale s of log-linear KLA (Log-Linear page, "Mathematical formalization": the
// Fenwick buckets; level l = 7 + s holds, seen from a token of chunk c whose bit s is set, the
// 2^s chunks below c's bit s). Let C_l(t) be the KLA output of token t from the tokens whose
// level seen from t is at most l. For l = 7 + s these are the tokens from the start of the
// aligned block of 2^(s+1) chunks that holds t, so C_l is the output of a KLA walk restarted
// from zero at every multiple of 2^(s+1) chunks. Then
//   o_t = sum_l lambda^(l) (C_l - C_{l-1}) = sum_l (lambda^(l) - lambda^(l+1)) C_l,
// and on a chunk whose bit s is clear C_{7+s} = C_{6+s}. So the scale's walk covers only its
// right half-blocks (bit s set), one segment each; a segment starts from the state that the
// walk of scale s - 1 leaves at the end of the left sibling (its own right half-block of even
// index), and its outputs are added to out with the weight lambda^(7+s) - lambda^(7+s'), s' the
// next set bit of the chunk index above s (lambda^(7+s) alone if there is none). Each segment
// of even index leaves its end state for scale s + 1. Scale 0 walks each pair of chunks from
// zero, the left chunk without outputs (lead = 1). The chunk-local term P T' V that every C_l
// carries sums over a chunk's scales to lambda^(7 + lowest set bit of c) P T' V, which the
// intra-chunk kernel takes off its pairs. A workgroup walks wg_segs consecutive segments one
// after another, so the copies run on across segment boundaries.
constexpr int WALK_THREADS = 576;  // four recurrence waves, four output waves, one copy wave
// the walk's kinds: with outputs, a log-linear scale s >= 1, log-linear scale 0 (lead chunks)
constexpr int WALK_PLAIN = 0, WALK_LL = 1, WALK_LL_PAIRS = 2;

template <int DK, int WK>
__global__ __launch_bounds__(WALK_THREADS) void state_walk_kernel(StateDmaArgs a) {
  constexpr bool LL = WK != WALK_PLAIN;
  constexpr bool PAIRS = WK == WALK_LL_PAIRS;
  using TR = Tr<MODE_BF16>;
  constexpr int NCOLS = 64;
  constexpr int KRB = DK * 2;
  constexpr int VRB = NCOLS * 2;
  constexpr int KBYTES = CHUNK * KRB;
  constexpr int VBYTES = CHUNK * VRB;
  constexpr int RECB = CREC_BYTES;  // the last 1 KB copy is cut to the record's 768 remaining bytes
  constexpr int K_OFF = 0;
  constexpr int Q_OFF = K_OFF + KBYTES;
  constexpr int R_OFF = Q_OFF + KBYTES;
  constexpr int BUF = R_OFF + RECB;
  constexpr int KPR = KRB / 16, KRPB = 1024 / KRB;
  constexpr int VPR = VRB / 16, VRPB = 1024 / VRB;

  static_assert(BUF % 256 == 0, "buffers start on the 256-byte bank period");
  __shared__ __align__(256) uint8_t lds0[BUF];
  __shared__ __align__(256) uint8_t lds1[BUF];
  __shared__ __align__(256) uint8_t ldsV[VBYTES];  // V rows: read before the mid-chunk barrier only
  __shared__ __align__(256) uint8_t ldsP[CREC_EG_OFF];
  __shared__ __align__(16) u32x4 ldsUb[4][2][2][64];         // [slice][kb][hi, lo][lane]: U split, 8 KB
  __shared__ __align__(16) u32x4 ldsSb[4][DK / 32][2][64];   // [slice][kb][hi, lo][lane]: S split, 32 KB
  // LL: the chunk's two output weights per token, [buffer][lambda^(7+s), lambda^(7+s')][token], 1 KB
  __shared__ __align__(256) float ldsL[LL ? 2 : 1][2][LL ? CHUNK : 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int sl = wu & 3;
  const int gq = lane >> 4, ln = lane & 15;
  int cg, unit;
  decode_wg_dma(blockIdx.x, a.ncg, static_cast<int>(gridDim.x) / a.ncg, cg, unit);
  // segments [i0, i1) of this workgroup: one, except for the log-linear scales
  const int ngrp = LL ? (a.nseg + a.wg_segs - 1) / a.wg_segs : a.nseg;
  const int bh = unit / ngrp, grp = unit - bh * ngrp;
  const int i0 = LL ? grp * a.wg_segs : grp;
  const int i1 = LL ? min(a.nseg, i0 + a.wg_segs) : grp + 1;
  const int seg = i0;
  const int H = a.H, T = a.T, DV = a.DV;
  const int b = bh / H, h = bh - b * H;
  const int col0 = cg * NCOLS;
  const int col = col0 + 16 * sl + ln;
  const int c_begin = (seg * a.seg_mul + a.seg_add) * a.seg_chunks;
  const int c_end = min(a.nc, c_begin + a.seg_chunks);
  // LL: segment i covers chunks [seg_start(i), seg_end(i)), its first `lead` chunks without outputs
  const int lead = PAIRS ? 1 : 0;
  auto seg_begin = [&](int i) { return (i * a.seg_mul + a.seg_add) * a.seg_chunks; };
  auto seg_start = [&](int i) { return seg_begin(i) - lead; };
  auto seg_end = [&](int i) { return min(a.nc, seg_begin(i) + a.seg_chunks); };
  int nchunks = 0;
  if constexpr (LL)
    for (int i = i0; i < i1; ++i) nchunks += seg_end(i) - seg_start(i);
  const int rowK = H * DK * 2, rowV = H * DV * 2, rowO = H * DV * 4;
  const uint8_t* kb_ = static_cast<const uint8_t*>(a.k) + static_cast<size_t>(b) * T * rowK;
  const uint8_t* qb_ = static_cast<const uint8_t*>(a.q) + static_cast<size_t>(b) * T * rowK;
  const uint8_t* vb_ = static_cast<const uint8_t*>(a.v) + static_cast<size_t>(b) * T * rowV;
  uint8_t* ob_ = reinterpret_cast<uint8_t*>(a.out) + static_cast<size_t>(b) * T * rowO;

  if (wu == 8) {  // the copy wave, as in state_dma_kernel
    // chunk c's rows of K and Q and its record into buffer B; its V rows into the one V buffer
    auto copy_kqr = [&](int c, uint8_t* B) __attribute__((always_inline)) {
      const int t0 = c * CHUNK;
      const rsrc_t rr = make_rsrc_wu(a.rec + (static_cast<size_t>(bh) * a.nc + c) * CREC_BYTES, CREC_BYTES);
#pragma unroll
      for (int m = 0; m < CREC_BYTES / 1024; ++m) dma16(rr, B + R_OFF + 1024 * m, 1024 * m + 16 * lane);
      if (lane < (CREC_BYTES % 1024) / 16)
        dma16(rr, B + R_OFF + (CREC_BYTES / 1024) * 1024, (CREC_BYTES / 1024) * 1024 + 16 * lane);
      const rsrc_t rk = make_rsrc_wu(kb_ + static_cast<size_t>(t0) * rowK, static_cast<long long>(T - t0) * rowK);
      const rsrc_t rq = make_rsrc_wu(qb_ + static_cast<size_t>(t0) * rowK, static_cast<long long>(T - t0) * rowK);
#pragma unroll
      for (int blk = 0; blk < KBYTES / 1024; ++blk) {
        const int row = blk * KRPB + lane / KPR;
        const int off = row * rowK + h * DK * 2 + 16 * ((lane % KPR) ^ swz<KRB>(row));
        dma16(rk, B + K_OFF + 1024 * blk, off);
        dma16(rq, B + Q_OFF + 1024 * blk, off);
      }
    };
    auto copy_v = [&](int c) __attribute__((always_inline)) {
      const int t0 = c * CHUNK;
      const rsrc_t rv = make_rsrc_wu(vb_ + static_cast<size_t>(t0) * rowV, static_cast<long long>(T - t0) * rowV);
#pragma unroll
      for (int blk = 0; blk < VBYTES / 1024; ++blk) {
        const int row = blk * VRPB + lane / VPR;
        dma16(rv, ldsV + 1024 * blk, row * rowV + (h * DV + col0) * 2 + 16 * ((lane % VPR) ^ swz<VRB>(row)));
      }
    };
    if constexpr (LL) {
      // chunk c's weights lambda^(7+s) and lambda^(7+s') (see out_chunk) of its 64 tokens into
      // weight buffer `par`, one dword per lane (zero past T)
      auto copy_lam = [&](int c, int par) __attribute__((always_inline)) {
        const int t0 = c * CHUNK, HL = H * a.lam_L;
        const int s = __builtin_ctz(static_cast<unsigned>(a.seg_chunks));
        const unsigned above = static_cast<unsigned>(c) >> (s + 1);
        const int lev2 = above ? a.lam_level + 1 + __builtin_ctz(above) : a.lam_level;
        const rsrc_t rl = make_rsrc_wu(a.lam + ((static_cast<size_t>(b) * T + t0) * H + h) * a.lam_L,
                                       (static_cast<long long>(T - t0 - 1) * HL + a.lam_L) * 4);
        dma4(rl, &ldsL[par][0][0], (lane * HL + a.lam_level) * 4);
        dma4(rl, &ldsL[par][1][0], (lane * HL + lev2) * 4);
      };
      int i = i0, c = seg_start(i0);  // the next chunk to copy
      if (nchunks > 0) {
        copy_kqr(c, lds0);
        copy_lam(c, 0);
        copy_v(c);
      }
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      for (int j = 0; j < nchunks; ++j) {
        if (++c >= seg_end(i)) c = seg_start(++i);
        if (j + 1 < nchunks) {
          copy_kqr(c, ((j + 1) & 1) ? lds1 : lds0);
          copy_lam(c, (j + 1) & 1);
        }
        asm volatile("s_barrier" ::: "memory");  // past it, this chunk's V rows have been read
        if (j + 1 < nchunks) copy_v(c);
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      }
    } else {
      if (c_begin < c_end) {
        copy_kqr(c_begin, lds0);
        copy_v(c_begin);
      }
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      for (int c = c_begin; c < c_end; ++c) {
        if (c + 1 < c_end) copy_kqr(c + 1, ((c + 1 - c_begin) & 1) ? lds1 : lds0);
        asm volatile("s_barrier" ::: "memory");  // past it, this chunk's V rows have been read
        if (c + 1 < c_end) copy_v(c + 1);
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      }
    }
    return;
  }

  int oK[DK / 32], oT[DK / 32], oRt[2], oRb[2][2];
#pragma unroll
  for (int kb = 0; kb < DK / 32; ++kb) {
    oK[kb] = swz_off<KRB>(tok(0, ln), 64 * kb + 16 * gq);
    oT[kb] = swz_off<KRB>(8 * gq + (ln >> 2), 2 * (32 * kb + 8 * (ln & 3)));
  }
#pragma unroll
  for (int hl = 0; hl < 2; ++hl) {
    oRt[hl] = CREC_TOP_OFF + swz_off<128>(tok(0, ln), 64 * hl + 16 * gq);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) oRb[kb][hl] = CREC_BOT_OFF + swz_off<256>(tok(0, ln), 128 * hl + 64 * kb + 16 * gq);
  }
  const int oV = swz_off<VRB>(8 * gq + (ln >> 2), 2 * (16 * sl + 4 * (ln & 3)));
  auto mrow = [](int m) { return 32 * (m >> 1) + 4 * (m & 1); };
  auto fragK = [&](const uint8_t* X, int m, int kb) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(X + oK[kb] + mrow(m) * KRB));
  };
  auto fragKT = [&](const uint8_t* X, int m, int kb) __attribute__((always_inline)) {
    const uint8_t* p = X + oT[m >> 1] + 32 * kb * KRB + 8 * (m & 1);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * KRB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto fragR = [&](const uint8_t* X, int m, int kb) __attribute__((always_inline)) {
    const uint8_t* p = m < 2 ? X + oRt[0] + 4 * (m & 1) * 128 : X + oRb[kb][0] + 4 * (m & 1) * 256;
    const int lo = m < 2 ? oRt[1] - oRt[0] : oRb[kb][1] - oRb[kb][0];
    S8 r;
    r.h = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
    r.l = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p + lo));
    return r;
  };
  auto trV = [&](const uint8_t* X, int m) __attribute__((always_inline)) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(X + oV + mrow(m) * VRB));
    return __builtin_bit_cast(u32x2, v);
  };

  if (wu < 4) {  // recurrence wave
    f32x4 S[DK / 16];
    // the start state of segment i (zero without init)
    // (row tok(mt, 4 gq + e) = 8 gq + 32 (mt >> 1) + 4 (mt & 1) + e: a lane base plus a uniform offset)
    auto load_init = [&](int i) __attribute__((always_inline)) {
      if (a.init) {
        const float* ip = a.init + (static_cast<size_t>(bh) * a.init_segs + i) * DK * DV + 8 * gq * DV + col;
#pragma unroll
        for (int mt = 0; mt < DK / 16; ++mt) {
#pragma unroll
          for (int e = 0; e < 4; ++e) S[mt][e] = ip[(32 * (mt >> 1) + 4 * (mt & 1) + e) * DV];
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < DK / 16; ++mt) S[mt] = zero4();
      }
    };
    load_init(seg);
    // S split hi/lo: kept in registers for this wave's next chunk and handed to the output wave
    S8 Sb[DK / 32];
    auto split_and_publish = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        Sb[kb] = split8(frag_from_acc(S[2 * kb], S[2 * kb + 1]));
        ldsSb[sl][kb][0][lane] = __builtin_bit_cast(u32x4, Sb[kb].h);
        ldsSb[sl][kb][1][lane] = __builtin_bit_cast(u32x4, Sb[kb].l);
      }
    };
    // one chunk from buffer B; `zero`: S is zero (a lead chunk), `last`: the end of segment i,
    // `lead_next`: the next chunk is a lead chunk (S restarts from zero, and its split is not read)
    auto rec_chunk = [&](const uint8_t* B, bool zero, bool last, int i, bool lead_next) __attribute__((always_inline)) {
      const uint8_t* sK = B + K_OFF;
      const uint8_t* sV = ldsV;
      const uint8_t* sR = B + R_OFF;
      const float* sEG = reinterpret_cast<const float*>(sR + CREC_EG_OFF);
      const float* sEGC = reinterpret_cast<const float*>(sR + CREC_EGC_OFF);
      f32x4 Rr[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc = zero4();
        if (!zero) {
#pragma unroll
          for (int kb = 0; kb < DK / 32; ++kb) acc = TR::mma_xd(acc, fragK(sK, mt, kb), Sb[kb]);
        }
        const f32x4 eg = *reinterpret_cast<const f32x4*>(sEG + tok(mt, 4 * gq));
        const u32x2 x = trV(sV, mt);
        f32x4 vv;
        vv[0] = __uint_as_float(x[0] << 16);
        vv[1] = __uint_as_float(x[0] & 0xFFFF0000u);
        vv[2] = __uint_as_float(x[1] << 16);
        vv[3] = __uint_as_float(x[1] & 0xFFFF0000u);
        Rr[mt] = vv - eg * acc;
      }
      S8 Rb[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) Rb[kb] = split8(frag_from_acc(Rr[2 * kb], Rr[2 * kb + 1]));
      f32x4 U[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        U[mt] = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if (kb == 0 || mt >= 2) U[mt] = TR::mma_dd(U[mt], fragR(sR, mt, kb), Rb[kb]);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const S8 ub = split8(frag_from_acc(U[2 * kb], U[2 * kb + 1]));
        ldsUb[sl][kb][0][lane] = __builtin_bit_cast(u32x4, ub.h);
        ldsUb[sl][kb][1][lane] = __builtin_bit_cast(u32x4, ub.l);
      }
      // U published; the output wave has read this chunk's S split (its reads precede its
      // arrival here), so the next one may be written after this barrier
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      f32x4 Ue[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) Ue[mt] = U[mt] * *reinterpret_cast<const f32x4*>(sEGC + tok(mt, 4 * gq));
      S8 Ud[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) Ud[kb] = split8(frag_from_acc(Ue[2 * kb], Ue[2 * kb + 1]));
      const float gC = sEG[CHUNK - 1];
#pragma unroll
      for (int mt = 0; mt < DK / 16; ++mt) {
        S[mt] *= gC;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) S[mt] = TR::mma_xd(S[mt], fragKT(sK, mt, kb), Ud[kb]);
      }
      if constexpr (LL) {
        if (last) {  // the segment's end state for the next scale (even segments), then the next start
          if (a.fin && !(i & 1) && (i >> 1) < a.fin_segs) {
            float* F = a.fin + (static_cast<size_t>(bh) * a.fin_segs + (i >> 1)) * DK * DV + 8 * gq * DV + col;
#pragma unroll
            for (int mt = 0; mt < DK / 16; ++mt) {
#pragma unroll
              for (int e = 0; e < 4; ++e) F[(32 * (mt >> 1) + 4 * (mt & 1) + e) * DV] = S[mt][e];
            }
          }
          if (lead_next) {
#pragma unroll
            for (int mt = 0; mt < DK / 16; ++mt) S[mt] = zero4();
          } else if (i + 1 < i1) {
            load_init(i + 1);
          }
        }
      }
      if (!lead_next) split_and_publish();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    split_and_publish();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (PAIRS) {  // scale 0: every segment is a lead chunk (buffer 0) and an output chunk (buffer 1)
      for (int i = i0; i < i1; ++i) {
        rec_chunk(lds0, true, false, i, false);
        rec_chunk(lds1, false, true, i, true);
      }
    } else if constexpr (LL) {
      {
        // Segments of 2^s >= 2 chunks: a segment ends on buffer 1, except the last one of the
        // sequence when it is cut short by its end, whose end state no scale reads
        int i = i0, c = seg_start(i0);
        for (int j = 0; j < nchunks; j += 2) {
          rec_chunk(lds0, false, false, i, false);
          if (++c >= seg_end(i)) c = seg_start(++i);
          if (j + 1 < nchunks) {
            rec_chunk(lds1, false, c + 1 >= seg_end(i), i, false);
            if (++c >= seg_end(i)) c = seg_start(++i);
          }
        }
      }
    } else {
      for (int c = c_begin; c < c_end; c += 2) {
        rec_chunk(lds0, false, false, seg, false);
        if (c + 1 < c_end) rec_chunk(lds1, false, false, seg, false);
      }
      if (a.fin && (!a.fin_last_only || seg == a.nseg - 1)) {
        float* F = a.fin + (static_cast<size_t>(bh) * a.fin_segs + (a.fin_last_only ? 0 : seg)) * DK * a.fin_ld;
#pragma unroll
        for (int mt = 0; mt < DK / 16; ++mt) {
#pragma unroll
          for (int e = 0; e < 4; ++e) F[(tok(mt, 4 * gq) + e) * a.fin_ld + col] = S[mt][e];
        }
      }
    }
  } else {  // output wave
    auto store_out = [&](int c, int mt, const f32x4& o) __attribute__((always_inline)) {
      const int t0 = c * CHUNK;
      const rsrc_t ro = make_rsrc_wu(ob_ + static_cast<size_t>(t0) * rowO, static_cast<long long>(T - t0) * rowO);
      const int obase = (h * DV + col0 + 16 * sl + 4 * gq) * 4;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), ro, obase + tok(mt, ln) * rowO, 0, 0);
    };
    auto out_chunk = [&](int c, const uint8_t* B, int par) __attribute__((always_inline)) {
      // LL: the outputs already there, loaded first so that the adds never wait on a memory round
      // trip (a load issued after the stores would also wait for them: loads and stores retire in
      // order on one counter); the weights come from LDS (buffer `par`), combined as
      // lambda^(7+s) - lambda^(7+s'), s' the next set bit of c above s (none: lambda^(7+s))
      u32x4 acc_old[LL ? 4 : 1];
      float keep_b = 0.f;
      if constexpr (LL) {
        const int t0 = c * CHUNK;
        const rsrc_t ra = make_rsrc_wu(ob_ + static_cast<size_t>(t0) * rowO, static_cast<long long>(T - t0) * rowO);
        const int obase = (h * DV + col0 + 16 * sl + 4 * gq) * 4;
        const int s = __builtin_ctz(static_cast<unsigned>(a.seg_chunks));
        keep_b = (static_cast<unsigned>(c) >> (s + 1)) ? 1.f : 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc_old[mt] = bload16(ra, obase + tok(mt, ln) * rowO);
      }
      const uint8_t* sK = B + K_OFF;
      const uint8_t* sQ = B + Q_OFF;
      const uint8_t* sR = B + R_OFF;
      const float* sG = reinterpret_cast<const float*>(sR + CREC_G_OFF);
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int mi = (sl >> 1) + (j == 2 ? 2 : 0), mj = (sl & 1) + (j >= 1 ? 2 : 0);
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) acc = mfma_bf16(fragK(sK, mi, kb), fragK(sQ, mj, kb), acc);
        const int r = tok(mj, ln), i0 = tok(mi, 4 * gq);
        const float gr = sG[r];
        const f32x4 gi = *reinterpret_cast<const f32x4*>(sG + i0);
        f32x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = __expf(gr - gi[e]) * acc[e];
          pv[e] = (j == 1 || i0 + e <= r) ? x : 0.f;
        }
        const u32x2 hw = __builtin_bit_cast(u32x2, __builtin_convertvector(pv, bf16x4));
        f32x4 hf;
        hf[0] = __uint_as_float(hw[0] << 16);
        hf[1] = __uint_as_float(hw[0] & 0xFFFF0000u);
        hf[2] = __uint_as_float(hw[1] << 16);
        hf[3] = __uint_as_float(hw[1] & 0xFFFF0000u);
        const f32x4 lv = pv - hf;
        const u32x2 lw = __builtin_bit_cast(u32x2, __builtin_convertvector(lv, bf16x4));
        int oh, ol;
        if (j == 0) {
          oh = CREC_TOP_OFF + swz_off<128>(r, 2 * i0);
          ol = CREC_TOP_OFF + swz_off<128>(r, 64 + 2 * i0);
        } else {
          oh = CREC_BOT_OFF + swz_off<256>(r - 32, 2 * i0);
          ol = CREC_BOT_OFF + swz_off<256>(r - 32, 128 + 2 * i0);
        }
        *reinterpret_cast<u32x2*>(ldsP + oh) = hw;
        *reinterpret_cast<u32x2*>(ldsP + ol) = lw;
      }
      f32x4 Oacc[4];
      {
        S8 Sb[DK / 32];
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          Sb[kb].h = __builtin_bit_cast(bf16x8, ldsSb[sl][kb][0][lane]);
          Sb[kb].l = __builtin_bit_cast(bf16x8, ldsSb[sl][kb][1][lane]);
        }
        // the split of S is read before the mid-chunk barrier (past it the recurrence wave may
        // overwrite it) and used after it: Q S off the first half, where the P tiles already
        // keep this wave longer than the recurrence wave takes to publish U
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const float* sEG = reinterpret_cast<const float*>(sR + CREC_EG_OFF);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kb = 0; kb < DK / 32; ++kb) {
            const bf16x8 qf = fragK(sQ, mt, kb);
            acc = mfma_bf16(Sb[kb].h, qf, acc);
            acc = mfma_bf16(Sb[kb].l, qf, acc);
          }
          Oacc[mt] = acc * sEG[tok(mt, ln)];
        }
      }
      // LL: nothing below may be hoisted above the barrier; the scheduler would otherwise move
      // the weights' arithmetic up and with it a wait for the loads of this chunk's weights
      if constexpr (LL) __builtin_amdgcn_sched_barrier(0);
      S8 Ub[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Ub[kb].h = __builtin_bit_cast(bf16x8, ldsUb[sl][kb][0][lane]);
        Ub[kb].l = __builtin_bit_cast(bf16x8, ldsUb[sl][kb][1][lane]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc = Oacc[mt];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          if (kb == 0 || mt >= 2) acc = TR::mma_dd(acc, Ub[kb], fragR(ldsP, mt, kb));
        if constexpr (LL) {  // rows past T are not stored
          const int r = tok(mt, ln);
          const float wt = ldsL[par][0][r] - keep_b * ldsL[par][1][r];
          acc = __builtin_bit_cast(f32x4, acc_old[mt]) + wt * acc;
        }
        store_out(c, mt, acc);
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    asm volatile("s_barrier" ::: "memory");
    if constexpr (PAIRS) {  // a lead chunk has no outputs: its two barriers only
      for (int i = i0; i < i1; ++i) {
        asm volatile("s_barrier\n\ts_barrier" ::: "memory");
        out_chunk(seg_begin(i), lds1, 1);
      }
    } else if constexpr (LL) {
      {
        int i = i0, c = seg_start(i0);
        for (int j = 0; j < nchunks; j += 2) {
          out_chunk(c, lds0, 0);
          if (++c >= seg_end(i)) c = seg_start(++i);
          if (j + 1 < nchunks) {
            out_chunk(c, lds1, 1);
            if (++c >= seg_end(i)) c = seg_start(++i);
          }
        }
      }
    } else {
      for (int c = c_begin; c < c_end; c += 2) {
        out_chunk(c, lds0, 0);
        if (c + 1 < c_end) out_chunk(c + 1, lds1, 1);
      }
    }
  }
}

bool state_dma_supported(int mode, int dk) { return mode == MODE_BF16 && (dk == 64 || dk == 128); }

hipError_t launch_state_dma(bool with_out, bool aug, int dk, int nwg, const void* q, const void* k, const void* v,
                            const uint8_t* rec, int T, int H, int DV, int nc, int seg_chunks, const float* init,
                            int init_segs, float* out, float* fin, int fin_ld, int fin_segs, int fin_last_only,
                            int ncg, int nseg, hipStream_t stream, int seg_mul, int seg_add, int skip_ident0) {
  const StateDmaArgs a{q, k, v, rec, T, H, DV, nc, seg_chunks, init, init_segs, out, fin, fin_ld, fin_segs,
                       fin_last_only, ncg, nseg, seg_mul, seg_add, nullptr, 0, 0, 1, skip_ident0};
  if (with_out && aug) return hipErrorInvalidValue;  // a walk with outputs carries the plain state
  if (dk == 64) {
    if (with_out) return launch_kernel(state_walk_kernel<64, WALK_PLAIN>, dim3(nwg), dim3(WALK_THREADS), stream, a);
    if (aug) return launch_kernel(state_map_kernel<64, true>, dim3(nwg), dim3(MAP_THREADS), stream, a);
    return launch_kernel(state_map_kernel<64, false>, dim3(nwg), dim3(MAP_THREADS), stream, a);
  }
  if (dk == 128) {
    if (with_out) return launch_kernel(state_walk_kernel<128, WALK_PLAIN>, dim3(nwg), dim3(WALK_THREADS), stream, a);
    if (aug) return launch_kernel(state_map_kernel<128, true>, dim3(nwg), dim3(MAP_THREADS), stream, a);
    return launch_kernel(state_map_kernel<128, false>, dim3(nwg), dim3(MAP_THREADS), stream, a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_loglinear_scale_dma(int dk, const void* q, const void* k, const void* v, const uint8_t* rec, int T,
                                      int H, int DV, int nc, int BH, int s, int nright, const float* init, float* fin,
                                      int fin_segs, const float* lam, int L, float* out, hipStream_t stream) {
  if (nright <= 0) return hipSuccess;
  if (s < 0 || s > 24 || 7 + s >= L || DV % 64 != 0) return hipErrorInvalidValue;
  const int ncg = DV / 64;
  // about one workgroup per compute unit: a (b, h, column group) walks all of its segments when
  // there are enough of them, else they are shared out in consecutive runs
  const int units = ncg * BH;
  const int groups = std::max(1, std::min(nright, (256 + units - 1) / units));
  const int wg_segs = (nright + groups - 1) / groups;
  const int ngrp = (nright + wg_segs - 1) / wg_segs;
  const StateDmaArgs a{q, k, v, rec, T, H, DV, nc, 1 << s, init, nright, out, fin, DV, fin_segs, 0, ncg, nright,
                       2, 1, lam, L, 7 + s, wg_segs, 0};
  const dim3 grid(units * ngrp), block(WALK_THREADS);
  if (dk == 64)
    return s == 0 ? launch_kernel(state_walk_kernel<64, WALK_LL_PAIRS>, grid, block, stream, a)
                  : launch_kernel(state_walk_kernel<64, WALK_LL>, grid, block, stream, a);
  if (dk == 128)
    return s == 0 ? launch_kernel(state_walk_kernel<128, WALK_LL_PAIRS>, grid, block, stream, a)
                  : launch_kernel(state_walk_kernel<128, WALK_LL>, grid, block, stream, a);
  return hipErrorInvalidValue;
}

}  // namespace kla
