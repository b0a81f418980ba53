// Device-side building blocks shared by the KLA kernels (gfx950 / CDNA4).
//
// Matrix products run on the 16x16 MFMA tiles of one 64-lane wavefront:
//   bf16 mode: v_mfma_f32_16x16x32_bf16 (fp32 accumulate)
//   fp32 mode: v_mfma_f32_16x16x4_f32
// Lane l of a wave is split into a column index ln = l % 16 and a lane group
// gq = l / 16. A 16x16 accumulator tile holds D[4*gq + i][ln], i = 0..3.
//
// Contraction order. A 32-wide contraction block is consumed by lane group gq
// as 8 values whose contraction indices are kslot(gq, j):
//     j = 0..3  ->  4*gq + j
//     j = 4..7  -> 16 + 4*gq + (j - 4)
// These are exactly the rows that two stacked 16x16 accumulator tiles hold in a
// lane, so the result of one product (rows = contraction index of the next
// product) feeds the next product's B operand straight from registers, with no
// LDS round trip. Operands read from LDS use the same order. The sum is the
// same for any order in which both operands agree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
// Raw 16- and 8-byte vectors. Native vector types (not the uint4 struct) keep register
// copies out of memory: a conditional struct copy lowers to a select of addresses.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int MODE_BF16 = 0;  // q, k, v in bf16; derived operands split into hi + lo bf16
constexpr int MODE_F32 = 1;   // q, k, v in fp32; fp32 MFMA throughout

constexpr int CHUNK = 64;     // tokens per chunk

// Per-chunk record written by the prep kernel and read by the state kernels.
//   [0, 16384)      T' = (I + A)^-1 diag(beta): 64 rows of 256 bytes
//   [16384, 32768)  P  = (Q K^T) masked by the inclusive decay mask: 64 rows of 256 bytes
//   [32768, 33024)  exp(g_r), 64 floats (g = chunk-local inclusive cumsum of log alpha)
//   [33024, 33280)  exp(g_C - g_r), 64 floats
//   [33280, 33536)  g_r, 64 floats
// A 256-byte row holds 64 fp32 values (fp32 mode) or 64 hi bf16 then 64 lo bf16 (bf16 mode).
constexpr int REC_T_OFF = 0;
constexpr int REC_P_OFF = 16384;
constexpr int REC_EG_OFF = 32768;
constexpr int REC_EGC_OFF = 33024;
constexpr int REC_G_OFF = 33280;
constexpr int REC_BYTES = 33536;

// Compact per-chunk record, for the state kernel that forms P itself (bf16, dk <= 128):
//   [0, 4096)       T' rows 0..31, 128 bytes each: hi of columns 0..31, then lo
//   [4096, 12288)   T' rows 32..63, 256 bytes each: hi of columns 0..63, then lo
//   [12288, 13056)  exp(g_r), exp(g_C - g_r), g_r as above
// T' is lower triangular, so its upper-right 32 x 32 quadrant (zero) is left out. Rows
// 0..31 are swizzled as 128-byte rows (swz<128>), rows 32..63 as 256-byte rows numbered
// from 0 (swz<256> of row - 32).
constexpr int CREC_TOP_OFF = 0;
constexpr int CREC_BOT_OFF = 4096;
constexpr int CREC_EG_OFF = 12288;
constexpr int CREC_EGC_OFF = 12544;
constexpr int CREC_G_OFF = 12800;
constexpr int CREC_BYTES = 13056;

// LDS row pitch of a derived 64x64 matrix: 256 bytes of data + 16 bytes of padding.
constexpr int DROW_BYTES = 272;

// ---------------------------------------------------------------------------
// Buffer resources. A raw buffer access is bounds-checked against num_records on
// its per-lane offset (the scalar offset is not checked): out-of-range loads return
// zero and out-of-range stores are dropped. Resources are built per chunk with the
// chunk's first row as base and num_records ending at token T, so the ragged last
// chunk needs no branches.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int BUF_FLAGS = 0x00020000;  // raw (untyped) dword access

// num_records is capped below BUF_OOB, an offset that is therefore always out of range;
// the host keeps every in-chunk offset below it.
constexpr int BUF_OOB = 0x40000000;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, long long bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= BUF_OOB ? BUF_OOB - 1 : static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, BUF_FLAGS);
}
// The same for a base and size that are uniform across the wave but that the compiler
// cannot prove uniform (they depend on the wave index): the values are passed through
// readfirstlane, so the descriptor lives in scalar registers. Without this, every buffer
// instruction using the descriptor is wrapped in a loop over the distinct values of the
// wave's lanes (readfirstlane, compare, exec mask), which costs about a hundred cycles per
// instruction.
__device__ __forceinline__ rsrc_t make_rsrc_wu(const void* base, long long bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  const int n = bytes <= 0 ? 0 : (bytes >= BUF_OOB ? BUF_OOB - 1 : static_cast<int>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), 0,
                                           __builtin_amdgcn_readfirstlane(n), BUF_FLAGS);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, int voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}
// Workgroup barrier that waits for the wave's LDS operations only: global loads and stores
// issued before it stay in flight (__syncthreads also waits for every one of them).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t bload4(rsrc_t r, int voff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}
__device__ __forceinline__ void bstore_f32(float x, rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS row swizzle. Rows of RB bytes are split into 16-byte pieces; logical piece p of
// row r is stored at piece p ^ swz<RB>(r), swz linear over GF(2) in the row bits:
//   256-byte rows: piece bits (0, r0, r1, r3);   128-byte rows: piece bits (0, r1, r3).
// The bank model behind the choice was measured on gfx950 with bank-conflict counters:
// 64 banks of 4 bytes, reads of one address broadcast; a 16-byte read is served in four
// phases, lane (g, l) (g = lane / 16, l = lane % 16) in phase g ^ parity((l >> 2) & 3); an
// 8-byte read (also ds_read_b64_tr_b16) in two phases of 32 consecutive lanes. The state
// kernels read operand fragments from rows in the permuted order 32a + 8b + 4c + d (a
// 16-lane group takes rows with b, d varying) and transposed 8-byte blocks from four
// consecutive rows. Under these swizzles the 16-byte fragment reads are conflict-free; a
// transposed read of a K^T operand, whose 32 lanes all read the same 8-byte half of their
// pieces, is two-way, the least possible with 16-byte pieces. Chunk records are written in
// this layout so that they can be copied into LDS unchanged.
template <int RB>
__device__ __forceinline__ int swz(int row) {
  if constexpr (RB >= 256) {
    return ((row & 1) << 1) | (row & 2) << 1 | (((row >> 3) & 1) << 3);
  } else {
    return (row & 2) | (((row >> 3) & 1) << 2);
  }
}
template <int RB>
__device__ __forceinline__ int swz_off(int row, int byte) {
  return row * RB + (((byte >> 4) ^ swz<RB>(row)) << 4) + (byte & 15);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ int kslot(int gq, int j) {
  return j < 4 ? 4 * gq + j : 12 + 4 * gq + j;
}

// 32-bit word i (compile-time after unrolling) of a 16-byte vector, without taking its address
// (an address would force the vector out of registers).
__device__ __forceinline__ uint32_t u4word(const u32x4& v, int i) { return v[i]; }

// Element j of a 16-byte vector holding bf16 (ELEM_BYTES = 2) or fp32 (4) values, as raw bits.
template <int ELEM_BYTES>
__device__ __forceinline__ uint32_t u4elem(const u32x4& v, int j) {
  if constexpr (ELEM_BYTES == 2) return (u4word(v, j >> 1) >> (16 * (j & 1))) & 0xFFFFu;
  else return u4word(v, j);
}

struct F8 {
  float v[8];
};

struct S8 {  // hi + lo bf16 split of 8 fp32 values
  bf16x8 h, l;
};

__device__ __forceinline__ F8 frag_from_acc(const f32x4& a, const f32x4& b) {
  F8 r;
  r.v[0] = a[0]; r.v[1] = a[1]; r.v[2] = a[2]; r.v[3] = a[3];
  r.v[4] = b[0]; r.v[5] = b[1]; r.v[6] = b[2]; r.v[7] = b[3];
  return r;
}

__device__ __forceinline__ S8 split8(const F8& x) {
  // hi = round-to-nearest-even bf16 of x; lo = bf16 of the exact residual x - hi.
  // Vector conversions make the compiler pair values into v_cvt_pk_bf16_f32.
  f32x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = x.v[j];
  S8 s;
  s.h = __builtin_convertvector(v, bf16x8);
  const u32x4 hw = __builtin_bit_cast(u32x4, s.h);
  f32x8 hf;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    hf[2 * m] = __uint_as_float(hw[m] << 16);
    hf[2 * m + 1] = __uint_as_float(hw[m] & 0xFFFF0000u);
  }
  s.l = __builtin_convertvector(v - hf, bf16x8);
  return s;
}

// Fused PSD lift (KATA page, section 2.2: psi(u) = vec(u u^T), feature a*16 + b = u_a u_b).
// The kernels that read queries and keys in lifted form take the 16-wide u rows of bf16 and
// form the features as they load them. LIFT_P is the width of u, LIFT_DK the feature width.
constexpr int LIFT_P = 16;
constexpr int LIFT_DK = LIFT_P * LIFT_P;

// Eight lifted features u_a * u_{b0 + i}, i = 0..7, each rounded to the nearest bf16 (ties to
// even), as 16 raw bytes. `ua_bits` holds u_a in the high half of a word; `ub` holds
// u_{b0} .. u_{b0+7} as bf16. The product of two bf16 values has at most 16 significant
// bits, so the fp32 multiply is exact and the conversion is the only rounding.
__device__ __forceinline__ u32x4 lift8(uint32_t ua_bits, const u32x4& ub) {
  const float ua = __uint_as_float(ua_bits & 0xFFFF0000u);
  f32x8 f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    f[2 * m] = ua * __uint_as_float(ub[m] << 16);
    f[2 * m + 1] = ua * __uint_as_float(ub[m] & 0xFFFF0000u);
  }
  return __builtin_bit_cast(u32x4, __builtin_convertvector(f, bf16x8));
}

// u_a of a lifted row as the high half of a word: `w` is the 32-bit word holding u_{2m} (low
// half) and u_{2m+1} (high half), `odd` picks u_{2m+1}.
__device__ __forceinline__ uint32_t lift_pick(uint32_t w, bool odd) { return odd ? w : w << 16; }

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// ---------------------------------------------------------------------------
// Mode traits: storage type of q/k/v and the three kinds of product
//   xx: exact input x exact input
//   xd: exact input x derived (fp32 value carried as hi + lo in bf16 mode)
//   dd: derived x derived
// ---------------------------------------------------------------------------
template <int MODE>
struct Tr;

template <>
struct Tr<MODE_BF16> {
  using in_t = uint16_t;  // bf16 bit pattern
  using XF = bf16x8;      // exact operand fragment
  using DF = S8;          // derived operand fragment

  // Exact operand from a row-major LDS matrix with pitch `ld` elements:
  // row = row0 + ln, contraction columns k0 + kslot(gq, 0..7).
  static __device__ __forceinline__ XF ldx(const in_t* base, int ld, int row0, int k0, int lane) {
    const in_t* p = base + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    const u32x2 a = *reinterpret_cast<const u32x2*>(p);
    const u32x2 b = *reinterpret_cast<const u32x2*>(p + 16);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3));
  }
  // Derived operand from a 64x64 matrix stored with DROW_BYTES rows (hi at byte 0, lo at byte 128).
  static __device__ __forceinline__ DF ldd(const uint8_t* base, int row0, int k0, int lane) {
    const uint8_t* p = base + (row0 + (lane & 15)) * DROW_BYTES + 2 * (k0 + 4 * (lane >> 4));
    const u32x2 a = *reinterpret_cast<const u32x2*>(p);
    const u32x2 b = *reinterpret_cast<const u32x2*>(p + 32);
    const u32x2 c = *reinterpret_cast<const u32x2*>(p + 128);
    const u32x2 d = *reinterpret_cast<const u32x2*>(p + 160);
    DF r;
    r.h = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3));
    r.l = __builtin_bit_cast(bf16x8, __builtin_shufflevector(c, d, 0, 1, 2, 3));
    return r;
  }
  static __device__ __forceinline__ DF mk(const F8& x) { return split8(x); }
  static __device__ __forceinline__ f32x4 mma_xx(f32x4 c, const XF& a, const XF& b) {
    return mfma_bf16(a, b, c);
  }
  static __device__ __forceinline__ f32x4 mma_xd(f32x4 c, const XF& a, const DF& b) {
    c = mfma_bf16(a, b.h, c);
    return mfma_bf16(a, b.l, c);
  }
  static __device__ __forceinline__ f32x4 mma_dd(f32x4 c, const DF& a, const DF& b) {
    c = mfma_bf16(a.h, b.h, c);
    c = mfma_bf16(a.h, b.l, c);
    return mfma_bf16(a.l, b.h, c);
  }
  static __device__ __forceinline__ float to_f32(in_t x) { return bf16_bits_to_f32(x); }
};

template <>
struct Tr<MODE_F32> {
  using in_t = float;
  using XF = F8;
  using DF = F8;

  static __device__ __forceinline__ XF ldx(const in_t* base, int ld, int row0, int k0, int lane) {
    const in_t* p = base + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 16);
    F8 r;
    r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
    r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
    return r;
  }
  static __device__ __forceinline__ DF ldd(const uint8_t* base, int row0, int k0, int lane) {
    const float* p = reinterpret_cast<const float*>(base + (row0 + (lane & 15)) * DROW_BYTES) + k0 +
                     4 * (lane >> 4);
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 16);
    F8 r;
    r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
    r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
    return r;
  }
  static __device__ __forceinline__ DF mk(const F8& x) { return x; }
  static __device__ __forceinline__ f32x4 mma8(f32x4 c, const F8& a, const F8& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ f32x4 mma_xx(f32x4 c, const XF& a, const XF& b) { return mma8(c, a, b); }
  static __device__ __forceinline__ f32x4 mma_xd(f32x4 c, const XF& a, const DF& b) { return mma8(c, a, b); }
  static __device__ __forceinline__ f32x4 mma_dd(f32x4 c, const DF& a, const DF& b) { return mma8(c, a, b); }
  static __device__ __forceinline__ float to_f32(in_t x) { return x; }
};

}  // namespace kla
