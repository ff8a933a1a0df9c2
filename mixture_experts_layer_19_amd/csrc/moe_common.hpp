// moe_common.hpp -- device helpers shared by the MoE layer kernels (gfx950).
//
// Fragment layout used by every matrix kernel.  A "chunk" is 256 bytes of
// one row along the reduction axis K (128 bf16, 256 fp8 or 64 fp32
// elements), split into two 128-byte halves.  A block of 16 rows x 1 chunk
// is held by one wave: lane l owns row l % 16 and, with lane group
// g = l / 16, four 16-byte pieces p = 0..3 at chunk byte offset
//     off(g, p) = 128 * (p / 2) + 64 * (p % 2) + 16 * g,
// i.e. in half h the row's bytes [0, 64) are piece 2h of lane groups 0-3 and
// bytes [64, 128) are piece 2h+1.  A half-chunk stage therefore reads one
// contiguous 128-byte line of every row.  Packed weight blocks and LDS tiles
// store a block as [piece][lane][16 bytes] (4 KiB, or 2 KiB per half), so
// one wave-wide 16-byte access touches a contiguous 1 KiB.
//
// Matrix-core steps: bf16 v_mfma_f32_16x16x32_bf16 contracts one piece (8
// elements per lane), 2 per half-chunk; fp32 v_mfma_f32_16x16x4f32 one
// element, 8 per half-chunk; MX-fp8 v_mfma_scale_f32_16x16x128_f8f6f4 both
// pieces of a half (32 bytes per lane), 1 per half-chunk.  The weight and
// the token operand use the same (lane group, piece, element) -> k
// assignment, so every step contracts matching k on both sides.
//
// MX scales.  On gfx950 the scaled 16x16x128 instruction treats byte i of
// lane group g's 32 operand bytes as K index 64 * (i / 16) + 16 * g + i % 16,
// and takes the scale of K block b (K in [32b, 32b + 32)) from lane group b
// (measured on the device).  With the piece offsets above, K block b of half
// h is exactly the 32-element MX block 4h + b of the chunk (row bytes
// [32b, 32b + 32) of the half), so lane group g supplies the E8M0 scale of
// MX block 4h + g while its data bytes belong to blocks g/2 and 2 + g/2.
//
// MXFP4 weights (W4A8).  An E2M1 chunk is 128 bytes per row, so a block of
// 16 rows x 1 chunk is 2 KiB, stored [half][lane][16 bytes].  For E2M1 A
// operands the scaled 16x16x128 instruction reads four registers per lane:
// nibble i of lane group g (low nibble first) is K index 32 * g + i, and the
// scale of K block b again comes from lane group b (measured on the device).
// So lane group g of half h holds the contiguous MX block 4h + g of its row
// (16 bytes), multiplies the fp8 token bytes the token layout above assigns
// to the same K, and supplies that block's scale: the scale layout is the
// MX-fp8 one.
//
// The weights are the MFMA A operand (16 output features) and the tokens
// the B operand (16 tokens), so the 16x16 accumulator of lane l holds
// token m = l % 16 and output features n = 4 * (l / 16) + r, r = 0..3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace moe {

constexpr int kChunkBytes = 256;      // bytes of one row per K chunk
constexpr int kBlockBytes = 4096;     // 16 rows x 1 chunk
constexpr int kLaneBytes = 64;        // one lane's share of a block

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

// Weight formats.  FMT_MX4 is MXFP4 (E2M1) weights multiplied with MX-fp8
// activations; FMT_FP8 is E4M3 with one static scale per tensor (applied in
// the epilogue); every other format uses the same type on both sides.
enum Fmt { FMT_F32 = 0, FMT_BF16 = 1, FMT_MX8 = 2, FMT_MX4 = 3, FMT_FP8 = 4 };

template <int F> struct FmtInfo;
template <> struct FmtInfo<FMT_F32> { static constexpr int elem_bytes = 4, chunk_elems = 64; };
template <> struct FmtInfo<FMT_BF16> { static constexpr int elem_bytes = 2, chunk_elems = 128; };
template <> struct FmtInfo<FMT_MX8> { static constexpr int elem_bytes = 1, chunk_elems = 256; };
template <> struct FmtInfo<FMT_MX4> { static constexpr int elem_bytes = 1, chunk_elems = 256; };
template <> struct FmtInfo<FMT_FP8> { static constexpr int elem_bytes = 1, chunk_elems = 256; };

// format of the token-side operand for weight format F
template <int F> constexpr int tok_fmt = (F == FMT_MX4) ? FMT_MX8 : F;
// block-scaled formats (E8M0 scales on both operands)
template <int F> constexpr bool is_mx = (F == FMT_MX8 || F == FMT_MX4);
// bytes of one packed weight block (16 rows x one K chunk)
template <int F> constexpr int wblock_bytes = (F == FMT_MX4) ? 2048 : kBlockBytes;

// ----------------------------------------------------------------------------- conversions

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// OCP MX E4M3 (FN) rounding of a finite fp32 value: round to nearest even,
// saturate to +-448, keep the sign (also for results that round to zero).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fabsf(v);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {                         // below 2^-6: multiples of 2^-9
    return sign | (uint32_t)rintf(a * 512.0f);  // 8 becomes the smallest normal
  }
  uint32_t bits = __float_as_uint(a);
  int e = (int)((bits >> 23) & 0xFFu) - 127;
  uint32_t man = bits & 0x7FFFFFu;
  uint32_t q = man >> 20, rem = man & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
  if (q == 8u) { q = 0u; ++e; }
  if (e > 8 || (e == 8 && q == 7u)) return sign | 0x7Eu;
  return sign | ((uint32_t)(e + 7) << 3) | q;
}

// OCP MX E2M1 rounding of a finite scaled value: magnitudes 0, 0.5, 1, 1.5,
// 2, 3, 4, 6; a value between two of them goes to the nearer, a midpoint to
// the code with mantissa bit 0 (the comparisons against the seven midpoints
// are strict where the lower code is even), and values above 5 to 6
// (saturation).  Sign in bit 3.
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
  const float a = fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return sign | c;
}

// Shared exponent of an MXFP4 block: X = floor(log2 amax) - 2 (2 is the
// exponent of E2M1's largest normal, 6), clamped below at -127.  Returned
// as the E8M0 byte X + 127.
__device__ __forceinline__ uint32_t mx4_scale_byte(float amax) {
  int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  int X = ef - 127 - 2;
  if (ef == 0 || X < -127) X = -127;
  return (uint32_t)(X + 127);
}

// Shared exponent X of an MX block from its largest magnitude (exact):
// X = floor(log2 amax) - 8, clamped below at -127 (zero and fp32-subnormal
// maxima give -127).  Returned as the E8M0 byte X + 127.
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);   // 0 for zero/subnormal
  int X = ef - 127 - 8;
  if (ef == 0 || X < -127) X = -127;
  return (uint32_t)(X + 127);
}

// 2^-X as an fp32 for an E8M0 byte s = X + 127 (X in [-127, 125]).
__device__ __forceinline__ float mx_inv_scale(uint32_t s) {
  return __uint_as_float((uint32_t)(254 - (int)s) << 23);
}

// ----------------------------------------------------------------------------- buffer access

// Raw buffer descriptor over [base, base + bytes) (stride 0, 32-bit data
// format word of the gfx9 family).  Loads through it take a per-lane 32-bit
// offset and a wave-uniform scalar offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// ----------------------------------------------------------------------------- wave helpers

// For the lambdas that make up a kernel's main loop: they must be inlined
// (a call would move the accumulators they capture to scratch memory), and
// a large stage can exceed the inliner's cost threshold.
#define MOE_INLINE __attribute__((always_inline))

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N - 1>{})
template <typename Fn, int... Q>
__device__ __forceinline__ void static_for_impl(Fn &&f, std::integer_sequence<int, Q...>) {
  (f(std::integral_constant<int, Q>{}), ...);
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}


__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

// ----------------------------------------------------------------------------- MFMA

__device__ __forceinline__ int chunk_off(int g, int p) { return 128 * (p >> 1) + 64 * (p & 1) + 16 * g; }

// LDS slot of (row r16, lane group g) inside a staged token piece p (0 or 1
// within a half-chunk): the 16 slots of
// a lane group are XOR-permuted so the stores of one wave (8 rows x 4 lane
// groups x 2 pieces, 16 bytes each) fall into distinct banks, while a wave's
// fragment read (lane group g reads slots 16 g .. 16 g + 15) stays
// conflict-free.
__device__ __forceinline__ int tslot(int r16, int g, int p) {
  return 16 * g + (r16 ^ ((2 * g + 8 * p) & 15));
}

// acc += W x T over one half-chunk.  w0, w1 / t0, t1: the lane's two
// 16-byte pieces of this half (pieces 2h and 2h + 1).  ws, ts: E8M0 scale
// bytes of the lane's MX block (MX only): the weight scale is byte WSEL of
// ws and the token scale byte TSEL of ts (the instruction's operand selects
// pick them, so a packed pair of scales needs no shift).
template <int F, int WSEL = 0, int TSEL = 0>
__device__ __forceinline__ void mfma_half(f32x4 &acc, const i32x4 &w0, const i32x4 &w1,
                                          const i32x4 &t0, const i32x4 &t1, uint32_t ws,
                                          uint32_t ts) {
  if constexpr (F == FMT_BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w0),
                                                  __builtin_bit_cast(bf16x8, t0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w1),
                                                  __builtin_bit_cast(bf16x8, t1), acc, 0, 0, 0);
  } else if constexpr (F == FMT_F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(w0[e]), __int_as_float(t0[e]), acc,
                                                 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(w1[e]), __int_as_float(t1[e]), acc,
                                                 0, 0, 0);
  } else if constexpr (F == FMT_MX4) {
    // A: the half's E2M1 piece (w0; only four registers are read for E2M1),
    // operand format 4 = E2M1; B: fp8 E4M3 tokens
    const i32x4 z = {0, 0, 0, 0};
    const i32x8 a = __builtin_shufflevector(w0, z, 0, 1, 2, 3, 4, 5, 6, 7);
    const i32x8 b = __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 4, 0, WSEL, (int)ws, TSEL,
                                                           (int)ts);
  } else if constexpr (F == FMT_FP8) {
    // per-tensor scales are applied in the epilogue: unit block scales (127)
    const i32x8 a = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
    const i32x8 b = __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
  } else {
    const i32x8 a = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
    const i32x8 b = __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7);
    // operand format 0 = fp8 E4M3 for A and B; scale bytes WSEL and TSEL
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, WSEL, (int)ws, TSEL,
                                                           (int)ts);
  }
}

// One lane's operand for one half-chunk (pieces 2h and 2h + 1).  MX-fp8
// keeps both pieces in one 8-register tuple, the operand its scaled
// instruction reads, so nothing is copied between loading and multiplying.
template <int F>
struct Frag {
  i32x4 p0, p1;
};
template <>
struct Frag<FMT_MX8> {
  i32x8 v;
};
template <>
struct Frag<FMT_FP8> {
  i32x8 v;
};
// E2M1 weights: one 16-byte piece per half-chunk
template <>
struct Frag<FMT_MX4> {
  i32x4 v;
};

template <int F>
__device__ __forceinline__ Frag<F> make_frag(const i32x4 &a, const i32x4 &b) {
  Frag<F> f;
  if constexpr (F == FMT_MX8 || F == FMT_FP8) {
    f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  } else if constexpr (F == FMT_MX4) {
    f.v = a;
  } else {
    f.p0 = a;
    f.p1 = b;
  }
  return f;
}

// acc += W x T over one half-chunk from a weight fragment (format F) and a
// token fragment (format tok_fmt<F>).
template <int F, int WSEL = 0>
__device__ __forceinline__ void mfma_frag(f32x4 &acc, const Frag<F> &w, const Frag<tok_fmt<F>> &t,
                                          uint32_t ws, uint32_t ts) {
  if constexpr (F == FMT_MX8) {
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.v, t.v, acc, 0, 0, WSEL, (int)ws, 0,
                                                           (int)ts);
  } else if constexpr (F == FMT_MX4) {
    const i32x4 z = {0, 0, 0, 0};
    const i32x8 a = __builtin_shufflevector(w.v, z, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, t.v, acc, 4, 0, WSEL, (int)ws, 0,
                                                           (int)ts);
  } else if constexpr (F == FMT_FP8) {
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w.v, t.v, acc, 0, 0, 0, 127, 0, 127);
  } else {
    mfma_half<F>(acc, w.p0, w.p1, t.p0, t.p1, ws, ts);
  }
}

}  // namespace moe
