// mx.hip -- MX-fp8 quantisation of activations and packing of expert weights.
//
// MX-fp8 follows the OCP Microscaling Formats (MX) v1.0 specification: blocks
// of 32 consecutive elements along the reduction axis share one E8M0 scale
// X + 127 with X = floor(log2 max|v|) - 8 (8 is the exponent of E4M3's
// largest normal, 448), clamped to [-127, 127]; each element is the E4M3 (FN)
// round-to-nearest-even of v / 2^X, saturated to +-448.  The Hy3 on CANN NPU
// guide (section 8.2) quantises linear layers to MXFP8 (W8A8) with the
// activations quantised on the fly.
//
// Weight packing produces the 4 KiB fragment blocks described in
// moe_common.hpp, ordered [expert][16-row block][256-byte K chunk] (2 KiB
// blocks of 256 K elements for MXFP4, whose E2M1 elements follow the same
// OCP specification with X = floor(log2 max|v|) - 2).  For the
// gate/up matrix the row blocks alternate: block 2j holds gate rows
// 16j..16j+15 and block 2j+1 the up rows with the same indices, so the SwiGLU
// epilogue finds a gate value and its up value in the same lane.
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

template <bool BF16>
__device__ __forceinline__ float load_src(const void *p, long long i) {
  if constexpr (BF16) return bf16_to_f32(((const uint16_t *)p)[i]);
  else return ((const float *)p)[i];
}

// v[0..N) = src[i0, i0 + N) widened to fp32; VEC: with 16-byte loads (the
// address of element i0 is 16-byte aligned), else one element at a time.
template <bool BF16, bool VEC, int N>
__device__ __forceinline__ void load_run(const void *src, long long i0, float (&v)[N]) {
  if constexpr (VEC && BF16) {
    static_assert(N % 8 == 0, "whole 16-byte vectors");
    const uint4 *p = (const uint4 *)((const uint16_t *)src + i0);
#pragma unroll
    for (int q = 0; q < N / 8; ++q) {
      const uint4 u = p[q];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * q + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * q + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  } else if constexpr (VEC) {
    static_assert(N % 4 == 0, "whole 16-byte vectors");
    const float4 *p = (const float4 *)((const float *)src + i0);
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const float4 a = p[q];
      v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = load_src<BF16>(src, i0 + i);
  }
}

// Quantise 32 values v[0..31] (registers) to codes and scale byte.
__device__ __forceinline__ void mx_block(const float (&v)[32], uint32_t (&codes)[8], uint32_t &sb) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
  sb = mx_scale_byte(am);
  const float inv = mx_inv_scale(sb);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t c = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) c |= e4m3_rne(v[4 * w + b] * inv) << (8 * b);
    codes[w] = c;
  }
}

// Quantise 32 values to MXFP4: E2M1 codes (nibble i of word i / 8, low
// nibble first) and the scale byte.
__device__ __forceinline__ void mx4_block(const float (&v)[32], uint32_t (&codes)[4],
                                          uint32_t &sb) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
  sb = mx4_scale_byte(am);
  const float inv = mx_inv_scale(sb);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) c |= e2m1_rne(v[8 * w + j] * inv) << (4 * j);
    codes[w] = c;
  }
}

// ----------------------------------------------------------------------------- activations
// One thread per 32-element block of a row-major [rows, cols] matrix.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const void *__restrict__ src,
                                                          long long rows, long long cols,
                                                          uint8_t *__restrict__ q,
                                                          uint8_t *__restrict__ scale) {
  const long long nblk = rows * (cols / 32);
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblk) return;
  float v[32];
  load_run<BF16, VEC>(src, b * 32, v);
  uint32_t codes[8], sb;
  mx_block(v, codes, sb);
  uint4 *o = (uint4 *)(q + b * 32);
  o[0] = make_uint4(codes[0], codes[1], codes[2], codes[3]);
  o[1] = make_uint4(codes[4], codes[5], codes[6], codes[7]);
  scale[b] = (uint8_t)sb;
}

hipError_t launch_mx_quantize(const void *src, int src_is_bf16, long long rows, long long cols,
                              uint8_t *q, uint8_t *scale, hipStream_t stream) {
  const long long nblk = rows * (cols / 32);
  if (nblk <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((nblk + 255) / 256);
  // every 32-element block starts 16-byte aligned when the array does
  const bool vec = ((uintptr_t)src & 15) == 0;
  if (src_is_bf16 && vec)
    mx_quantize_kernel<true, true><<<grid, 256, 0, stream>>>(src, rows, cols, q, scale);
  else if (src_is_bf16)
    mx_quantize_kernel<true, false><<<grid, 256, 0, stream>>>(src, rows, cols, q, scale);
  else if (vec)
    mx_quantize_kernel<false, true><<<grid, 256, 0, stream>>>(src, rows, cols, q, scale);
  else
    mx_quantize_kernel<false, false><<<grid, 256, 0, stream>>>(src, rows, cols, q, scale);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- static FP8
// Static per-tensor FP8 (the FP8 / w8a8 checkpoints of the Hy3 and Hy4
// families): one fp32 scale per weight tensor, max|w| / 448, and fixed
// activation scales; codes are E4M3 of fp32(v / scale).
// E4M3 codes of fp32(src / scale): one thread per 8 elements (n % 8 == 0).
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const void *__restrict__ src,
                                                           long long n8, float scale,
                                                           uint8_t *__restrict__ q) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float v[8];
  load_run<BF16, VEC>(src, 8 * i, v);
  uint32_t c[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j >> 2] |= e4m3_rne(v[j] / scale) << (8 * (j & 3));
  *(uint2 *)(q + 8 * i) = make_uint2(c[0], c[1]);
}

hipError_t launch_fp8_quantize(const void *src, int src_is_bf16, long long n, float scale,
                               uint8_t *q, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  const long long n8 = n / 8;
  const unsigned grid = (unsigned)((n8 + 255) / 256);
  // runs of 8 elements start 16-byte aligned when the array does
  const bool vec = ((uintptr_t)src & 15) == 0;
  if (src_is_bf16 && vec)
    fp8_quantize_kernel<true, true><<<grid, 256, 0, stream>>>(src, n8, scale, q);
  else if (src_is_bf16)
    fp8_quantize_kernel<true, false><<<grid, 256, 0, stream>>>(src, n8, scale, q);
  else if (vec)
    fp8_quantize_kernel<false, true><<<grid, 256, 0, stream>>>(src, n8, scale, q);
  else
    fp8_quantize_kernel<false, false><<<grid, 256, 0, stream>>>(src, n8, scale, q);
  return hipGetLastError();
}

// Per-tensor weight scale of each source matrix: workgroup m reduces matrix
// m (m = e * nmat + j; j selects source a or b) of `elems` elements to its
// largest magnitude and writes max / 448 (1 for an all-zero matrix).
template <bool BF16>
__global__ __launch_bounds__(256) void fp8_tensor_scale_kernel(const void *__restrict__ a,
                                                               const void *__restrict__ b,
                                                               int nmat, long long elems,
                                                               float *__restrict__ tscale) {
  const int m = blockIdx.x, e = m / nmat, j = m % nmat;
  const void *src = j ? b : a;
  const long long base = (long long)e * elems;
  float am = 0.0f;
  for (long long i = threadIdx.x; i < elems; i += 256) am = fmaxf(am, fabsf(load_src<BF16>(src, base + i)));
  __shared__ float red[256];
  red[threadIdx.x] = am;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) tscale[m] = red[0] == 0.0f ? 1.0f : red[0] / 448.0f;
}

// ----------------------------------------------------------------------------- weights
// One thread per (expert, virtual row, K chunk): it converts the row's 256
// chunk bytes and scatters them into the fragment block -- piece p of lane
// group g is chunk bytes off(g, p) -- and, for MX, quantises the chunk's
// eight 32-element blocks; lane group g of half h receives the scale byte of
// block 4h + g (bits 8h..8h+7 of its uint16).
template <bool BF16, int F>
__global__ __launch_bounds__(256) void pack_kernel(const void *__restrict__ a,
                                                   const void *__restrict__ b, int E, int N, int K,
                                                   int gate_up, uint8_t *__restrict__ out,
                                                   uint16_t *__restrict__ scale_out,
                                                   const float *__restrict__ tscale) {
  constexpr int CE = FmtInfo<F>::chunk_elems;
  constexpr int EB = FmtInfo<F>::elem_bytes;
  const int nbtot = N / 16, kcn = K / CE;
  const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)E * N * kcn;
  if (tid >= total) return;
  const int kc = (int)(tid % kcn);
  const long long rest = tid / kcn;
  const int v = (int)(rest % N);            // virtual row (gate/up interleaved by 16-row blocks)
  const int e = (int)(rest / N);
  const int nb = v >> 4, r16 = v & 15;
  const void *src;
  long long row;
  int src_rows;
  if (gate_up) {
    src = (nb & 1) ? b : a;
    src_rows = N / 2;
    row = (long long)(nb >> 1) * 16 + r16;
  } else {
    src = a;
    src_rows = N;
    row = v;
  }
  const long long base = ((long long)e * src_rows + row) * K + (long long)kc * CE;
  uint8_t *blk = out + (((long long)e * nbtot + nb) * kcn + kc) * wblock_bytes<F>;
  if constexpr (F == FMT_MX4) {
    // E2M1: lane group g of half h holds MX block 4h + g of the row (16
    // bytes, contiguous K) and supplies its scale, like the MX-fp8 layout
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float vals[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) vals[i] = load_src<BF16>(src, base + 32 * (4 * h + g) + i);
        uint32_t c[4];
        mx4_block(vals, c, sc[h]);
        *(uint4 *)(blk + h * 1024 + (r16 + 16 * g) * 16) = make_uint4(c[0], c[1], c[2], c[3]);
      }
      scale_out[(((long long)e * nbtot + nb) * kcn + kc) * 64 + r16 + 16 * g] =
          (uint16_t)(sc[0] | (sc[1] << 8));
    }
  } else if constexpr (F == FMT_MX8 || F == FMT_FP8) {
    uint32_t sc[8];
    uint32_t codes[8][8];
    if constexpr (F == FMT_FP8) {
      // one scale for the whole source matrix (gate or up of the expert)
      const float ts = tscale[gate_up ? 2 * e + (nb & 1) : e];
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          uint32_t c = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            c |= e4m3_rne(load_src<BF16>(src, base + 32 * m + 4 * w + q) / ts) << (8 * q);
          codes[m][w] = c;
        }
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        float vals[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) vals[i] = load_src<BF16>(src, base + 32 * m + i);
        mx_block(vals, codes[m], sc[m]);
      }
    }
    // chunk byte o lives in MX block o / 32, code word (o % 32) / 4
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int o = chunk_off(g, p);
        const uint32_t *c = &codes[o >> 5][(o & 31) >> 2];
        *(uint4 *)(blk + p * 1024 + (r16 + 16 * g) * 16) = make_uint4(c[0], c[1], c[2], c[3]);
      }
      if constexpr (F == FMT_MX8)
        scale_out[(((long long)e * nbtot + nb) * kcn + kc) * 64 + r16 + 16 * g] =
            (uint16_t)(sc[g] | (sc[4 + g] << 8));
    }
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const long long k0 = base + chunk_off(g, p) / EB;
        uint32_t wv[4];
        if constexpr (F == FMT_BF16) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            wv[i] = (uint32_t)f32_to_bf16_rne(load_src<BF16>(src, k0 + 2 * i)) |
                    ((uint32_t)f32_to_bf16_rne(load_src<BF16>(src, k0 + 2 * i + 1)) << 16);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) wv[i] = __float_as_uint(load_src<BF16>(src, k0 + i));
        }
        *(uint4 *)(blk + p * 1024 + (r16 + 16 * g) * 16) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
    }
  }
}

hipError_t launch_pack(const void *a, const void *b, int src_is_bf16, int E, int N, int K,
                       int gate_up, int fmt, uint8_t *out, uint16_t *scale_out, float *tscale,
                       hipStream_t stream) {
  int ce = fmt == FMT_F32 ? 64 : (fmt == FMT_BF16 ? 128 : 256);
  if (fmt < FMT_F32 || fmt > FMT_FP8) return hipErrorInvalidValue;
  const long long total = (long long)E * N * (K / ce);
  if (total <= 0) return hipSuccess;
  if (fmt == FMT_FP8) {
    // per-tensor scales first: one workgroup per source matrix
    const int nmat = gate_up ? 2 : 1;
    const long long elems = (long long)(N / nmat) * K;
    if (src_is_bf16)
      fp8_tensor_scale_kernel<true><<<E * nmat, 256, 0, stream>>>(a, b, nmat, elems, tscale);
    else
      fp8_tensor_scale_kernel<false><<<E * nmat, 256, 0, stream>>>(a, b, nmat, elems, tscale);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const unsigned grid = (unsigned)((total + 255) / 256);
#define MOE_PACK(BF, F)                                                                        \
  pack_kernel<BF, F><<<grid, 256, 0, stream>>>(a, b, E, N, K, gate_up, out, scale_out, tscale)
  if (src_is_bf16) {
    if (fmt == FMT_F32) MOE_PACK(true, FMT_F32);
    else if (fmt == FMT_BF16) MOE_PACK(true, FMT_BF16);
    else if (fmt == FMT_MX8) MOE_PACK(true, FMT_MX8);
    else if (fmt == FMT_MX4) MOE_PACK(true, FMT_MX4);
    else MOE_PACK(true, FMT_FP8);
  } else {
    if (fmt == FMT_F32) MOE_PACK(false, FMT_F32);
    else if (fmt == FMT_BF16) MOE_PACK(false, FMT_BF16);
    else if (fmt == FMT_MX8) MOE_PACK(false, FMT_MX8);
    else if (fmt == FMT_MX4) MOE_PACK(false, FMT_MX4);
    else MOE_PACK(false, FMT_FP8);
  }
#undef MOE_PACK
  return hipGetLastError();
}

}  // namespace moe
