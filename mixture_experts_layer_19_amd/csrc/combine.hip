// combine.hip -- FinalizeRouting and the shared-expert add.
//
// Hy3 on CANN NPU guide, section 8.5 (FinalizeRouting, then the final add of
// the shared expert); HunyuanImage-3.0 multi-stream article, source
// walkthrough part 3 (output = shared-MLP output + combined output):
//   out[t] = (sum_{j<k} w[t,j] * y[dest[t*k+j]]) + shared[t]
// accumulated in fp32, slot order j ascending, shared output added last.
// Memory-bound: each workgroup owns one token row; every thread moves 16
// bytes per access of each of the k gathered y rows.
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

constexpr int kMaxK = 16;

template <bool BF16>
__device__ __forceinline__ void load8(const void *base, long long off, float (&v)[8]) {
  if constexpr (BF16) {
    uint4 u = *(const uint4 *)((const uint16_t *)base + off);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4 *p = (const float4 *)((const float *)base + off);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool YBF16, bool OBF16>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y,
                                                      const int32_t *__restrict__ dest,
                                                      const float *__restrict__ topk_w,
                                                      const void *__restrict__ shared_out, int T,
                                                      int H, int k, void *__restrict__ out) {
  const int t = blockIdx.x;
  if (t >= T) return;
  long long rows[kMaxK];
  float w[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      rows[j] = (long long)dest[(long long)t * k + j] * H;
      w[j] = topk_w[(long long)t * k + j];
    }
  }
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        float v[8];
        load8<YBF16>(y, rows[j] + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[j], v[i], acc[i]);
      }
    }
    if (shared_out) {
      float v[8];
      load8<YBF16>(shared_out, (long long)t * H + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    if constexpr (OBF16) {
      uint32_t wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        wv[i] = (uint32_t)f32_to_bf16_rne(acc[2 * i]) | ((uint32_t)f32_to_bf16_rne(acc[2 * i + 1]) << 16);
      *(uint4 *)((uint16_t *)out + (long long)t * H + c) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    } else {
      float4 *o = (float4 *)((float *)out + (long long)t * H + c);
      o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

hipError_t launch_combine(const void *y, int y_fmt, const int32_t *dest, const float *topk_w,
                          const void *shared_out, int T, int H, int k, void *out, int out_fmt,
                          hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (k > kMaxK || H % 8) return hipErrorInvalidValue;
  const bool yb = y_fmt == FMT_BF16, ob = out_fmt == FMT_BF16;
  if (yb && ob)
    combine_kernel<true, true><<<T, 256, 0, stream>>>(y, dest, topk_w, shared_out, T, H, k, out);
  else if (!yb && !ob)
    combine_kernel<false, false><<<T, 256, 0, stream>>>(y, dest, topk_w, shared_out, T, H, k, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
