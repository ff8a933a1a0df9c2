// combine.hip -- FinalizeRouting and the shared-expert add.
//
// Hy3 on CANN NPU guide, section 8.5 (FinalizeRouting, then the final add of
// the shared expert); HunyuanImage-3.0 multi-stream article, source
// walkthrough part 3 (output = shared-MLP output + combined output):
//   out[t] = (sum_{j<k} w[t,j] * y[dest[t*k+j]]) + shared[t]
// accumulated in fp32, slot order j ascending, shared output added last.
// Memory-bound: a workgroup owns 2048 columns of one token row and every
// thread gathers 16 bytes of each of the k y rows at once.
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

constexpr int kMaxK = 16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Eight elements of y or the shared output, widened to fp32.  Both are read
// exactly once, so the loads are non-temporal: they do not displace cached
// lines (Hy3 prefill combine 0.131 -> 0.112 ms, MX-fp8 at T = 4096 0.067 ->
// 0.061 ms); the output keeps ordinary stores, so whatever reads it next
// finds it in the caches.
template <bool BF16>
__device__ __forceinline__ void load8(const void *base, long long off, float (&v)[8]) {
  if constexpr (BF16) {
    const u32x4 u = __builtin_nontemporal_load((const u32x4 *)((const uint16_t *)base + off));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4 *p = (const f32x4 *)((const float *)base + off);
    const f32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// Grid (T, ceil(H / 2048)): workgroup (t, slice) makes 2048 columns of row
// t, 8 per thread.  KT > 0 is k fixed at compile time, so every gathered
// load of a thread is issued before the first product; KT = 0 reads k at
// run time (at most kMaxK).
template <bool YBF16, bool OBF16, int KT>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y,
                                                      const int32_t *__restrict__ dest,
                                                      const float *__restrict__ topk_w,
                                                      const void *__restrict__ shared_out, int T,
                                                      int H, int k_rt, void *__restrict__ out) {
  constexpr int KM = KT > 0 ? KT : kMaxK;
  const int k = KT > 0 ? KT : k_rt;
  const int t = blockIdx.x;
  const int c = blockIdx.y * 2048 + threadIdx.x * 8;
  if (t >= T || c >= H) return;
  long long rows[KM];
  float w[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (KT > 0 || j < k) {
      rows[j] = (long long)dest[(long long)t * k + j] * H;
      w[j] = topk_w[(long long)t * k + j];
    }
  }
  float v[KM][8];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (KT > 0 || j < k) load8<YBF16>(y, rows[j] + c, v[j]);
  float sh[8];
  if (shared_out) load8<YBF16>(shared_out, (long long)t * H + c, sh);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (KT > 0 || j < k) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[j], v[j][i], acc[i]);
    }
  if (shared_out) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += sh[i];
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

template <bool YB, bool OB>
static void launch_combine_k(dim3 grid, const void *y, const int32_t *dest, const float *topk_w,
                             const void *shared_out, int T, int H, int k, void *out,
                             hipStream_t stream) {
  if (k == 8)
    combine_kernel<YB, OB, 8><<<grid, 256, 0, stream>>>(y, dest, topk_w, shared_out, T, H, k, out);
  else if (k == 4)
    combine_kernel<YB, OB, 4><<<grid, 256, 0, stream>>>(y, dest, topk_w, shared_out, T, H, k, out);
  else
    combine_kernel<YB, OB, 0><<<grid, 256, 0, stream>>>(y, dest, topk_w, shared_out, T, H, k, out);
}

hipError_t launch_combine(const void *y, int y_fmt, const int32_t *dest, const float *topk_w,
                          const void *shared_out, int T, int H, int k, void *out, int out_fmt,
                          hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  if (k > kMaxK || H % 8) return hipErrorInvalidValue;
  const bool yb = y_fmt == FMT_BF16, ob = out_fmt == FMT_BF16;
  const dim3 grid((unsigned)T, (unsigned)((H + 2047) / 2048));
  if (yb && ob)
    launch_combine_k<true, true>(grid, y, dest, topk_w, shared_out, T, H, k, out, stream);
  else if (!yb && !ob)
    launch_combine_k<false, false>(grid, y, dest, topk_w, shared_out, T, H, k, out, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
