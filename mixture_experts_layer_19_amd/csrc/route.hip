// route.hip -- Gating: router logits, sigmoid scores, top-k, route_norm, scaling.
//
// Hy3 on CANN NPU guide, section 1 (model overview): each token picks its
// top-8 of the routed experts by sigmoid score (moe_router_use_sigmoid), the
// selected scores are renormalised to sum to one (route_norm) and scaled by
// router_scaling_factor = 2.826.  Selection key: higher fp32 score first,
// lower expert index first among equal scores.
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

// --------------------------------------------------------------------------- logits
// z[t,e] = sum_h x[t,h] * Wr[e,h] + b[e], rounded once to fp32.  Tile: TT
// tokens x 64 experts per workgroup, K staged through LDS 32 at a time;
// thread (tg, eg) owns tokens tg + 16 i and experts eg + 16 j.  Each 32-term
// slice is summed with fp32 FMAs and folded into an fp64 accumulator, which
// keeps the logit within a few fp32 ulps of the exact dot product (the
// selection compares scores that may differ by far less than a plain fp32
// running sum's error over 4096 terms).

template <typename XT, int TT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT *__restrict__ x,
                                                            const float *__restrict__ Wr,
                                                            const float *__restrict__ bias,
                                                            float *__restrict__ z, int T, int H,
                                                            int E) {
  constexpr int TE = 64, KB = 32, TI = TT / 16;
  __shared__ float xs[TT][KB + 1];
  __shared__ float wsh[TE][KB + 1];
  const int tid = threadIdx.x;
  const int tg = tid & 15, eg = tid >> 4;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE;
  double acc[TI][4];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

  for (int k0 = 0; k0 < H; k0 += KB) {
    for (int idx = tid; idx < TT * KB; idx += 256) {
      int r = idx / KB, c = idx % KB;
      int t = t0 + r;
      float v = 0.0f;
      if (t < T) {
        if constexpr (sizeof(XT) == 2) v = bf16_to_f32(((const uint16_t *)x)[(size_t)t * H + k0 + c]);
        else v = ((const float *)x)[(size_t)t * H + k0 + c];
      }
      xs[r][c] = v;
    }
    for (int idx = tid; idx < TE * KB; idx += 256) {
      int r = idx / KB, c = idx % KB;
      int e = e0 + r;
      wsh[r][c] = (e < E) ? Wr[(size_t)e * H + k0 + c] : 0.0f;
    }
    __syncthreads();
    float part[TI][4];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) part[i][j] = 0.0f;
#pragma unroll 8
    for (int c = 0; c < KB; ++c) {
      float xv[TI], wv[4];
#pragma unroll
      for (int i = 0; i < TI; ++i) xv[i] = xs[tg + 16 * i][c];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = wsh[eg + 16 * j][c];
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) part[i][j] = fmaf(xv[i], wv[j], part[i][j]);
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += (double)part[i][j];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    int t = t0 + tg + 16 * i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = e0 + eg + 16 * j;
      if (e < E) z[(size_t)t * E + e] = (float)(acc[i][j] + (bias ? (double)bias[e] : 0.0));
    }
  }
}

// --------------------------------------------------------------------------- top-k
// One wave per token.  Lane l holds experts l, l+64, l+128, ... (up to
// E <= 64 * kMaxPerLane).  Scores s = fp32(1 / (1 + exp(-z))) are evaluated
// in fp64 and rounded once.  k rounds of a wave-wide arg-max pick the
// selection in key order; the selected scores are summed in slot order in
// fp64 and each weight rho * s / sum is rounded once to fp32.

constexpr int kMaxPerLane = 16;   // E <= 1024

__device__ __forceinline__ bool better(float sa, int a, float sb, int b) {
  return sa > sb || (sa == sb && a < b);
}

template <int NPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ z,
                                                          int32_t *__restrict__ topk_idx,
                                                          float *__restrict__ topk_w, int T, int E,
                                                          int k, float rho, int route_norm) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float s[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    int e = lane + 64 * i;
    s[i] = (e < E) ? (float)(1.0 / (1.0 + exp(-(double)z[(size_t)t * E + e]))) : -INFINITY;
  }
  unsigned taken = 0;      // bit i: s[i] already selected
  float sel_s = 0.0f;      // lane j < k keeps the j-th selection
  int sel_e = 0;
  for (int j = 0; j < k; ++j) {
    // lane-local best among the remaining candidates
    float bs = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      int e = lane + 64 * i;
      if (e < E && !(taken & (1u << i)) && better(s[i], e, bs, be)) { bs = s[i]; be = e; }
    }
    // wave-wide arg-max, ties to the lower expert index
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      float os = __shfl_xor(bs, m, 64);
      int oe = __shfl_xor(be, m, 64);
      if (better(os, oe, bs, be)) { bs = os; be = oe; }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) { sel_s = bs; sel_e = be; }
  }
  // sum of the selected scores in slot order, then the weights
  double den = 0.0;
  for (int j = 0; j < k; ++j) den += (double)__shfl(sel_s, j, 64);
  if (lane < k) {
    float wv = route_norm ? (float)((double)rho * (double)sel_s / den) : (float)((double)rho * sel_s);
    topk_idx[(size_t)t * k + lane] = sel_e;
    topk_w[(size_t)t * k + lane] = wv;
  }
}

hipError_t launch_route(const void *x, int x_is_bf16, const float *Wr, const float *bias,
                        float *logits, int32_t *topk_idx, float *topk_w, int T, int H, int E, int k,
                        float rho, int route_norm, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  dim3 blk(256);
  if (T <= 256) {
    dim3 grid((T + 15) / 16, (E + 63) / 64);
    if (x_is_bf16)
      router_logits_kernel<uint16_t, 16><<<grid, blk, 0, stream>>>((const uint16_t *)x, Wr, bias,
                                                                  logits, T, H, E);
    else
      router_logits_kernel<float, 16><<<grid, blk, 0, stream>>>((const float *)x, Wr, bias, logits,
                                                               T, H, E);
  } else {
    dim3 grid((T + 63) / 64, (E + 63) / 64);
    if (x_is_bf16)
      router_logits_kernel<uint16_t, 64><<<grid, blk, 0, stream>>>((const uint16_t *)x, Wr, bias,
                                                                  logits, T, H, E);
    else
      router_logits_kernel<float, 64><<<grid, blk, 0, stream>>>((const float *)x, Wr, bias, logits,
                                                               T, H, E);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 g2((T + 3) / 4);
  int npl = (E + 63) / 64;
  if (npl <= 1)
    router_topk_kernel<1><<<g2, blk, 0, stream>>>(logits, topk_idx, topk_w, T, E, k, rho, route_norm);
  else if (npl <= 2)
    router_topk_kernel<2><<<g2, blk, 0, stream>>>(logits, topk_idx, topk_w, T, E, k, rho, route_norm);
  else if (npl <= 4)
    router_topk_kernel<4><<<g2, blk, 0, stream>>>(logits, topk_idx, topk_w, T, E, k, rho, route_norm);
  else if (npl <= 8)
    router_topk_kernel<8><<<g2, blk, 0, stream>>>(logits, topk_idx, topk_w, T, E, k, rho, route_norm);
  else
    router_topk_kernel<16><<<g2, blk, 0, stream>>>(logits, topk_idx, topk_w, T, E, k, rho, route_norm);
  return hipGetLastError();
}

}  // namespace moe
