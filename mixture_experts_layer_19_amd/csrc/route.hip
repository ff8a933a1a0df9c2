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
// Both logit kernels write fp32 partial dot products part[ks][t][e] over K
// slices; the top-k kernel adds the slices and the bias in fp64 and rounds
// z once to fp32.  Keeping every fp32 partial short keeps z within a few
// fp32 ulps of the exact dot product: the selection compares scores that may
// differ by far less than a plain fp32 running sum's error over 4096 terms.
//
// fp32 activations: FMA kernel.  Tile TT tokens x 64 experts, K staged
// through LDS 32 at a time; thread (tg, eg) owns tokens tg + 16 i and experts
// eg + 16 j; each 32-term slice is summed in fp32 and folded into fp64.

template <typename XT, int TT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT *__restrict__ x,
                                                            const float *__restrict__ Wr,
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
      if (e < E) z[(size_t)t * E + e] = (float)acc[i][j];
    }
  }
}

// bf16 activations: matrix-core kernel.  W_r is split exactly into three
// bf16 terms, w = hi + mid + lo (each remainder is exact in fp32 and the last
// holds at most 8 significant bits), so x . w = x . hi + x . mid + x . lo
// with every product exact in fp32; three bf16 MFMAs per step accumulate the
// sum in fp32.  Fragment layout as in moe_common.hpp with 128-element
// chunks: W_r rows are the A operand (lane row = expert), x rows the B
// operand (lane column = token).  Grid: (token tiles of 16*MBW, expert
// tiles of 64 = 4 waves x 16, K slices of KL).

__device__ __forceinline__ void split_bf16x3(const float (&v)[8], bf16x8 &hi, bf16x8 &mid,
                                             bf16x8 &lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t h = f32_to_bf16_rne(v[i]);
    const float r = v[i] - bf16_to_f32(h);
    const uint16_t m = f32_to_bf16_rne(r);
    const float r2 = r - bf16_to_f32(m);
    const uint16_t l = f32_to_bf16_rne(r2);
    hi[i] = __builtin_bit_cast(__bf16, h);
    mid[i] = __builtin_bit_cast(__bf16, m);
    lo[i] = __builtin_bit_cast(__bf16, l);
  }
}

template <int MBW>
__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t *__restrict__ x,
                                                          const float *__restrict__ Wr,
                                                          float *__restrict__ part, int T, int H,
                                                          int E, int KL) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int t0 = blockIdx.x * 16 * MBW;
  const int e0 = blockIdx.y * 64 + wave * 16;
  const int ks = blockIdx.z;
  const int ea = e0 + r;
  const float *wrow = Wr + (size_t)(ea < E ? ea : E - 1) * H;
  const uint16_t *xrow[MBW];
#pragma unroll
  for (int m = 0; m < MBW; ++m) {
    int t = t0 + 16 * m + r;
    xrow[m] = x + (size_t)(t < T ? t : T - 1) * H;
  }
  f32x4 acc[MBW];
#pragma unroll
  for (int m = 0; m < MBW; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int kend = (ks + 1) * KL;
  for (int kc = ks * KL; kc < kend; kc += 128) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int off = kc + chunk_off(g, p) / 2;
      const float4 w0 = *(const float4 *)(wrow + off);
      const float4 w1 = *(const float4 *)(wrow + off + 4);
      const float v[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      bf16x8 hi, mid, lo;
      split_bf16x3(v, hi, mid, lo);
#pragma unroll
      for (int m = 0; m < MBW; ++m) {
        const bf16x8 b = *(const bf16x8 *)(xrow[m] + off);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, b, acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc[m], 0, 0, 0);
      }
    }
  }
  // accumulator: expert e0 + 4 g + i, token t0 + 16 m + r
#pragma unroll
  for (int m = 0; m < MBW; ++m) {
    const int t = t0 + 16 * m + r;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = e0 + 4 * g + i;
      if (e < E) part[((size_t)ks * T + t) * E + e] = acc[m][i];
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
__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ part, int ksn,
                                                          const float *__restrict__ bias,
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
    if (e < E) {
      double zd = bias ? (double)bias[e] : 0.0;
      for (int ks = 0; ks < ksn; ++ks) zd += (double)part[((size_t)ks * T + t) * E + e];
      const float z = (float)zd;
      s[i] = (float)(1.0 / (1.0 + exp(-(double)z)));
    } else {
      s[i] = -INFINITY;
    }
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

// K slices of the bf16 logit kernel: short fp32 partials for small batches
// (which also spreads the few token tiles over many workgroups), long ones
// for large batches.
static void router_plan(int T, int H, int x_is_bf16, int &ksn, int &kl) {
  if (!x_is_bf16) { ksn = 1; kl = H; return; }
  kl = (T <= 256) ? 256 : 2048;
  if (H % kl) kl = 128;
  ksn = H / kl;
}

size_t route_ws_bytes(int T, int H, int E, int x_is_bf16) {
  int ksn, kl;
  router_plan(T, H, x_is_bf16, ksn, kl);
  return (size_t)ksn * T * E * sizeof(float);
}

hipError_t launch_route(const void *x, int x_is_bf16, const float *Wr, const float *bias,
                        float *part, int32_t *topk_idx, float *topk_w, int T, int H, int E, int k,
                        float rho, int route_norm, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  dim3 blk(256);
  int ksn, kl;
  router_plan(T, H, x_is_bf16, ksn, kl);
  if (x_is_bf16) {
    if (T <= 256) {
      dim3 grid((T + 15) / 16, (E + 63) / 64, ksn);
      router_mfma_kernel<1><<<grid, blk, 0, stream>>>((const uint16_t *)x, Wr, part, T, H, E, kl);
    } else {
      dim3 grid((T + 63) / 64, (E + 63) / 64, ksn);
      router_mfma_kernel<4><<<grid, blk, 0, stream>>>((const uint16_t *)x, Wr, part, T, H, E, kl);
    }
  } else {
    if (T <= 256) {
      dim3 grid((T + 15) / 16, (E + 63) / 64);
      router_logits_kernel<float, 16><<<grid, blk, 0, stream>>>((const float *)x, Wr, part, T, H, E);
    } else {
      dim3 grid((T + 63) / 64, (E + 63) / 64);
      router_logits_kernel<float, 64><<<grid, blk, 0, stream>>>((const float *)x, Wr, part, T, H, E);
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 g2((T + 3) / 4);
  int npl = (E + 63) / 64;
#define MOE_TOPK(N) \
  router_topk_kernel<N><<<g2, blk, 0, stream>>>(part, ksn, bias, topk_idx, topk_w, T, E, k, rho, route_norm)
  if (npl <= 1) MOE_TOPK(1);
  else if (npl <= 2) MOE_TOPK(2);
  else if (npl <= 4) MOE_TOPK(4);
  else if (npl <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
