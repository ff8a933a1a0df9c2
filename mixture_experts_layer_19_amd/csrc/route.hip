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
// fp32 activations: FMA kernel.  Tile TT tokens x 64 experts; the K axis is
// cut into gridDim.z slices of nkb whole 32-element blocks.  A workgroup
// sums its slice block by block (fp32 within a block, fp64 across blocks)
// and writes it rounded to fp32 as part[slice][t][e].  Blocks are staged
// through LDS; the loads of block b + 1 go out before block b is multiplied.
// Thread (tg, eg) owns tokens tg + 16 i and experts eg + 16 j.

template <typename XT, int TT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT *__restrict__ x,
                                                            const float *__restrict__ Wr,
                                                            float *__restrict__ part, int T, int H,
                                                            int E, int nkb) {
  constexpr int TE = 64, KB = 32, TI = TT / 16;
  constexpr int XL = TT * KB / 256, WL = TE * KB / 256;   // loads per thread and block
  __shared__ float xs[TT][KB + 1];
  __shared__ float wsh[TE][KB + 1];
  const int tid = threadIdx.x;
  const int tg = tid & 15, eg = tid >> 4;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE;
  const int kb0 = blockIdx.z * nkb, kb1 = min(H / KB, kb0 + nkb);
  float xr[XL], wr[WL];
  auto load = [&](int kb) MOE_INLINE {
    const int k0 = kb * KB;
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int idx = tid + 256 * i, t = t0 + idx / KB, c = idx % KB;
      float v = 0.0f;
      if (t < T) {
        if constexpr (sizeof(XT) == 2) v = bf16_to_f32(((const uint16_t *)x)[(size_t)t * H + k0 + c]);
        else v = ((const float *)x)[(size_t)t * H + k0 + c];
      }
      xr[i] = v;
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      const int idx = tid + 256 * i, e = e0 + idx / KB, c = idx % KB;
      wr[i] = (e < E) ? Wr[(size_t)e * H + k0 + c] : 0.0f;
    }
  };
  double acc[TI][4];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;

  load(kb0);
  for (int kb = kb0; kb < kb1; ++kb) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int idx = tid + 256 * i;
      xs[idx / KB][idx % KB] = xr[i];
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      const int idx = tid + 256 * i;
      wsh[idx / KB][idx % KB] = wr[i];
    }
    __syncthreads();
    if (kb + 1 < kb1) load(kb + 1);
    float p[TI][4];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) p[i][j] = 0.0f;
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
        for (int j = 0; j < 4; ++j) p[i][j] = fmaf(xv[i], wv[j], p[i][j]);
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += (double)p[i][j];
    __syncthreads();
  }
  float *out = part + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    int t = t0 + tg + 16 * i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = e0 + eg + 16 * j;
      if (e < E) out[(size_t)t * E + e] = (float)acc[i][j];
    }
  }
}

// Batches of at most this many tokens: the router GEMM splits the fp32
// weights itself, stage by stage, instead of reading a copy split once per
// call by router_split_kernel.  Both give the same bits.  On large batches
// the split repeated by every token tile costs more than the separate pass
// (gating at T = 2048 / 4096 / 8192: 53 / 66 / 107 us fused against 48 / 58
// / 92), so they keep it.
constexpr int kRouterFusedSplitT = 256;

// Slices of at most this many 64-element stages issue all their loads at
// once (router_gemm_kernel's NSH path).
constexpr int kRouterShortStages = 4;

// bf16 activations: matrix-core kernels.  W_r is split exactly into three
// bf16 terms, w = hi + mid + lo: hi is w truncated to its leading 8
// significant bits, mid the leading 8 of the remainder w - hi, lo the rest
// (each remainder is exact in fp32, and the 24-bit significand leaves at
// most 8 bits for lo; for |w| < 2^-110 lo falls below the normal range and
// keeps only its bits down to 2^-133), so x . w = x . hi + x . mid + x . lo
// with every product exact in fp32; three bf16 MFMAs per step accumulate
// the sum in fp32.  For large batches the split is done once per call by
// router_split_kernel into fragment order, and router_gemm_kernel only loads
// and multiplies; for small ones the GEMM splits the fp32 rows it loads.
//
// Fragment layout as in moe_common.hpp: W_r rows are the A operand (lane
// row = expert), x rows the B operand (lane column = token).  A stage is 64
// K elements (half a 128-element chunk); in stage s lane (g, r) holds, for
// piece pp = 0, 1, the 8 elements from K = 64 s + 32 pp + 8 g.  The split
// weights are stored [term][expert block][stage][pp][lane][8 bf16], so one
// wave-wide 16-byte load reads a contiguous KiB.

// Eight fp32 values -> the three terms, each as four dwords of two bf16
// (element 2 j in the low half of dword j).  A term's bf16 is the upper half
// of its fp32 bits (the lower half is zero for hi and mid by construction,
// and for lo because it holds at most 8 significant bits); one byte
// permute packs two of them.
__device__ __forceinline__ void split_bf16x3(const float (&v)[8], uint32_t (&t)[3][4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t b[3][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t h = __float_as_uint(v[2 * j + u]) & 0xFFFF0000u;
      const float r = v[2 * j + u] - __uint_as_float(h);
      const uint32_t m = __float_as_uint(r) & 0xFFFF0000u;
      const float l = r - __uint_as_float(m);
      b[0][u] = h;
      b[1][u] = m;
      b[2][u] = __float_as_uint(l);
    }
#pragma unroll
    for (int term = 0; term < 3; ++term)
      t[term][j] = __builtin_amdgcn_perm(b[term][1], b[term][0], 0x07060302u);
  }
}

// One thread per (expert block, stage, pp, lane); experts past E are zero.
__global__ __launch_bounds__(256) void router_split_kernel(const float *__restrict__ Wr, int E,
                                                           int H, int EB, uint4 *__restrict__ out) {
  const int nst = H / 64;
  const long long per_term = (long long)EB * nst * 2 * 64;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_term) return;
  const int lane = (int)(i & 63), pp = (int)((i >> 6) & 1);
  const long long q = i >> 7;
  const int st = (int)(q % nst), eb = (int)(q / nst);
  const int e = eb * 16 + (lane & 15), k0 = 64 * st + 32 * pp + 8 * (lane >> 4);
  float v[8];
  if (e < E) {
    const float4 a = *(const float4 *)(Wr + (size_t)e * H + k0);
    const float4 b = *(const float4 *)(Wr + (size_t)e * H + k0 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  }
  uint32_t t[3][4];
  split_bf16x3(v, t);
#pragma unroll
  for (int term = 0; term < 3; ++term) out[term * per_term + i] = uint4{t[term][0], t[term][1], t[term][2], t[term][3]};
}

// Workgroup: 4 waves, 16 MBT tokens x 64 experts; wave w takes expert block
// w of the workgroup's range and all MBT token blocks.  The token tile (one
// 128-byte line per row and stage) is staged through LDS, double-buffered,
// with the same slot permutation as the expert GEMM; the split weights go
// from global memory into registers WPF stages ahead.  The work per loaded
// byte is small, so latency is hidden by depth and by many resident waves
// (few registers per wave).
//
// Work order: K slice major, then token tile, then expert tile.  The 1-D
// grid is dealt round-robin to the 8 XCDs and each XCD takes one contiguous
// range of that order, so an XCD's L2 holds the split weights of one or two
// K slices while the expert tiles that share a token tile run side by side.
//
// NSH > 0 (slices of at most NSH stages, as in small batches): the loads of
// every stage go out at once, each stage's token tile gets an LDS slot of its
// own, and one barrier separates the loads from the products, so the
// workgroup waits for memory once instead of once per stage.
template <int MBT, int WPF, bool FS, int NSH = 0>
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t *__restrict__ x,
                                                          const uint4 *__restrict__ wsplit,
                                                          const float *__restrict__ Wr,
                                                          float *__restrict__ part, int T, int H,
                                                          int E, int EB, int nsl, int n_et,
                                                          int n_tt, int ksn) {
  constexpr int TBYTES = MBT * 2048;
  constexpr int TLD = MBT * 16 * 8 / 256;   // 16-byte token loads per thread per stage
  constexpr int NSET = NSH > 0 ? NSH : WPF + 1;
  static_assert(TLD >= 1, "tile shape");
  constexpr int PBYTES = NSH > 0 ? 16 : TBYTES;     // the pipelined path's two slots
  __shared__ __attribute__((aligned(16))) uint8_t tb0[PBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t tb1[PBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t tbn[NSH > 0 ? NSH : 1][NSH > 0 ? TBYTES : 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int total = n_et * n_tt * ksn, per_xcd = (total + 7) >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd || logical >= total) return;
  const int et = logical % n_et, tt = (logical / n_et) % n_tt, ks = logical / (n_et * n_tt);
  const int t0 = tt * 16 * MBT;
  const int eb = min(et * 4 + wave, EB - 1);   // loads; stores test the real block
  const bool eb_ok = et * 4 + wave < EB;
  const int nst = H / 64, s_begin = ks * nsl;
  const int s_end = min(nst, s_begin + nsl);
  if (s_begin >= nst) return;
  const long long per_term = (long long)EB * nst * 2 * 64;
  const uint4 *wbase = wsplit + (long long)eb * nst * 128 + lane;

  // token rows of this thread (clamped into [0, T))
  const uint8_t *tsrc[TLD];
  int tdst[TLD];
#pragma unroll
  for (int i = 0; i < TLD; ++i) {
    const int idx = tid + 256 * i, rl = idx >> 3, seg = idx & 7;
    const int t = min(t0 + rl, T - 1);
    tsrc[i] = (const uint8_t *)(x + (size_t)t * H) + seg * 16;
    tdst[i] = (rl >> 4) * 2048 + (seg >> 2) * 1024 + tslot(rl & 15, seg & 3, seg >> 2) * 16;
  }
  i32x4 treg[TLD];
  auto load_tokens = [&](int s) MOE_INLINE {
#pragma unroll
    for (int i = 0; i < TLD; ++i) treg[i] = *(const i32x4 *)(tsrc[i] + s * 128);
  };
  auto store_tokens = [&](uint8_t *buf) MOE_INLINE {
#pragma unroll
    for (int i = 0; i < TLD; ++i) *(i32x4 *)(buf + tdst[i]) = treg[i];
  };
  // FS: fp32 weights of one stage, [pp][2 x 4 elements], split into the
  // three bf16 terms when the stage multiplies them.  Otherwise the split
  // fragments of one stage, [term][pp].
  const int we = 16 * eb + (lane & 15);
  const bool we_ok = we < E;
  const float *wrow = Wr + (size_t)min(we, E - 1) * H + 8 * (lane >> 4);
  f32x4 wf[NSET][2][2];
  i32x4 wr[NSET][3][2];
  auto load_weights = [&](int s, int set) MOE_INLINE {
    if constexpr (FS) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4 v = *(const f32x4 *)(wrow + 64 * s + 32 * pp + 4 * h);
#pragma unroll
          for (int q = 0; q < NSET; ++q)
            if (q == set) wf[q][pp][h] = v;
        }
    } else {
#pragma unroll
      for (int term = 0; term < 3; ++term)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const uint4 v = wbase[term * per_term + (long long)s * 128 + pp * 64];
#pragma unroll
          for (int q = 0; q < NSET; ++q)
            if (q == set) wr[q][term][pp] = i32x4{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        }
    }
  };
  auto split_weights = [&](int set, i32x4 (&w)[3][2]) MOE_INLINE {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = we_ok ? wf[set][pp][0][j] : 0.0f;
        v[4 + j] = we_ok ? wf[set][pp][1][j] : 0.0f;
      }
      uint32_t t[3][4];
      split_bf16x3(v, t);
#pragma unroll
      for (int term = 0; term < 3; ++term)
        w[term][pp] = i32x4{(int)t[term][0], (int)t[term][1], (int)t[term][2], (int)t[term][3]};
    }
  };
  f32x4 acc[MBT];
#pragma unroll
  for (int m = 0; m < MBT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the products of one stage: weights in register set `set`, tokens at base
  auto products = [&](auto set_c, const uint8_t *base) MOE_INLINE {
    constexpr int set = decltype(set_c)::value;
    i32x4 ws[3][2];
    if constexpr (FS) {
      split_weights(set, ws);
    } else {
#pragma unroll
      for (int term = 0; term < 3; ++term)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) ws[term][pp] = wr[set][term][pp];
    }
#pragma unroll
    for (int m = 0; m < MBT; ++m) {
      const uint8_t *p = base + m * 2048;
      const i32x4 b0 = *(const i32x4 *)(p + tslot(lane & 15, lane >> 4, 0) * 16);
      const i32x4 b1 = *(const i32x4 *)(p + 1024 + tslot(lane & 15, lane >> 4, 1) * 16);
#pragma unroll
      for (int term = 0; term < 3; ++term) {
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, ws[term][0]), __builtin_bit_cast(bf16x8, b0), acc[m], 0,
            0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, ws[term][1]), __builtin_bit_cast(bf16x8, b1), acc[m], 0,
            0, 0);
      }
    }
  };
  // stage s of the pipelined path: weights in register set `set`, tokens in
  // LDS slot `slot`
  auto stage = [&](int s, auto set_c, auto slot_c) MOE_INLINE {
    constexpr int set = decltype(set_c)::value, slot = decltype(slot_c)::value;
    load_weights(min(s + WPF, s_end - 1), (set + WPF) % NSET);
    products(set_c, slot ? tb1 : tb0);
    store_tokens(slot ? tb0 : tb1);
    load_tokens(min(s + 2, s_end - 1));
    __syncthreads();
  };

  if constexpr (NSH > 0) {
    // A stage past the slice's end loads the last stage again and stores a
    // zero token tile, so its products add exactly zero: every product is
    // unconditional, which keeps all loads ahead of the barrier.
    i32x4 tall[NSH][TLD];
    static_for<NSH>([&](auto q) MOE_INLINE {
      load_tokens(min(s_begin + q.value, s_end - 1));
#pragma unroll
      for (int i = 0; i < TLD; ++i) tall[q.value][i] = treg[i];
    });
    static_for<NSH>([&](auto q) MOE_INLINE { load_weights(min(s_begin + q.value, s_end - 1), q.value); });
    static_for<NSH>([&](auto q) MOE_INLINE {
      const bool live = s_begin + q.value < s_end;
#pragma unroll
      for (int i = 0; i < TLD; ++i)
        *(i32x4 *)(tbn[q.value] + tdst[i]) = live ? tall[q.value][i] : i32x4{0, 0, 0, 0};
    });
    __syncthreads();
    static_for<NSH>([&](auto q) MOE_INLINE { products(std::integral_constant<int, q.value>{}, tbn[q.value]); });
  } else {
  load_tokens(s_begin);
#pragma unroll
  for (int q = 0; q < WPF; ++q) load_weights(min(s_begin + q, s_end - 1), q);
  store_tokens(tb0);
  load_tokens(min(s_begin + 1, s_end - 1));
  __syncthreads();
  // periods of P = lcm(NSET, 2) stages keep set and slot compile-time
  constexpr int P = (NSET % 2 == 0) ? NSET : 2 * NSET;
  auto stage_q = [&](int s, auto q) MOE_INLINE {
    constexpr int Q = decltype(q)::value;
    stage(s, std::integral_constant<int, Q % NSET>{}, std::integral_constant<int, Q % 2>{});
  };
  int s = s_begin;
  for (; s + P <= s_end; s += P) static_for<P>([&](auto q) MOE_INLINE { stage_q(s + q.value, q); });
  static_for<P - 1>([&](auto q) MOE_INLINE {
    if (s + q.value < s_end) stage_q(s + q.value, q);
  });
  }

  // accumulator: expert 16 eb + 4 g + i, token t0 + 16 m + r
  const int g = lane >> 4, r = lane & 15;
#pragma unroll
  for (int m = 0; m < MBT; ++m) {
    const int t = t0 + 16 * m + r;
    if (t >= T || !eb_ok) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 16 * eb + 4 * g + i;
      if (e < E) part[((size_t)ks * T + t) * E + e] = acc[m][i];
    }
  }
}

// --------------------------------------------------------------------------- top-k
// One wave per token.  Lane l holds experts l, l+64, l+128, ... (up to
// E <= 64 * kMaxPerLane), or four consecutive ones (PK below).  Scores
// s = fp32(1 / (1 + exp(-z))) are evaluated in fp64 and rounded once.  The
// selection key of expert e is the 64-bit number bits(s) * 2^32 +
// (2^32 - 1 - e): scores are never negative, so their bit patterns order
// like their values, and of two equal scores the lower expert index has the
// larger key (a NaN score counts as zero, in the ranking and in the weights,
// so the selection is always k valid experts).  k rounds of a wave-wide key
// maximum pick the selection in key order; the selected scores are summed
// in slot order in fp64 and each weight rho * s / sum is rounded once to
// fp32.

constexpr int kMaxPerLane = 16;   // E <= 1024

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Maximum over the 64 lanes of a wave (all active), in every lane: within
// each row of 16 lanes by DPP moves (swap neighbours, swap pairs, mirror
// each half row, mirror the row; after each step a lane holds the maximum
// of twice as many lanes), then over the four rows by reading one lane of
// each into scalar registers.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp_u64<0xB1>(v));    // quad_perm [1, 0, 3, 2]
  v = umax64(v, dpp_u64<0x4E>(v));    // quad_perm [2, 3, 0, 1]
  v = umax64(v, dpp_u64<0x141>(v));   // row_half_mirror
  v = umax64(v, dpp_u64<0x140>(v));   // row_mirror
  uint64_t r = 0;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * row);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * row);
    r = umax64(r, ((uint64_t)hi << 32) | lo);
  }
  return r;
}

// PK: lane l holds the four consecutive experts 4 l .. 4 l + 3 (E <= 256,
// E a multiple of 4), so one 16-byte load reads a slice of all four logits.
template <int NPL, bool PK>
__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ part, int ksn,
                                                          const float *__restrict__ bias,
                                                          int32_t *__restrict__ topk_idx,
                                                          float *__restrict__ topk_w, int T, int E,
                                                          int k, float rho, int route_norm) {
  static_assert(!PK || NPL == 4, "packed lanes hold four experts");
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  auto expert = [&](int i) MOE_INLINE { return PK ? 4 * lane + i : lane + 64 * i; };
  // z = bias + the K slices in order (fp64).  The slices are read KU at a
  // time before any is added (all 16 at once for up to four logits per
  // lane); lanes past E read the last expert(s) and drop them.
  constexpr int KU = NPL <= 4 ? 16 : 8;
  const size_t stride = (size_t)T * E;
  double zd[NPL];
  float bv[NPL];
  if (bias) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) bv[i] = bias[min(expert(i), E - 1)];
  } else {
#pragma unroll
    for (int i = 0; i < NPL; ++i) bv[i] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) zd[i] = (double)bv[i];
  const float *prow = part + (size_t)t * E;
  for (int ks0 = 0; ks0 < ksn; ks0 += KU) {
    float a[NPL][KU];
    if constexpr (PK) {
      const float *pe = prow + min(4 * lane, E - 4);
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const f32x4 v = *(const f32x4 *)(pe + (size_t)min(ks0 + u, ksn - 1) * stride);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i][u] = v[i];
      }
      // every load goes out before the first add waits for one
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const float *pe = prow + min(expert(i), E - 1);
#pragma unroll
        for (int u = 0; u < KU; ++u) a[i][u] = pe[(size_t)min(ks0 + u, ksn - 1) * stride];
      }
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i)
#pragma unroll
      for (int u = 0; u < KU; ++u)
        if (ks0 + u < ksn) zd[i] += (double)a[i][u];
  }
  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = expert(i);
    key[i] = 0;
    if (e < E) {
      const float s = (float)(1.0 / (1.0 + exp(-(double)(float)zd[i])));
      const uint32_t hi = s == s ? __float_as_uint(s) : 0u;
      key[i] = ((uint64_t)hi << 32) | (0xFFFFFFFFu - (uint32_t)e);
    }
  }
  float sel_s = 0.0f;      // lane j < k keeps the j-th selection
  int sel_e = 0;
  double den = 0.0;        // the selected scores in slot order
  for (int j = 0; j < k; ++j) {
    uint64_t b = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) b = umax64(b, key[i]);
    const uint64_t w = wave_max_u64(b);
    const float ws = __uint_as_float((uint32_t)(w >> 32));
    // keys are distinct: only the owner's slot matches
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (key[i] == w) key[i] = 0;
    if (lane == j) {
      sel_s = ws;
      sel_e = (int)(0xFFFFFFFFu - (uint32_t)w);
    }
    den += (double)ws;
  }
  if (lane < k) {
    float wv = route_norm ? (float)((double)rho * (double)sel_s / den) : (float)((double)rho * sel_s);
    topk_idx[(size_t)t * k + lane] = sel_e;
    topk_w[(size_t)t * k + lane] = wv;
  }
}

// Partial-sum slices of the logits: a power of two of them, at most 16 (the
// top-k pass adds them), dividing the K blocks evenly.  fp32 activations:
// enough 32-element-block slices for about 256 workgroups, so a small batch
// does not walk K block by block in a few workgroups.  bf16: enough slices
// of whole 64-element stages for about a thousand workgroups.
struct RoutePlan {
  int ebw, mbt, ksn, nsl, eb, tt;
};

static RoutePlan router_plan(int T, int H, int E, int x_is_bf16) {
  RoutePlan p{};
  p.eb = (E + 15) / 16;
  if (!x_is_bf16) {
    p.tt = T <= 256 ? 16 : 64;
    const int tiles = ((T + p.tt - 1) / p.tt) * ((E + 63) / 64);
    const int nkb = H / 32;
    int ksn = 1;
    while (tiles * ksn < 256 && ksn < 16 && nkb % (ksn * 2) == 0) ksn *= 2;
    p.ksn = ksn;
    p.nsl = nkb / ksn;
    return p;
  }
  // 64-token tiles, one expert block per wave: few registers, many waves
  p.mbt = 4;
  p.ebw = 1;
  const int tiles = ((T + 16 * p.mbt - 1) / (16 * p.mbt)) * ((p.eb + 4 * p.ebw - 1) / (4 * p.ebw));
  const int nst = H / 64;
  // about a thousand workgroups, but at most 16 slices for the top-k pass to add
  int ksn = 1;
  while (tiles * ksn < 1024 && ksn < 16 && ksn * 2 <= nst && nst % (ksn * 2) == 0) ksn *= 2;
  p.ksn = ksn;
  p.nsl = nst / ksn;
  return p;
}

size_t route_ws_bytes(int T, int H, int E, int x_is_bf16) {
  const RoutePlan p = router_plan(T, H, E, x_is_bf16);
  size_t bytes = (size_t)p.ksn * T * E * sizeof(float);
  if (x_is_bf16) {
    bytes = (bytes + 255) & ~(size_t)255;
    bytes += (size_t)3 * p.eb * H * 32;   // split weights: 3 terms x 16 rows x 2 bytes per element
  }
  return bytes;
}

hipError_t launch_route(const void *x, int x_is_bf16, const float *Wr, const float *bias,
                        float *part, int32_t *topk_idx, float *topk_w, int T, int H, int E, int k,
                        float rho, int route_norm, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  dim3 blk(256);
  const RoutePlan p = router_plan(T, H, E, x_is_bf16);
  const int ksn = p.ksn;
  if (x_is_bf16) {
    const bool fused = T <= kRouterFusedSplitT;
    const size_t pbytes = (((size_t)ksn * T * E * sizeof(float)) + 255) & ~(size_t)255;
    uint4 *wsplit = (uint4 *)((char *)part + pbytes);
    if (!fused) {
      const long long nthr = (long long)p.eb * (H / 64) * 128;
      router_split_kernel<<<(unsigned)((nthr + 255) / 256), blk, 0, stream>>>(Wr, E, H, p.eb,
                                                                               wsplit);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    const int n_et = (p.eb + 3) / 4, n_tt = (T + 16 * p.mbt - 1) / (16 * p.mbt);
    const int per_xcd = (n_et * n_tt * ksn + 7) / 8;
#define MOE_RGEMM(FS, NSH)                                                                  \
  router_gemm_kernel<4, 2, FS, NSH><<<per_xcd * 8, blk, 0, stream>>>(                       \
      (const uint16_t *)x, wsplit, Wr, part, T, H, E, p.eb, p.nsl, n_et, n_tt, ksn)
    if (p.nsl <= kRouterShortStages) {
      if (fused) MOE_RGEMM(true, kRouterShortStages);
      else MOE_RGEMM(false, kRouterShortStages);
    } else {
      if (fused) MOE_RGEMM(true, 0);
      else MOE_RGEMM(false, 0);
    }
#undef MOE_RGEMM
  } else {
    dim3 grid((T + p.tt - 1) / p.tt, (E + 63) / 64, ksn);
    if (p.tt == 16)
      router_logits_kernel<float, 16><<<grid, blk, 0, stream>>>((const float *)x, Wr, part, T, H, E,
                                                                p.nsl);
    else
      router_logits_kernel<float, 64><<<grid, blk, 0, stream>>>((const float *)x, Wr, part, T, H, E,
                                                                p.nsl);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 g2((T + 3) / 4);
  int npl = (E + 63) / 64;
#define MOE_TOPK(N, PK)                                                                        \
  router_topk_kernel<N, PK><<<g2, blk, 0, stream>>>(part, ksn, bias, topk_idx, topk_w, T, E, k, rho, \
                                                    route_norm)
  if (E <= 256 && E % 4 == 0) MOE_TOPK(4, true);
  else if (npl <= 1) MOE_TOPK(1, false);
  else if (npl <= 2) MOE_TOPK(2, false);
  else if (npl <= 4) MOE_TOPK(4, false);
  else if (npl <= 8) MOE_TOPK(8, false);
  else MOE_TOPK(16, false);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
