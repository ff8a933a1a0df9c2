// gemm_common.hpp -- device pieces shared by the grouped GEMM kernels:
// the epilogues (SwiGLU, MX / static-FP8 quantising, plain), the row ->
// token gather, and the device-side m-tile map over the expert segments.
#pragma once
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// ----------------------------------------------------------------------------- epilogue
// Two adjacent 16-column blocks of bf16 output, a (block blk) and b (block
// blk + 1), four values each per lane: lane (r, g) = (lane % 16, lane / 16)
// holds columns 4 g .. 4 g + 3 of row r in both.  One 16-lane row swap
// (odd lane rows of the first operand with even lane rows of the second)
// leaves lane g = 0, 2 with a's columns 4 g .. 4 g + 7 and lane g = 1, 3
// with b's columns 4 (g - 1) .. 4 g + 3, so every lane stores 16 bytes and
// one store writes 64 contiguous bytes of each of 16 rows (instead of 32
// bytes from 8-byte stores, which measured slower).  All lanes must be
// active; only lanes with `valid` store.
__device__ __forceinline__ void store_pair_bf16(const float (&a)[4], const float (&b)[4], int blk,
                                                long long row, bool valid, const GemmArgs &g,
                                                int lane, void *out) {
  const uint32_t x0 = (uint32_t)f32_to_bf16_rne(a[0]) | ((uint32_t)f32_to_bf16_rne(a[1]) << 16);
  const uint32_t x1 = (uint32_t)f32_to_bf16_rne(a[2]) | ((uint32_t)f32_to_bf16_rne(a[3]) << 16);
  const uint32_t y0 = (uint32_t)f32_to_bf16_rne(b[0]) | ((uint32_t)f32_to_bf16_rne(b[1]) << 16);
  const uint32_t y1 = (uint32_t)f32_to_bf16_rne(b[2]) | ((uint32_t)f32_to_bf16_rne(b[3]) << 16);
  const auto s0 = __builtin_amdgcn_permlane16_swap(x0, y0, false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(x1, y1, false, false);
  if (valid) {
    const int gq = lane >> 4;
    const long long col = (long long)(blk + (gq & 1)) * 16 + 4 * (gq & 2);
    *(uint4 *)((uint16_t *)out + row * g.n_out + col) = uint4{s0[0], s1[0], s0[1], s1[1]};
  }
}

// acc[n] (n < NB) is one 16-token column of NB consecutive 16-row weight
// blocks starting at global block nb0.  Lane: token row `row` of out (stores
// only if `valid`), features 4 * (lane / 16) + r of each block.  Static per-tensor
// FP8 (F == FMT_FP8) first multiplies the gate (and plain) sums by fa and the
// up sums by fb: the product of the expert's weight scale and the
// activation scale.
template <int F, int EPI, int OT, int NB>
__device__ __forceinline__ void epilogue(f32x4 (&acc)[NB], int nb0, long long row, bool valid,
                                         const GemmArgs &g, int lane, float fa, float fb,
                                         void *out) {
  const int c4 = 4 * (lane >> 4);
  if constexpr (F == FMT_FP8) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
      acc[n] *= (EPI == EPI_SWIGLU && (n & 1)) ? fb : fa;
  }
  if constexpr (EPI == EPI_SWIGLU && OT == FMT_FP8) {
    // h codes E4M3(fp32(h / s_h)), four per lane and block pair
    const float sh = g.out_tscale;
#pragma unroll
    for (int q = 0; q < NB / 2; ++q) {
      uint32_t c = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) c |= e4m3_rne((silu(acc[2 * q][r]) * acc[2 * q + 1][r]) / sh) << (8 * r);
      if (valid) {
        const long long col = (long long)(nb0 / 2 + q) * 16 + c4;
        *(uint32_t *)((uint8_t *)out + row * g.n_out + col) = c;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // gate block 2q and up block 2q+1 make h columns (nb0/2 + q)*16 + [0,16)
    if constexpr (OT == FMT_MX8) {
      static_assert(NB % 4 == 0, "MX epilogue needs whole 32-column blocks");
#pragma unroll
      for (int u = 0; u < NB / 4; ++u) {
        float v0[4], v1[4];
        float am = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v0[r] = silu(acc[4 * u][r]) * acc[4 * u + 1][r];
          v1[r] = silu(acc[4 * u + 2][r]) * acc[4 * u + 3][r];
          am = fmaxf(am, fmaxf(fabsf(v0[r]), fabsf(v1[r])));
        }
        // the 32 columns of this MX block sit in lanes with the same token
        am = wave_max_xor(am, 16);
        am = wave_max_xor(am, 32);
        const uint32_t sb = mx_scale_byte(am);
        const float inv = mx_inv_scale(sb);
        uint32_t c0 = 0, c1 = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          c0 |= e4m3_rne(v0[r] * inv) << (8 * r);
          c1 |= e4m3_rne(v1[r] * inv) << (8 * r);
        }
        if (valid) {
          const int hb = nb0 / 2 + 2 * u;          // first h block (16 columns)
          uint8_t *o = (uint8_t *)out + row * g.n_out + hb * 16 + c4;
          *(uint32_t *)o = c0;
          *(uint32_t *)(o + 16) = c1;
          if (lane < 16) g.out_scale[row * (g.n_out / 32) + hb / 2] = (uint8_t)sb;
        }
      }
    } else if constexpr (OT == FMT_BF16 && NB % 4 == 0) {
      // h blocks nb0/2 + q and nb0/2 + q + 1 stored together
#pragma unroll
      for (int q = 0; q < NB / 2; q += 2) {
        float v0[4], v1[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v0[r] = silu(acc[2 * q][r]) * acc[2 * q + 1][r];
          v1[r] = silu(acc[2 * q + 2][r]) * acc[2 * q + 3][r];
        }
        store_pair_bf16(v0, v1, nb0 / 2 + q, row, valid, g, lane, out);
      }
    } else {
#pragma unroll
      for (int q = 0; q < NB / 2; ++q) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = silu(acc[2 * q][r]) * acc[2 * q + 1][r];
        if (!valid) continue;
        const long long col = (long long)(nb0 / 2 + q) * 16 + c4;
        if constexpr (OT == FMT_BF16) {
          uint2 p;
          p.x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
          p.y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
          *(uint2 *)((uint16_t *)out + row * g.n_out + col) = p;
        } else {
          *(float4 *)((float *)out + row * g.n_out + col) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  } else if constexpr (OT == FMT_BF16 && NB % 2 == 0) {
#pragma unroll
    for (int q = 0; q < NB / 2; ++q) {
      float v0[4], v1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v0[r] = acc[2 * q][r];
        v1[r] = acc[2 * q + 1][r];
      }
      store_pair_bf16(v0, v1, nb0 + 2 * q, row, valid, g, lane, out);
    }
  } else {
    if (!valid) return;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const long long col = (long long)(nb0 + n) * 16 + c4;
      if constexpr (OT == FMT_BF16) {
        uint2 p;
        p.x = (uint32_t)f32_to_bf16_rne(acc[n][0]) | ((uint32_t)f32_to_bf16_rne(acc[n][1]) << 16);
        p.y = (uint32_t)f32_to_bf16_rne(acc[n][2]) | ((uint32_t)f32_to_bf16_rne(acc[n][3]) << 16);
        *(uint2 *)((uint16_t *)out + row * g.n_out + col) = p;
      } else {
        *(float4 *)((float *)out + row * g.n_out + col) =
            make_float4(acc[n][0], acc[n][1], acc[n][2], acc[n][3]);
      }
    }
  }
}

// Epilogue factors of expert e under static per-tensor FP8 (1 otherwise).
template <int F, int EPI>
__device__ __forceinline__ void tensor_factors(const GemmArgs &g, int e, float &fa, float &fb) {
  fa = fb = 1.0f;
  if constexpr (F == FMT_FP8) {
    if constexpr (EPI == EPI_SWIGLU) {
      fa = g.w_tscale[2 * e] * g.a_tscale;
      fb = g.w_tscale[2 * e + 1] * g.a_tscale;
    } else {
      fa = fb = g.w_tscale[e] * g.a_tscale;
    }
  }
}

__device__ __forceinline__ long long token_of(const GemmArgs &g, int r) {
  return g.sorted_src ? (long long)(g.sorted_src[r] / g.k_route) : (long long)r;
}

// ----------------------------------------------------------------------------- tile map
// m-tiles are numbered expert by expert (TM rows each, the last one of an
// expert ragged), then those of the extra segment (index E, rows2 rows) if
// there is one.  tile_scan computes, from the segment offsets alone (they
// stay on the device), cum[e] = m-tiles of segments 0..e and returns the
// total; tile_locate below maps a tile index to its segment, rows and n-tile.
// At least 256 threads; cum holds >= 1024 ints (E + 1 <= 1024 with an extra
// segment).
template <int TM>
__device__ int tile_scan(const GemmArgs &g, int *cum) {
  if (!g.offsets) return (g.rows + TM - 1) / TM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int wtot[4];
  int v[4], run = 0;
  if (tid < 256) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ex = tid * 4 + i;
      int c = ex < g.E ? g.offsets[ex + 1] - g.offsets[ex] : (ex == g.E ? g.rows2 : 0);
      if (c <= g.split) c = 0;               // left to the streaming kernel
      run += (c + TM - 1) / TM;
      v[i] = run;
    }
  }
  // inclusive scan of per-thread totals: within the wave, then across the
  // first four waves (threads past 256 contribute nothing)
  int x = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63 && wave < 4) wtot[wave] = x;
  __syncthreads();
  if (tid < 256) {
    int before = x - run;
    for (int w = 0; w < wave; ++w) before += wtot[w];
#pragma unroll
    for (int i = 0; i < 4; ++i) cum[tid * 4 + i] = before + v[i];
  }
  __syncthreads();
  return cum[g.E - 1 + (g.rows2 > 0 ? 1 : 0)];
}

// Tile order inside one expert: its m-tiles are taken in groups of GM; a
// group's tiles run n-tile by n-tile, and within an n-tile over the group's
// m-tiles.  The m-tiles that read the same weight tile are therefore
// neighbours in dispatch order (they start within moments of each other
// and walk K in step, so the weights come from HBM once and from L2 for the
// others), and the n-tiles that share a token tile are at most GM apart.
// Tile t -> segment e (E: the extra segment, whose rows count from 0), rows
// [row0, row_end) of it (row0 is the first row of the m-tile), n-tile nt.
template <int TM, int GM>
__device__ void tile_locate(const GemmArgs &g, const int *cum, int ntn, int t, int &e, int &row0,
                            int &row_end, int &nt) {
  int first, mte, seg0, seg1;
  if (!g.offsets) {
    e = 0;
    first = 0;
    mte = (g.rows + TM - 1) / TM;
    seg0 = 0;
    seg1 = g.rows;
  } else {
    int lo = 0, hi = g.E - 1 + (g.rows2 > 0 ? 1 : 0);
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if (cum[mid] * ntn > t) hi = mid;
      else lo = mid + 1;
    }
    e = lo;
    first = lo ? cum[lo - 1] : 0;
    mte = cum[lo] - first;
    if (lo < g.E) {
      seg0 = g.offsets[lo];
      seg1 = g.offsets[lo + 1];
    } else {
      seg0 = 0;
      seg1 = g.rows2;
    }
  }
  const int local = t - first * ntn;
  const int grp = local / (GM * ntn), in = local - grp * (GM * ntn);
  const int gsz = min(GM, mte - grp * GM);
  nt = in / gsz;
  row0 = seg0 + (grp * GM + in % gsz) * TM;
  row_end = seg1;
}

}  // namespace moe
