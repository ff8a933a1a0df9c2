// gemm.hip -- grouped expert GEMM with fused SwiGLU / plain epilogues.
//
// The grouped GMM of the Hy3 on CANN NPU guide (sections 8.1 and 8.5) and the
// FusedMoEGMM(num_experts, hidden_size, intermediate_size) module of the
// HunyuanImage-3.0 multi-stream article (source walkthrough part 1): one
// GEMM per expert over the variable-length run of rows InitRouting gave it.
// Expert FFN: y = W_d ( silu(W_g x) * (W_u x) ), a SwiGLU reading of the
// pages' expert FFN (they give its sizes only).
//
// Two kernels, chosen per launch from the expected rows per expert:
//  * gemm_skinny -- few rows per expert (decode).  Weight-streaming: each wave
//    owns NW 16-row weight blocks of one expert over the whole K axis and
//    reads them straight from HBM into registers (1 KiB contiguous per wave
//    access); the expert's <= 16*MB token rows are read per chunk (they stay
//    in L2).  No LDS, no barriers.  Untouched experts exit at once.
//  * gemm_tile -- many rows per expert (prefill).  Workgroup tile of TN
//    weight rows x TM token rows, K staged through LDS half a chunk at a time
//    (double-buffered, one barrier per stage), register prefetch of the next
//    stage.  The m-tile -> (expert, rows) map is computed on the device from
//    the segment offsets, so no host synchronisation is needed; the grid is
//    sized from an upper bound and surplus workgroups exit.
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// ----------------------------------------------------------------------------- epilogue
// acc[n] (n < NB) is one 16-token column of NB consecutive 16-row weight
// blocks starting at global block nb0.  Lane: token row `row` (stores only if
// `valid`), features 4 * (lane / 16) + r of each block.
template <int EPI, int OT, int NB>
__device__ __forceinline__ void epilogue(const f32x4 (&acc)[NB], int nb0, long long row, bool valid,
                                         const GemmArgs &g, int lane) {
  const int c4 = 4 * (lane >> 4);
  if constexpr (EPI == EPI_SWIGLU) {
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
          uint8_t *o = (uint8_t *)g.out + row * g.n_out + hb * 16 + c4;
          *(uint32_t *)o = c0;
          *(uint32_t *)(o + 16) = c1;
          if (lane < 16) g.out_scale[row * (g.n_out / 32) + hb / 2] = (uint8_t)sb;
        }
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
          *(uint2 *)((uint16_t *)g.out + row * g.n_out + col) = p;
        } else {
          *(float4 *)((float *)g.out + row * g.n_out + col) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
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
        *(uint2 *)((uint16_t *)g.out + row * g.n_out + col) = p;
      } else {
        *(float4 *)((float *)g.out + row * g.n_out + col) =
            make_float4(acc[n][0], acc[n][1], acc[n][2], acc[n][3]);
      }
    }
  }
}

__device__ __forceinline__ long long token_of(const GemmArgs &g, int r) {
  return g.sorted_src ? (long long)(g.sorted_src[r] / g.k_route) : (long long)r;
}

// ----------------------------------------------------------------------------- skinny
// Grid: E * (N/16 / (4*NW)) workgroups of 4 waves.  Workgroup (e, group)
// covers 4*NW consecutive weight blocks; wave w takes NW of them.

template <int F, int EPI, int OT, int NW, int MB>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nbtot = g.N >> 4;
  const int ngroups = nbtot / (4 * NW);
  const int e = blockIdx.x / ngroups, grp = blockIdx.x % ngroups;
  int s0, s1;
  if (g.offsets) { s0 = g.offsets[e]; s1 = g.offsets[e + 1]; }
  else { s0 = 0; s1 = g.rows; }
  if (s1 <= s0) return;
  const int nb0 = (grp * 4 + wave) * NW;
  const int kcn = g.K / FmtInfo<F>::chunk_elems;     // chunks along K
  const int grp_l = lane >> 4;
  const uint8_t *wb = g.w + (size_t)e * g.w_expert_stride + (size_t)nb0 * kcn * kBlockBytes +
                      lane * 16;
  const uint16_t *wsb = nullptr;
  if constexpr (F == FMT_MX8)
    wsb = g.w_scale + (size_t)e * g.ws_expert_stride + (size_t)nb0 * kcn * 64 + lane;

  for (int mbase = s0; mbase < s1; mbase += 16 * MB) {
    const uint8_t *tp[MB];
    const uint8_t *tsp[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      int r = mbase + 16 * i + (lane & 15);
      int rr = r < s1 ? r : s1 - 1;
      long long tok = token_of(g, rr);
      tp[i] = g.a + tok * g.a_row_bytes + 16 * grp_l;
      if constexpr (F == FMT_MX8) tsp[i] = g.a_scale + tok * (g.K / 32) + grp_l;
    }
    f32x4 acc[NW][MB];
#pragma unroll
    for (int n = 0; n < NW; ++n)
#pragma unroll
      for (int i = 0; i < MB; ++i) acc[n][i] = f32x4{0.f, 0.f, 0.f, 0.f};


    for (int kc = 0; kc < kcn; ++kc) {
      i32x4 wf[NW][4], tf[MB][4];
      uint32_t wsc[NW], tsc[MB];
#pragma unroll
      for (int n = 0; n < NW; ++n)
#pragma unroll
        for (int p = 0; p < 4; ++p)
          wf[n][p] = __builtin_nontemporal_load(
              (const i32x4 *)(wb + ((size_t)n * kcn + kc) * kBlockBytes + p * 1024));
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int p = 0; p < 4; ++p) tf[i][p] = *(const i32x4 *)(tp[i] + kc * 256 + chunk_off(0, p));
      if constexpr (F == FMT_MX8) {
#pragma unroll
        for (int n = 0; n < NW; ++n) wsc[n] = wsb[((size_t)n * kcn + kc) * 64];
#pragma unroll
        for (int i = 0; i < MB; ++i) tsc[i] = tsp[i][8 * kc] | ((uint32_t)tsp[i][8 * kc + 4] << 8);
      } else {
#pragma unroll
        for (int n = 0; n < NW; ++n) wsc[n] = 0;
#pragma unroll
        for (int i = 0; i < MB; ++i) tsc[i] = 0;
      }
#pragma unroll
      for (int n = 0; n < NW; ++n)
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          mfma_half<F>(acc[n][i], wf[n][0], wf[n][1], tf[i][0], tf[i][1], wsc[n] & 0xFF,
                       tsc[i] & 0xFF);
          mfma_half<F>(acc[n][i], wf[n][2], wf[n][3], tf[i][2], tf[i][3], wsc[n] >> 8,
                       tsc[i] >> 8);
        }
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      f32x4 col[NW];
#pragma unroll
      for (int n = 0; n < NW; ++n) col[n] = acc[n][i];
      const int r = mbase + 16 * i + (lane & 15);
      epilogue<EPI, OT, NW>(col, nb0, r, r < s1, g, lane);
    }
  }
}

// ----------------------------------------------------------------------------- tile map
// Locate m-tile `mt`: expert e and its rows [row0, row_end).  Uses the
// segment offsets only (device-resident), 256 threads, scratch >= 1024 ints.
template <int TM>
__device__ bool find_tile(const GemmArgs &g, int mt, int *cum, int &e, int &row0, int &row_end) {
  if (!g.offsets) {
    if (mt >= (g.rows + TM - 1) / TM) return false;
    e = 0;
    row0 = mt * TM;
    row_end = g.rows;
    return true;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ int wtot[4];
  int v[4], run = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ex = tid * 4 + i;
    const int c = ex < g.E ? g.offsets[ex + 1] - g.offsets[ex] : 0;
    run += (c + TM - 1) / TM;
    v[i] = run;
  }
  // inclusive scan of per-thread totals: within the wave, then across waves
  int x = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  int before = x - run;
  for (int w = 0; w < wave; ++w) before += wtot[w];
#pragma unroll
  for (int i = 0; i < 4; ++i) cum[tid * 4 + i] = before + v[i];
  __syncthreads();
  const int total = cum[g.E - 1];
  if (mt >= total) return false;
  int lo = 0, hi = g.E - 1;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (cum[mid] > mt) hi = mid;
    else lo = mid + 1;
  }
  e = lo;
  const int first = lo ? cum[lo - 1] : 0;
  row0 = g.offsets[lo] + (mt - first) * TM;
  row_end = g.offsets[lo + 1];
  return true;
}

// ----------------------------------------------------------------------------- tile
// Workgroup tile: TN weight rows (NBT blocks) x TM tokens (MBT blocks); waves
// arranged WN x WM, each owning NBW x MBW accumulator blocks.  Stages are
// half-chunks: per stage the weight tile is NBT contiguous 2 KiB pieces and
// the token tile is one 128-byte line of each of TM rows.

template <int F, int EPI, int OT, int TN, int TM, int WN, int WM>
__global__ __launch_bounds__(256, 1) void gemm_tile_kernel(GemmArgs g) {
  constexpr int NBT = TN / 16, MBT = TM / 16;
  constexpr int NBW = NBT / WN, MBW = MBT / WM;
  constexpr int WBYTES = NBT * 2048, TBYTES = MBT * 2048;
  constexpr int STAGE = WBYTES + TBYTES;
  constexpr int WLD = NBT / 2;          // 16-byte weight loads per thread per stage
  constexpr int TLD = TM / 32;          // 16-byte token loads per thread per stage
  static_assert(WN * WM == 4, "4 waves");
  static_assert(WLD >= 1 && TLD >= 1, "tile too small");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int cum[1024];
  __shared__ uint8_t wscl[2][NBT * 64];
  __shared__ uint8_t tscl[2][MBT * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wm = wave / WN;
  const int logical = xcd_swizzle(blockIdx.x, gridDim.x);
  const int nt = logical / g.mt_upper, mt = logical % g.mt_upper;
  if (nt >= g.N / TN) return;
  int e, row0, row_end;
  if (!find_tile<TM>(g, mt, cum, e, row0, row_end)) return;

  const int kcn = g.K / FmtInfo<F>::chunk_elems;
  const int nstage = 2 * kcn;
  const uint8_t *wsrc = g.w + (size_t)e * g.w_expert_stride + (size_t)(nt * NBT) * kcn * kBlockBytes;

  // this thread's token rows (fixed across stages)
  const uint8_t *tsrc[TLD];
  int tdst[TLD];
#pragma unroll
  for (int i = 0; i < TLD; ++i) {
    const int idx = tid + 256 * i;
    const int rl = idx >> 3, seg = idx & 7;
    int r = row0 + rl;
    if (r >= row_end) r = row_end - 1;
    tsrc[i] = g.a + token_of(g, r) * g.a_row_bytes + seg * 16;
    tdst[i] = WBYTES + (rl >> 4) * 2048 + (seg >> 2) * 1024 + ((rl & 15) + 16 * (seg & 3)) * 16;
  }
  // MX scales: per stage NBT*64 weight-lane bytes and MBT*64 token-lane bytes,
  // spread over the 256 threads (entry idx = tid + 256 i: block idx / 64,
  // lane idx % 64).
  constexpr int WSL = (F == FMT_MX8) ? NBT * 64 / 256 : 1;
  constexpr int TSL = (F == FMT_MX8) ? MBT * 64 / 256 : 1;
  static_assert(F != FMT_MX8 || (NBT % 4 == 0 && MBT % 4 == 0), "scale staging");
  const uint8_t *tss[TSL];
  if constexpr (F == FMT_MX8) {
#pragma unroll
    for (int i = 0; i < TSL; ++i) {
      const int idx = tid + 256 * i;
      const int rl = (idx >> 6) * 16 + (idx & 15);
      int r = row0 + rl;
      if (r >= row_end) r = row_end - 1;
      tss[i] = g.a_scale + token_of(g, r) * (g.K / 32) + ((idx >> 4) & 3);
    }
  }

  i32x4 wreg[WLD], treg[TLD];
  uint32_t wsreg[WSL], tsreg[TSL];
  auto load_stage = [&](int s) {
    const int kc = s >> 1, h = s & 1;
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const int idx = tid + 256 * i;
      const int blk = idx >> 7, within = idx & 127;
      wreg[i] = *(const i32x4 *)(wsrc + ((size_t)blk * kcn + kc) * kBlockBytes + h * 2048 +
                                 within * 16);
    }
#pragma unroll
    for (int i = 0; i < TLD; ++i) treg[i] = *(const i32x4 *)(tsrc[i] + kc * 256 + h * 128);
    if constexpr (F == FMT_MX8) {
#pragma unroll
      for (int i = 0; i < WSL; ++i) {
        const int idx = tid + 256 * i;
        const uint32_t v = g.w_scale[(size_t)e * g.ws_expert_stride +
                                     ((size_t)(nt * NBT + (idx >> 6)) * kcn + kc) * 64 + (idx & 63)];
        wsreg[i] = (v >> (8 * h)) & 0xFFu;
      }
#pragma unroll
      for (int i = 0; i < TSL; ++i) tsreg[i] = tss[i][8 * kc + 4 * h];
    }
  };
  auto store_stage = [&](int s) {
    uint8_t *base = lds + (s & 1) * STAGE;
#pragma unroll
    for (int i = 0; i < WLD; ++i) *(i32x4 *)(base + (tid + 256 * i) * 16) = wreg[i];
#pragma unroll
    for (int i = 0; i < TLD; ++i) *(i32x4 *)(base + tdst[i]) = treg[i];
    if constexpr (F == FMT_MX8) {
#pragma unroll
      for (int i = 0; i < WSL; ++i) wscl[s & 1][tid + 256 * i] = (uint8_t)wsreg[i];
#pragma unroll
      for (int i = 0; i < TSL; ++i) tscl[s & 1][tid + 256 * i] = (uint8_t)tsreg[i];
    }
  };

  f32x4 acc[NBW][MBW];
#pragma unroll
  for (int n = 0; n < NBW; ++n)
#pragma unroll
    for (int m = 0; m < MBW; ++m) acc[n][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_stage(0);
  store_stage(0);
  if (nstage > 1) load_stage(1);
  __syncthreads();

  for (int s = 0; s < nstage; ++s) {
    const uint8_t *base = lds + (s & 1) * STAGE;
    i32x4 wf[NBW][2], tf[MBW][2];
    uint32_t wsc[NBW], tsc[MBW];
#pragma unroll
    for (int n = 0; n < NBW; ++n) {
      const uint8_t *p = base + (wn * NBW + n) * 2048 + lane * 16;
      wf[n][0] = *(const i32x4 *)p;
      wf[n][1] = *(const i32x4 *)(p + 1024);
      wsc[n] = 0;
      if constexpr (F == FMT_MX8) wsc[n] = wscl[s & 1][(wn * NBW + n) * 64 + lane];
    }
#pragma unroll
    for (int m = 0; m < MBW; ++m) {
      const uint8_t *p = base + WBYTES + (wm * MBW + m) * 2048 + lane * 16;
      tf[m][0] = *(const i32x4 *)p;
      tf[m][1] = *(const i32x4 *)(p + 1024);
      tsc[m] = 0;
      if constexpr (F == FMT_MX8) tsc[m] = tscl[s & 1][(wm * MBW + m) * 64 + lane];
    }
#pragma unroll
    for (int n = 0; n < NBW; ++n)
#pragma unroll
      for (int m = 0; m < MBW; ++m)
        mfma_half<F>(acc[n][m], wf[n][0], wf[n][1], tf[m][0], tf[m][1], wsc[n], tsc[m]);
    if (s + 1 < nstage) store_stage(s + 1);
    if (s + 2 < nstage) load_stage(s + 2);
    __syncthreads();
  }

  const int nb0 = nt * NBT + wn * NBW;
#pragma unroll
  for (int m = 0; m < MBW; ++m) {
    f32x4 col[NBW];
#pragma unroll
    for (int n = 0; n < NBW; ++n) col[n] = acc[n][m];
    const int r = row0 + (wm * MBW + m) * 16 + (lane & 15);
    epilogue<EPI, OT, NBW>(col, nb0, r, r < row_end, g, lane);
  }
}

// ----------------------------------------------------------------------------- dispatch

template <int F, int EPI, int OT>
static hipError_t run_gemm(const GemmArgs &g0, int total_rows, hipStream_t stream) {
  GemmArgs g = g0;
  const int segs = g.offsets ? g.E : 1;
  const int nbtot = g.N / 16;
  // rows per segment: the mean for expert segments, all rows for one segment
  const int per = g.offsets ? (total_rows + segs - 1) / segs : total_rows;
  if (per <= 64 && nbtot % 16 == 0) {
    // weight-streaming kernel, 4 weight blocks per wave, MB token blocks
    const int grid = segs * (nbtot / 16);
    if (per <= 16)
      gemm_skinny_kernel<F, EPI, OT, 4, 1><<<grid, 256, 0, stream>>>(g);
    else if (per <= 32)
      gemm_skinny_kernel<F, EPI, OT, 4, 2><<<grid, 256, 0, stream>>>(g);
    else
      gemm_skinny_kernel<F, EPI, OT, 4, 4><<<grid, 256, 0, stream>>>(g);
    return hipGetLastError();
  }
  constexpr int TN = 256, TM = 128;
  if (g.N % TN != 0) return hipErrorInvalidValue;
  const int mtiles = g.offsets ? (total_rows + TM - 1) / TM + g.E : (g.rows + TM - 1) / TM;
  g.mt_upper = mtiles;
  long long nblocks = (long long)mtiles * (g.N / TN);
  nblocks = (nblocks + 7) & ~7LL;
  const size_t lds = 2 * (size_t)(TN / 16 + TM / 16) * 2048;
  auto kern = gemm_tile_kernel<F, EPI, OT, TN, TM, 2, 2>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void *)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  kern<<<(unsigned)nblocks, 256, lds, stream>>>(g);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmArgs &g, int fmt, int epi, int out_fmt, int total_rows,
                               hipStream_t stream) {
  if (total_rows <= 0) return hipSuccess;
  if (fmt == FMT_BF16) {
    if (epi == EPI_SWIGLU) return run_gemm<FMT_BF16, EPI_SWIGLU, FMT_BF16>(g, total_rows, stream);
    return run_gemm<FMT_BF16, EPI_PLAIN, FMT_BF16>(g, total_rows, stream);
  }
  if (fmt == FMT_F32) {
    if (epi == EPI_SWIGLU) return run_gemm<FMT_F32, EPI_SWIGLU, FMT_F32>(g, total_rows, stream);
    return run_gemm<FMT_F32, EPI_PLAIN, FMT_F32>(g, total_rows, stream);
  }
  if (fmt == FMT_MX8) {
    if (epi == EPI_SWIGLU) return run_gemm<FMT_MX8, EPI_SWIGLU, FMT_MX8>(g, total_rows, stream);
    if (out_fmt == FMT_BF16) return run_gemm<FMT_MX8, EPI_PLAIN, FMT_BF16>(g, total_rows, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
