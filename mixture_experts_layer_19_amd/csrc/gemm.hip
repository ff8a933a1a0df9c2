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
//    owns NW 16-row weight blocks of one expert and reads them straight from
//    HBM into registers with non-temporal loads (1 KiB contiguous per wave
//    access), over the whole K axis or, with KSW = 4, over a quarter of it
//    (the four waves' partial sums then added in LDS in wave order); the
//    expert's <= 16*MB token rows are read per chunk (they stay in L2).
//    Untouched experts exit at once.
//  * gemm_tile -- many rows per expert (prefill).  Workgroup tile of TN
//    weight rows x TM token rows, K staged through LDS half a chunk at a time
//    (double-buffered, one barrier per stage), register prefetch of the next
//    stage.  The m-tile -> (expert, rows) map is computed on the device from
//    the segment offsets, so no host synchronisation is needed; the grid is
//    sized from an upper bound and surplus workgroups exit.  For f32 / bf16
//    it can take one more segment after the experts (the shared expert, with
//    its own weights, rows and output).
// Dispatch (run_gemm): batches of at most 64 tokens use gemm_skinny alone;
// larger ones with at most 32 rows per expert on average send the experts of
// up to 32 rows to gemm_skinny and the rest to gemm_tile; beyond that
// gemm_tile takes every expert.
//
// Both kernels take the weight format as a template parameter: fp32, bf16,
// MX-fp8, E2M1 weights against MX-fp8 tokens (W4A8), or E4M3 with static
// per-tensor scales, which the epilogue applies.
#include "gemm_common.hpp"

namespace moe {

// Decode streaming kernel: weight blocks per wave, and the dynamic LDS
// reserved per workgroup (the kernel uses none), which caps its residency.
// Fewer concurrent weight streams read HBM faster than a full CU, and leave
// slots for the shared expert's workgroups on the side stream.  Measured at
// T = 64 (Hy3 shape):
//  * bf16 and fp32: 2 blocks per wave at 5 workgroups per CU (30000 bytes);
//    4 blocks at 3 workgroups per CU measured 1.097 ms for the layer against
//    1.085, and 2 blocks at 3, 4 or 6 workgroups per CU 1.10-1.11 ms;
//  * 8-bit weights (static FP8, MX-fp8): 4 blocks at 3 workgroups per CU
//    (45000 bytes); the bf16 setting slows the FP8 gate/up 0.351 -> 0.372 ms;
//  * E2M1 weights: 8 blocks per wave for the gate/up GEMM, whose blocks are
//    half as large (0.212 -> 0.205 ms against 4), 2 for the down GEMM, at 5
//    workgroups per CU (layer 0.367 -> 0.363 ms against 4 blocks at 3).
//  * bf16 and fp32 at up to 16 rows per expert: each workgroup's four waves
//    split the K axis of the same 2 blocks (partial sums added in LDS in
//    wave order), 3 workgroups per CU (35000 bytes of padding beside the
//    6 KiB reduction buffer): four times as many, shorter workgroups, so the
//    launch's last round leaves HBM idle for less time (Hy3 decode layer
//    1.041 ms against 1.084 with whole-K waves; 4, 5 or 6 workgroups per
//    CU: 1.044 / 1.048 / 1.075 ms; 4 blocks per workgroup: 1.061).  The same
//    split measured slower for E2M1 (W4A8 decode 0.396 ms against 0.373)
//    and no better for 8-bit weights, which keep whole-K waves.
constexpr int kSkinnyLdsPad = 30000, kSkinnyLdsPad8 = 45000, kSkinnyLdsPadKs = 35000;
constexpr int kSkinnyNW = 2, kSkinnyNW8 = 4, kSkinnyNWMx4 = 8;
// streaming kernel for the short segments of a mixed launch: weight blocks
// per wave, token blocks per pass, and the longest segment it takes (the
// tiled kernel takes the longer ones)
constexpr int kHybNW = 4, kHybMB = 2, kHybSplit = 32;
// The mixed launch is used only when the experts average at most kHybMean
// rows (beyond that the tiled kernel takes every expert: on the skewed Hy4
// batch, 64 rows per expert on average with 88 of 256 experts at 32 rows or
// fewer, 1.98 ms against 2.02 with the mixed launch, 2.04 / 2.05 with the
// split at 24 / 16 rows and 2.52 at 48)
constexpr int kHybMean = 32;
// m-tiles per group in the tiled kernel's tile order
constexpr int kTileGM = 8;
// tiled kernel (f32 / bf16): WN x WM waves of 64 weight rows x MBW token
// blocks, stages of weight prefetch, workgroups per CU
constexpr int kTileWN = 4, kTileWM = 1, kTileMBW = 8, kTileWPF = 1, kTileOcc = 2;
// token rows per tile of the 8- and 4-bit tiled kernel: 96 covers the ~171
// rows an expert gets at 4096 tokens (top-8 of 192) in two m-tiles with 11%
// padding, where 128 pads by 33%; two workgroups per CU
constexpr int kTileTMMx = 96, kTileOccMx = 2;



// ----------------------------------------------------------------------------- skinny
// Grid: segments x groups.  KSW == 1: workgroup (e, group) covers 4*NW
// consecutive weight blocks, wave w takes NW of them over the whole K axis.
// KSW == 4: the four waves share the same NW blocks and take every fourth K
// chunk each; their partial sums meet in LDS and are added in wave order
// (fixed, so results are deterministic).  Load latency is hidden by
// occupancy (few registers per wave, several waves per SIMD) rather than by
// double-buffered registers, which measured slower at decode.

template <int F, int NW, int MB>
struct SkinnyBuf {
  i32x4 w[NW][4], t[MB][4];
  uint32_t ws[NW], ts[MB];
};

template <int F, int EPI, int OT, int NW, int MB, int KSW>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nbtot = g.N >> 4;
  constexpr int BPW = (KSW == 4) ? NW : 4 * NW;       // weight blocks per workgroup
  const int ngroups = nbtot / BPW;
  const int e = blockIdx.x / ngroups, grp = blockIdx.x % ngroups;
  int s0, s1;
  if (g.offsets) { s0 = g.offsets[e]; s1 = g.offsets[e + 1]; }
  else { s0 = 0; s1 = g.rows; }
  if (s1 <= s0 || (g.split > 0 && s1 - s0 > g.split)) return;
  float fa, fb;
  tensor_factors<F, EPI>(g, e, fa, fb);
  const int nb0 = (KSW == 4) ? grp * NW : (grp * 4 + wave) * NW;
  const int kcn = g.K / FmtInfo<F>::chunk_elems;     // chunks along K
  const int k0 = (KSW == 4) ? wave : 0;
  const int grp_l = lane >> 4;
  constexpr int WB = wblock_bytes<F>;
  const uint8_t *wb = g.w + (size_t)e * g.w_expert_stride + (size_t)nb0 * kcn * WB + lane * 16;
  const uint16_t *wsb = nullptr;
  if constexpr (is_mx<F>)
    wsb = g.w_scale + (size_t)e * g.ws_expert_stride + (size_t)nb0 * kcn * 64 + lane;
  __shared__ f32x4 red[KSW == 4 ? 3 : 1][KSW == 4 ? NW * MB : 1][64];

  for (int mbase = s0; mbase < s1; mbase += 16 * MB) {
    // token blocks of this pass that hold rows (uniform): the others are
    // neither loaded nor multiplied
    const int live = min(MB, (s1 - mbase + 15) / 16);
    const uint8_t *tp[MB];
    const uint8_t *tsp[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      int r = mbase + 16 * i + (lane & 15);
      int rr = r < s1 ? r : s1 - 1;
      long long tok = token_of(g, rr);
      tp[i] = g.a + tok * g.a_row_bytes + 16 * grp_l;
      tsp[i] = nullptr;
      if constexpr (is_mx<F>) tsp[i] = g.a_scale + tok * (g.K / 32) + grp_l;
    }
    f32x4 acc[NW][MB];
#pragma unroll
    for (int n = 0; n < NW; ++n)
#pragma unroll
      for (int i = 0; i < MB; ++i) acc[n][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto load = [&](SkinnyBuf<F, NW, MB> &bf, int kc) MOE_INLINE {
      // weight pieces of the chunk: four for 4 KiB blocks, two (one per
      // half) for E2M1's 2 KiB blocks
      constexpr int NP = WB / 1024;
#pragma unroll
      for (int n = 0; n < NW; ++n)
#pragma unroll
        for (int p = 0; p < NP; ++p)
          bf.w[n][p] = __builtin_nontemporal_load(
              (const i32x4 *)(wb + ((size_t)n * kcn + kc) * WB + p * 1024));
#pragma unroll
      for (int i = 0; i < MB; ++i)
        if (i < live)
#pragma unroll
          for (int p = 0; p < 4; ++p) bf.t[i][p] = *(const i32x4 *)(tp[i] + kc * 256 + chunk_off(0, p));
      if constexpr (is_mx<F>) {
#pragma unroll
        for (int n = 0; n < NW; ++n) bf.ws[n] = wsb[((size_t)n * kcn + kc) * 64];
#pragma unroll
        for (int i = 0; i < MB; ++i)
          if (i < live) bf.ts[i] = tsp[i][8 * kc] | ((uint32_t)tsp[i][8 * kc + 4] << 8);
      } else {
#pragma unroll
        for (int n = 0; n < NW; ++n) bf.ws[n] = 0;
#pragma unroll
        for (int i = 0; i < MB; ++i) bf.ts[i] = 0;
      }
    };
    auto compute = [&](const SkinnyBuf<F, NW, MB> &bf) MOE_INLINE {
#pragma unroll
      for (int n = 0; n < NW; ++n)
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          if (i >= live) continue;
          // MX: byte h of the scale pairs is half h's scale
          if constexpr (F == FMT_MX4) {
            // E2M1: piece h is all of half h's weights
            mfma_half<F, 0, 0>(acc[n][i], bf.w[n][0], bf.w[n][0], bf.t[i][0], bf.t[i][1],
                               bf.ws[n], bf.ts[i]);
            mfma_half<F, 1, 1>(acc[n][i], bf.w[n][1], bf.w[n][1], bf.t[i][2], bf.t[i][3],
                               bf.ws[n], bf.ts[i]);
          } else {
            mfma_half<F, 0, 0>(acc[n][i], bf.w[n][0], bf.w[n][1], bf.t[i][0], bf.t[i][1],
                               bf.ws[n], bf.ts[i]);
            mfma_half<F, 1, 1>(acc[n][i], bf.w[n][2], bf.w[n][3], bf.t[i][2], bf.t[i][3],
                               bf.ws[n], bf.ts[i]);
          }
        }
    };

    for (int kc = k0; kc < kcn; kc += KSW) {
      SkinnyBuf<F, NW, MB> b0;
      load(b0, kc);
      compute(b0);
    }

    if constexpr (KSW == 4) {
      if (wave > 0) {
#pragma unroll
        for (int n = 0; n < NW; ++n)
#pragma unroll
          for (int i = 0; i < MB; ++i) red[wave - 1][n * MB + i][lane] = acc[n][i];
      }
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int w = 0; w < 3; ++w)
#pragma unroll
          for (int n = 0; n < NW; ++n)
#pragma unroll
            for (int i = 0; i < MB; ++i) acc[n][i] += red[w][n * MB + i][lane];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          f32x4 col[NW];
#pragma unroll
          for (int n = 0; n < NW; ++n) col[n] = acc[n][i];
          const int r = mbase + 16 * i + (lane & 15);
          epilogue<F, EPI, OT, NW>(col, nb0, r, r < s1, g, lane, fa, fb, g.out);
        }
      }
      __syncthreads();
    } else {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        f32x4 col[NW];
#pragma unroll
        for (int n = 0; n < NW; ++n) col[n] = acc[n][i];
        const int r = mbase + 16 * i + (lane & 15);
        epilogue<F, EPI, OT, NW>(col, nb0, r, r < s1, g, lane, fa, fb, g.out);
      }
    }
  }
}


// ----------------------------------------------------------------------------- tile


// Workgroup tile: TN = 64 WN weight rows (NBT blocks) x TM = 16 WM MBW tokens
// (MBT blocks), WN x WM waves.  Wave (wn, wm) owns weight blocks
// [wn*NBW, (wn+1)*NBW) and token blocks [wm*MBW, (wm+1)*MBW).  Its weight
// fragments come straight from global memory into registers (the packed
// layout makes every wave access one contiguous KiB), WPF stages ahead; with
// WM = 2 the two waves of a weight slice load the same lines at the same
// stage, so the second load is served by the CU's L1 and the L2 sees each
// weight byte once per tile.  The token tile is staged through LDS
// (double-buffered, one barrier per stage).  A stage is half a K chunk: one
// 128-byte line of each token row and two 1 KiB pieces of each weight block.
// Larger tiles fetch fewer bytes from L2 per multiply-add: TN-wide tiles
// fetch each token tile N / TN times, TM-tall tiles each weight tile M / TM
// times.

template <int F, int EPI, int OT, int WN, int WM, int MBW, int WPF, int OCC>
__global__ __launch_bounds__(64 * WN * WM, OCC) void gemm_tile_kernel(GemmArgs g) {
  constexpr int NWV = WN * WM;
  constexpr int NTH = 64 * NWV;         // threads
  constexpr int TN = 64 * WN, TM = 16 * WM * MBW;
  constexpr int NBT = TN / 16, MBT = TM / 16;
  constexpr int NBW = 4;                // weight blocks per wave
  constexpr int TBYTES = MBT * 2048;    // token bytes per stage
  constexpr int TLD = TM * 8 / NTH;     // 16-byte token loads per thread per stage
  static_assert(TLD >= 1 && TLD * NTH == TM * 8, "tile shape");
  // token tile: two LDS slots, one array each
  __shared__ __attribute__((aligned(16))) uint8_t tb0[TBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t tb1[TBYTES];
  auto tbuf = [&](int slot) -> uint8_t * { return slot == 0 ? tb0 : tb1; };
  __shared__ int cum[1024];
  __shared__ uint8_t tscl[2][MBT * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wm = wave / WN;
  // Tiles are numbered expert by expert in tile_locate's order.  Workgroups
  // are dealt round-robin to the 8 XCDs; each XCD takes one contiguous range
  // of the actual tiles (counted on the device), so neighbours meet in the
  // same L2 and the surplus workgroups of the upper-bound grid are spread
  // over all XCDs.
  const int ntn = g.N / TN;
  const int total = tile_scan<TM>(g, cum) * ntn;
  const int per_xcd = (total + 7) >> 3;
  const int local = blockIdx.x >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + local;
  if (local >= per_xcd || logical >= total) return;
  int e, row0, row_end, nt;
  tile_locate<TM, kTileGM>(g, cum, ntn, logical, e, row0, row_end, nt);
  // the extra segment (bf16 / fp32 only): its own weights, rows and output
  constexpr bool kExtra = (F == FMT_BF16 || F == FMT_F32);
  const bool xseg = kExtra && g.offsets && e == g.E;
  float fa, fb;
  tensor_factors<F, EPI>(g, e, fa, fb);

  const int kcn = g.K / FmtInfo<F>::chunk_elems;
  const int nstage = 2 * kcn;
  const int nb0 = nt * NBT + wn * NBW;         // this wave's first weight block
  // Operands are read through buffer descriptors (base and size in scalar
  // registers, 32-bit per-lane offsets): the per-stage address arithmetic is
  // scalar and each lane keeps one offset per stream instead of a 64-bit
  // pointer, which leaves the vector registers to the accumulators and the
  // operands in flight.
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(xseg ? g.w2 : g.w + (size_t)e * g.w_expert_stride,
                                              (uint32_t)g.w_expert_stride);
  constexpr int TF = tok_fmt<F>;         // token-side format
  constexpr int WB = wblock_bytes<F>;    // bytes per weight block
  const uint32_t wvoff = (uint32_t)(nb0 * kcn) * WB + lane * 16;
  const __amdgpu_buffer_rsrc_t trs =
      xseg ? make_rsrc(g.a2, (uint32_t)g.a2_bytes) : make_rsrc(g.a, (uint32_t)g.a_bytes);
  // MX scales: weight scale pairs [row block][chunk][lane] of this expert,
  // token scale bytes [row][K / 32]
  __amdgpu_buffer_rsrc_t wsrs = wrs, tsrs = trs;
  uint32_t wsvoff = 0;
  if constexpr (is_mx<F>) {
    wsrs = make_rsrc(g.w_scale + (size_t)e * g.ws_expert_stride,
                     (uint32_t)(g.ws_expert_stride * sizeof(uint16_t)));
    wsvoff = (uint32_t)((nb0 * kcn) * 64 + lane) * 2;
    tsrs = make_rsrc(g.a_scale, (uint32_t)(g.a_bytes / g.a_row_bytes * (g.K / 32)));
  }

  // this thread's token rows (fixed across stages)
  uint32_t tvoff[TLD];
  int tdst[TLD];
#pragma unroll
  for (int i = 0; i < TLD; ++i) {
    const int idx = tid + NTH * i;
    const int rl = idx >> 3, seg = idx & 7;
    int r = row0 + rl;
    if (r >= row_end) r = row_end - 1;
    tvoff[i] = (uint32_t)((xseg ? (long long)r : token_of(g, r)) * g.a_row_bytes) + seg * 16;
    tdst[i] = (rl >> 4) * 2048 + (seg >> 2) * 1024 + tslot(rl & 15, seg & 3, seg >> 2) * 16;
  }
  // MX token scales: entry idx = tid + NTH i is (token block idx / 64, lane idx % 64)
  constexpr int TSL = is_mx<F> ? (MBT * 64 + NTH - 1) / NTH : 1;
  uint32_t tsvoff[TSL];
#pragma unroll
  for (int i = 0; i < TSL; ++i) tsvoff[i] = 0;
  if constexpr (is_mx<F>) {
#pragma unroll
    for (int i = 0; i < TSL; ++i) {
      const int idx = min(tid + NTH * i, MBT * 64 - 1);
      const int rl = (idx >> 6) * 16 + (idx & 15);
      int r = row0 + rl;
      if (r >= row_end) r = row_end - 1;
      tsvoff[i] = (uint32_t)(token_of(g, r) * (g.K / 32)) + ((idx >> 4) & 3);
    }
  }

  i32x4 treg[TLD];
  uint32_t tsreg[TSL];
  auto load_tokens = [&](int s) MOE_INLINE {
    const int kc = s >> 1, h = s & 1;
#pragma unroll
    for (int i = 0; i < TLD; ++i)
      treg[i] = __builtin_amdgcn_raw_buffer_load_b128(trs, (int)tvoff[i], kc * 256 + h * 128, 0);
    if constexpr (is_mx<F>) {
#pragma unroll
      for (int i = 0; i < TSL; ++i)
        tsreg[i] = __builtin_amdgcn_raw_buffer_load_b8(tsrs, (int)tsvoff[i], 8 * kc + 4 * h, 0);
    }
  };
  auto store_tokens = [&](int s) MOE_INLINE {
    uint8_t *base = tbuf(s & 1);
#pragma unroll
    for (int i = 0; i < TLD; ++i) *(i32x4 *)(base + tdst[i]) = treg[i];
    if constexpr (is_mx<F>) {
#pragma unroll
      for (int i = 0; i < TSL; ++i)
        // in a partial last round the surplus threads write the last entry
        // again, with the value its owner writes (they loaded it from the
        // same clamped offset): no branch, so the stage stays one block
        tscl[s & 1][min(tid + NTH * i, MBT * 64 - 1)] = (uint8_t)tsreg[i];
    }
  };
  // NSET = WPF + 1 register sets of weight fragments: stage s multiplies
  // one set while the loads of stages s + 1 .. s + WPF fill the others
  constexpr int NSET = WPF + 1;
  Frag<F> wr[NSET][NBW];
  uint32_t wsr[NSET][NBW];
  auto load_weights = [&](int s, int set) MOE_INLINE {
    const int kc = s >> 1, h = s & 1;
#pragma unroll
    for (int n = 0; n < NBW; ++n) {
      if constexpr (F == FMT_MX4) {
        // E2M1: half h of the block is one 1 KiB piece
        const uint32_t so = (uint32_t)(n * kcn + kc) * WB + h * 1024;
        wr[set][n].v = __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)wvoff, (int)so, 0);
      } else {
        const uint32_t so = (uint32_t)(n * kcn + kc) * WB + h * 2048;
        wr[set][n] = make_frag<F>(
            __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)wvoff, (int)so, 0),
            __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)wvoff, (int)(so + 1024), 0));
      }
      // MX: the raw scale pair of this chunk (byte h is this half's; the
      // product selects it), so nothing waits on the load before its use
      wsr[set][n] = 0;
      if constexpr (is_mx<F>)
        wsr[set][n] = __builtin_amdgcn_raw_buffer_load_b16(wsrs, (int)wsvoff,
                                                           (n * kcn + kc) * 128, 0);
    }
  };

  f32x4 acc[NBW][MBW];
#pragma unroll
  for (int n = 0; n < NBW; ++n)
#pragma unroll
    for (int m = 0; m < MBW; ++m) acc[n][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One stage.  Every load and LDS store is issued unconditionally (stage
  // indices past the end are clamped to the last stage, whose data is then
  // fetched again and never used): with no branches in the loop body the
  // compiler counts the loads in flight exactly and waits only for the ones
  // a step needs.  The order inside a stage is pinned with scheduling
  // barriers: the next stage's weight loads go out first, so their latency
  // is covered by this stage's matrix work; then the products; then the
  // token tile of stage s + 1 moves from registers to LDS (its loads were
  // issued a stage earlier) and the loads of stage s + 2 go out.  The LDS
  // buffer written after the last stage is the one the stage before it
  // read, which every wave has finished with at that stage's barrier.
  // One stage: set and slot (the register set of its weights, the LDS slot
  // of its tokens) are compile-time constants.
  auto stage = [&](int s, auto set_c, auto slot_c) MOE_INLINE {
    constexpr int set = decltype(set_c)::value, slot = decltype(slot_c)::value;
    load_weights(min(s + WPF, nstage - 1), (set + WPF) % NSET);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t *base = tbuf(slot) + wm * MBW * 2048;
    // token fragments are read one token block ahead of the products that
    // use them, so the LDS latency overlaps the matrix work
    Frag<TF> tf[2];
    uint32_t tsf[2];
    auto read_frag = [&](int m, int b) MOE_INLINE {
      const uint8_t *p = base + m * 2048;
      tf[b] = make_frag<TF>(*(const i32x4 *)(p + tslot(lane & 15, lane >> 4, 0) * 16),
                            *(const i32x4 *)(p + 1024 + tslot(lane & 15, lane >> 4, 1) * 16));
      tsf[b] = 0;
      if constexpr (is_mx<F>) tsf[b] = tscl[slot][(wm * MBW + m) * 64 + lane];
    };
    // bf16: pin the order (the two LDS reads of block m + 1, then the eight
    // products of block m) with scheduling groups
    read_frag(0, 0);
    if constexpr (F == FMT_BF16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int m = 0; m < MBW; ++m) {
      if (m + 1 < MBW) {
        read_frag(m + 1, (m + 1) & 1);
        if constexpr (F == FMT_BF16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int n = 0; n < NBW; ++n)
        mfma_frag<F, slot>(acc[n][m], wr[set][n], tf[m & 1], wsr[set][n], tsf[m & 1]);
      if constexpr (F == FMT_BF16) __builtin_amdgcn_sched_group_barrier(0x008, 2 * NBW, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    store_tokens(s + 1);
    load_tokens(min(s + 2, nstage - 1));
    __syncthreads();
  };
  load_tokens(0);
#pragma unroll
  for (int q = 0; q < WPF; ++q) load_weights(min(q, nstage - 1), q);
  store_tokens(0);
  load_tokens(min(1, nstage - 1));
  __syncthreads();
  // stages in periods of P = lcm(NSET, 2) (slot = s % 2) so that set and
  // slot are constants; the last nstage % P stages follow the loop
  constexpr int P = (NSET % 2 == 0) ? NSET : 2 * NSET;
  auto stage_q = [&](int s, auto q) MOE_INLINE {
    constexpr int Q = decltype(q)::value;
    stage(s, std::integral_constant<int, Q % NSET>{}, std::integral_constant<int, Q % 2>{});
  };
  int s0 = 0;
  for (; s0 + P <= nstage; s0 += P) static_for<P>([&](auto q) MOE_INLINE { stage_q(s0 + q.value, q); });
  static_for<P - 1>([&](auto q) MOE_INLINE {
    if (s0 + q.value < nstage) stage_q(s0 + q.value, q);
  });

  if constexpr (EPI == EPI_PLAIN && F == FMT_BF16 && OT == FMT_BF16 && WM == 1 && TN == 256) {
    // bf16 output of the bf16 GEMMs through the token LDS slots (free after
    // the last stage): each pass writes RPP rows of the tile there, their
    // 16-byte segments permuted by row so that the 16 rows of one write hit
    // distinct banks, then every row leaves as 512 contiguous bytes (prefill
    // down GEMM 1.078 -> 1.025 ms against the 16-byte stores of epilogue();
    // the 8-bit kernels keep epilogue(): there this path spills)
    constexpr int RB = TN * 2, SEGS = RB / 16;
    constexpr int RPS = TBYTES / RB, RPP = 2 * RPS, MPP = RPP / 16;
    static_assert(RPP % 16 == 0 && TM % RPP == 0, "epilogue passes");
    static_assert(RPP * SEGS % NTH == 0, "every thread reads whole rounds of segments");
    uint16_t *outp = (uint16_t *)(xseg ? g.out2 : g.out);
    static_for<TM / RPP>([&](auto pc) MOE_INLINE {
      constexpr int pass = decltype(pc)::value;
      __syncthreads();
#pragma unroll
      for (int mm = 0; mm < MPP; ++mm) {
        const int rl = mm * 16 + (lane & 15);
        uint8_t *slot = rl < RPS ? tb0 : tb1;
        const int r2 = rl < RPS ? rl : rl - RPS;
#pragma unroll
        for (int n = 0; n < NBW; ++n) {
          const f32x4 v = acc[n][pass * MPP + mm];
          const int cb = ((wn * NBW + n) * 16 + 4 * (lane >> 4)) * 2;
          uint2 q;
          q.x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
          q.y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
          *(uint2 *)(slot + r2 * RB + (((cb >> 4) ^ (r2 & 31)) << 4) + (cb & 15)) = q;
        }
      }
      __syncthreads();
#pragma unroll
      for (int i0 = 0; i0 < RPP * SEGS; i0 += NTH) {
        const int i = i0 + tid;
        const int rl = i / SEGS, seg = i % SEGS;
        const uint8_t *slot = rl < RPS ? tb0 : tb1;
        const int r2 = rl < RPS ? rl : rl - RPS;
        const uint4 q = *(const uint4 *)(slot + r2 * RB + ((seg ^ (r2 & 31)) << 4));
        const int row = row0 + pass * RPP + rl;
        if (row < row_end) *(uint4 *)(outp + (long long)row * g.n_out + nt * TN + seg * 8) = q;
      }
    });
  } else {
#pragma unroll
  for (int m = 0; m < MBW; ++m) {
    f32x4 col[NBW];
#pragma unroll
    for (int n = 0; n < NBW; ++n) col[n] = acc[n][m];
    const int r = row0 + (wm * MBW + m) * 16 + (lane & 15);
    epilogue<F, EPI, OT, NBW>(col, nb0, r, r < row_end, g, lane, fa, fb, xseg ? g.out2 : g.out);
  }
  }
}

// ----------------------------------------------------------------------------- dispatch

// lds_pad: dynamic LDS per workgroup, which only caps residency.
template <int F, int EPI, int OT, int NW, int MB, int KSW>
static hipError_t launch_skinny(const GemmArgs &g, int segs, hipStream_t stream, int lds_pad = 0) {
  constexpr int BPW = (KSW == 4) ? NW : 4 * NW;
  const int nbtot = g.N / 16;
  if (nbtot % BPW) return hipErrorInvalidValue;
  gemm_skinny_kernel<F, EPI, OT, NW, MB, KSW>
      <<<segs * (nbtot / BPW), 256, lds_pad, stream>>>(g);
  return hipGetLastError();
}

// Tiled kernel over the segments longer than g.split: WN x WM waves, MBW
// token blocks per wave.
template <int F, int EPI, int OT, int WN, int WM, int MBW, int WPF, int OCC>
static hipError_t launch_tile(GemmArgs g, int total_rows, hipStream_t stream) {
  constexpr int TN = 64 * WN, TM = 16 * WM * MBW;
  if (g.N % TN != 0) return hipErrorInvalidValue;
  const int mtiles = g.offsets ? (total_rows + TM - 1) / TM + g.E + (g.rows2 + TM - 1) / TM
                               : (g.rows + TM - 1) / TM;
  g.mt_upper = mtiles;
  // upper bound on the tiles, rounded up to whole rounds of the 8 XCDs
  long long nblocks = (long long)mtiles * (g.N / TN);
  nblocks = ((nblocks + 7) / 8) * 8 + 8;
  gemm_tile_kernel<F, EPI, OT, WN, WM, MBW, WPF, OCC>
      <<<(unsigned)nblocks, 64 * WN * WM, 0, stream>>>(g);
  return hipGetLastError();
}

template <int F, int EPI, int OT>
static hipError_t run_gemm(const GemmArgs &g0, int total_rows, hipStream_t stream) {
  GemmArgs g = g0;
  if (g.rows2 > 0) {
    // The extra segment rides in the tiled launch (filling the routed
    // GEMM's last, partial round of tiles) where that launch takes long
    // segments; otherwise it runs as a GEMM of its own.
    const bool tiled = (F == FMT_BF16 || F == FMT_F32) && g.offsets && g.E < 1024 &&
                       g.rows > 64 * g.k_route && g.a_bytes <= 0xFFFFFFFFll &&
                       g.a2_bytes <= 0xFFFFFFFFll && g.w_expert_stride <= 0xFFFFFFFFull &&
                       g.N % (64 * kTileWN) == 0;
    if (!tiled) {
      GemmArgs gx = g0;
      gx.w = g0.w2;
      gx.a = g0.a2;
      gx.a_bytes = g0.a2_bytes;
      gx.sorted_src = nullptr;
      gx.offsets = nullptr;
      gx.rows = g0.rows2;
      gx.E = 1;
      gx.out = g0.out2;
      gx.rows2 = 0;
      const hipError_t err = run_gemm<F, EPI, OT>(gx, gx.rows, stream);
      if (err != hipSuccess) return err;
      g.rows2 = 0;
    }
  }
  const int segs = g.offsets ? g.E : 1;
  // rows per segment: the mean for expert segments, all rows for one segment
  const int per = g.offsets ? (total_rows + segs - 1) / segs : total_rows;
  // weight blocks a SwiGLU workgroup must hold: gate/up pairs (2), and for the
  // MX-quantising epilogue whole 32-column blocks (4)
  constexpr int NWS = (EPI == EPI_SWIGLU) ? (OT == FMT_MX8 ? 4 : 2) : 1;
  // The tiled kernel addresses its operands with 32-bit offsets; beyond 4 GiB
  // of token-side data or of one expert's weights every segment goes to the
  // streaming kernel, which walks any number of rows in passes.
  if (g.a_bytes > 0xFFFFFFFFll || g.w_expert_stride > 0xFFFFFFFFull) {
    if (!g.offsets) return launch_skinny<F, EPI, OT, NWS, 4, 4>(g, 1, stream);
    return launch_skinny<F, EPI, OT, 4, 4, 1>(g, segs, stream);
  }
  if (!g.offsets) {
    // one segment (shared expert): few weight blocks per workgroup, K split
    // over the four waves, so the weights spread over many workgroups
    if (per <= 16) return launch_skinny<F, EPI, OT, NWS, 1, 4>(g, 1, stream);
    if (per <= 32) return launch_skinny<F, EPI, OT, NWS, 2, 4>(g, 1, stream);
    if (per <= 64) return launch_skinny<F, EPI, OT, NWS, 4, 4>(g, 1, stream);
  } else if (g.rows <= 64 * g.k_route) {
    // at most T <= 64 rows per expert: the streaming kernel takes them all
    constexpr bool eight = (F == FMT_FP8 || F == FMT_MX8);
    constexpr int SNW0 = (F == FMT_MX4 && EPI == EPI_SWIGLU) ? kSkinnyNWMx4
                         : eight                              ? kSkinnyNW8
                                                              : kSkinnyNW;
    const int pad = eight ? kSkinnyLdsPad8 : kSkinnyLdsPad;
    // a SwiGLU epilogue needs gate/up pairs (2 weight blocks), an
    // MX-quantising one whole 32-column blocks (4)
    constexpr int SNW = (EPI == EPI_SWIGLU && OT == FMT_MX8 && SNW0 < 4)   ? 4
                        : (EPI == EPI_SWIGLU && SNW0 < 2) ? 2
                                                          : SNW0;
    if (per <= 16) {
      if constexpr (F == FMT_BF16 || F == FMT_F32)
        return launch_skinny<F, EPI, OT, SNW, 1, 4>(g, segs, stream, kSkinnyLdsPadKs);
      return launch_skinny<F, EPI, OT, SNW, 1, 1>(g, segs, stream, pad);
    }
    if (per <= 32) return launch_skinny<F, EPI, OT, 4, 2, 1>(g, segs, stream);
    return launch_skinny<F, EPI, OT, 4, 4, 1>(g, segs, stream);
  } else if (per <= kHybMean) {
    // experts of at most kHybSplit rows go to the streaming kernel, the
    // longer ones to the tiled kernel (the split is applied on the device,
    // where the counts are)
    g.split = kHybSplit;
    constexpr int HNW = (EPI == EPI_SWIGLU && OT == FMT_MX8) ? 4 : kHybNW;
    hipError_t err = launch_skinny<F, EPI, OT, HNW, kHybMB, 1>(g, segs, stream);
    if (err != hipSuccess) return err;
  }
  if constexpr (is_mx<F> || F == FMT_FP8) {
    return launch_tile<F, EPI, OT, 4, 1, kTileTMMx / 16, 1, kTileOccMx>(g, total_rows,
                                                                                  stream);
  } else {
    // two waves per SIMD: one workgroup of WN x WM = 8 waves, or two of 4
    constexpr int WN = kTileWN, WM = kTileWM;
    constexpr int OCC = (WN * WM >= 8) ? 1 : kTileOcc;
    if (g.N % (64 * WN) == 0)
      return launch_tile<F, EPI, OT, WN, WM, kTileMBW, kTileWPF, OCC>(g, total_rows,
                                                                               stream);
    return launch_tile<F, EPI, OT, 4, 1, 8, 1, 2>(g, total_rows, stream);
  }
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
  if (fmt == FMT_FP8) {
    // static per-tensor FP8: h is E4M3 under its own static scale
    if (epi == EPI_SWIGLU) return run_gemm<FMT_FP8, EPI_SWIGLU, FMT_FP8>(g, total_rows, stream);
    if (out_fmt == FMT_BF16) return run_gemm<FMT_FP8, EPI_PLAIN, FMT_BF16>(g, total_rows, stream);
  }
  if (fmt == FMT_MX4) {
    // E2M1 weights, MX-fp8 tokens; the SwiGLU output is MX-fp8 like the input
    if (epi == EPI_SWIGLU) return run_gemm<FMT_MX4, EPI_SWIGLU, FMT_MX8>(g, total_rows, stream);
    if (out_fmt == FMT_BF16) return run_gemm<FMT_MX4, EPI_PLAIN, FMT_BF16>(g, total_rows, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
