// moe_launch.hpp -- host-side launchers of the MoE layer kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// One grouped GEMM launch: out[r] = epilogue( W_e . a[token(r)] ) for the rows
// r of every expert segment.  Weights are packed 4 KiB blocks (16 rows x one
// 256-byte K chunk), ordered [expert][row block][chunk].
struct GemmArgs {
  const uint8_t *w;           // packed weights of expert 0
  const uint16_t *w_scale;    // MX: packed scale pairs [expert][row block][chunk][lane]
  size_t w_expert_stride;     // bytes between experts in w
  size_t ws_expert_stride;    // uint16 entries between experts in w_scale
  const uint8_t *a;           // token-side rows (x or h), row-major, expert format
  const uint8_t *a_scale;     // MX: [rows][K/32] E8M0 bytes
  long long a_row_bytes;      // bytes per token-side row
  long long a_bytes;          // bytes of the whole token-side array
  const int32_t *sorted_src;  // row r reads token sorted_src[r] / k_route; NULL: row r
  int k_route;
  const int32_t *offsets;     // [E+1] segment bounds; NULL: one segment [0, rows)
  int rows;                   // rows when offsets == NULL
  int E;                      // experts (segments)
  int N;                      // output features (virtual rows of W)
  int K;                      // reduction length (elements)
  void *out;                  // row-major [rows][n_out]
  uint8_t *out_scale;         // MX output scales [rows][n_out/32]
  int n_out;                  // output columns: N/2 for SwiGLU, N otherwise
  int mt_upper;               // tile kernel: m-tiles in the grid
  int split;                  // > 0: the streaming kernel takes segments of at most
                              // `split` rows and the tiled kernel the longer ones
  // bf16 / fp32 only: one more segment after the E expert segments when
  // rows2 > 0 (the shared expert folded into the routed GEMM): rows2 rows
  // read straight from a2 (no gather; a2_bytes bytes, a_row_bytes per row)
  // against the weight set w2 (one expert's layout and stride), written to
  // out2 ([rows2][n_out])
  const uint8_t *w2;
  const uint8_t *a2;
  long long a2_bytes;
  void *out2;
  int rows2;
  // static per-tensor FP8 only: weight scales per expert ([E][2] gate, up for
  // SwiGLU; [E] otherwise), the token-side activation scale, and the scale
  // the SwiGLU output is quantised with
  const float *w_tscale;
  float a_tscale;
  float out_tscale;
};

enum Epi { EPI_SWIGLU = 0, EPI_PLAIN = 1 };

// fmt: weight format (Fmt in moe_common.hpp; the token side is MX-fp8 for
// FMT_MX4 and the same format otherwise); out_fmt: FMT_F32, FMT_BF16, or for
// SwiGLU FMT_MX8 (MX formats) / FMT_FP8 (static FP8).  total_rows: rows of
// all segments, used only to choose between the streaming and the tiled
// kernel.
hipError_t launch_grouped_gemm(const GemmArgs &g, int fmt, int epi, int out_fmt, int total_rows,
                               hipStream_t stream);

// Gating.  part: route_ws_bytes() of scratch for the fp32 partial logits.
size_t route_ws_bytes(int T, int H, int E, int x_is_bf16);
hipError_t launch_route(const void *x, int x_is_bf16, const float *Wr, const float *bias,
                        float *part, int32_t *topk_idx, float *topk_w, int T, int H, int E, int k,
                        float rho, int route_norm, hipStream_t stream);

size_t permute_ws_bytes(int T, int E);
hipError_t launch_permute(const int32_t *topk_idx, int T, int E, int k, int32_t *counts,
                          int32_t *offsets, int32_t *sorted_src, int32_t *dest, void *ws,
                          hipStream_t stream);

hipError_t launch_combine(const void *y, int y_fmt, const int32_t *dest, const float *topk_w,
                          const void *shared_out, int T, int H, int k, void *out, int out_fmt,
                          hipStream_t stream);

hipError_t launch_mx_quantize(const void *src, int src_is_bf16, long long rows, long long cols,
                              uint8_t *q, uint8_t *scale, hipStream_t stream);

// E4M3 codes of fp32(src / scale) for n elements (static per-tensor FP8).
hipError_t launch_fp8_quantize(const void *src, int src_is_bf16, long long n, float scale,
                               uint8_t *q, hipStream_t stream);

// Pack [E][rows][K] sources (gate/up interleaved when gate_up != 0) into the
// block layout of fmt.  src_is_bf16 selects the source element type.
// Static per-tensor FP8: tscale receives each source matrix's scale
// max|w| / 448 ([E][2] gate, up when gate_up != 0, else [E]) before the
// codes are written.
hipError_t launch_pack(const void *a, const void *b, int src_is_bf16, int E, int N, int K,
                       int gate_up, int fmt, uint8_t *out, uint16_t *scale_out, float *tscale,
                       hipStream_t stream);

}  // namespace moe
