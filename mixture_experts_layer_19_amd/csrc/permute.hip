// permute.hip -- InitRouting: group the (token, slot) pairs by expert.
//
// Hy3 on CANN NPU guide, section 8.1 (MoE EP) and section 8.5: InitRouting
// matches tokens to experts ahead of the grouped GEMM.  Pair f = t*k + j goes
// to row r = offsets[e] + #{earlier pairs routed to e}, so each expert's rows
// are in ascending token order.  Because a token's k experts are distinct,
// that rank is the number of earlier *tokens* that picked e, which is what
// the kernels count: per block of 256 tokens a bitmap column per expert
// (bit t set when token t picked e), block totals scanned per expert, and a
// popcount of the bits below t.  Everything is integer and order-free, so the
// result is deterministic and exactly the stable order.
#include "moe_common.hpp"
#include "moe_launch.hpp"

namespace moe {

constexpr int kPermBlock = 256;               // tokens per block
constexpr int kPermWords = kPermBlock / 32;   // bitmap words per (block, expert)

constexpr int kMaxChoices = 16;               // largest k the library accepts

// The k expert indices of token t, all read before any is used so that the
// loads are in flight together: KT = 4 or 8 reads 16-byte vectors (the
// caller checks the alignment), KT = 0 reads k scalars (entries past k
// repeat the last one and are not used).
template <int KT>
__device__ __forceinline__ void load_choices(const int32_t *__restrict__ topk_idx, int t, int k,
                                             int (&ev)[kMaxChoices]) {
  if constexpr (KT == 4 || KT == 8) {
    const int4 *p = (const int4 *)(topk_idx + (size_t)t * KT);
#pragma unroll
    for (int q = 0; q < KT / 4; ++q) {
      const int4 v = p[q];
      ev[4 * q] = v.x;
      ev[4 * q + 1] = v.y;
      ev[4 * q + 2] = v.z;
      ev[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kMaxChoices; ++j) ev[j] = topk_idx[(size_t)t * k + min(j, k - 1)];
  }
}

// Phase 1: per token block, the bitmap column of every expert and its count.
template <int KT>
__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t *__restrict__ topk_idx, int T,
                                                         int E, int k, uint32_t *__restrict__ bits,
                                                         int32_t *__restrict__ blk_count) {
  constexpr int KM = KT > 0 ? KT : kMaxChoices;
  extern __shared__ uint32_t col[];           // [E][kPermWords]
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int i = tid; i < E * kPermWords; i += 256) col[i] = 0u;
  const int t = b * kPermBlock + tid;
  int ev[kMaxChoices];
  if (t < T) load_choices<KT>(topk_idx, t, k, ev);
  __syncthreads();
  if (t < T) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int e = ev[j];
      if ((KT > 0 || j < k) && e >= 0 && e < E)
        atomicOr(&col[e * kPermWords + (tid >> 5)], 1u << (tid & 31));
    }
  }
  __syncthreads();
  uint32_t *out = bits + (size_t)b * E * kPermWords;
  for (int i = tid; i < E * kPermWords; i += 256) out[i] = col[i];
  for (int e = tid; e < E; e += 256) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kPermWords; ++w) c += __popc(col[e * kPermWords + w]);
    blk_count[(size_t)b * E + e] = c;
  }
}

// Inclusive scan of tot[0, E) in LDS (E <= 1024) by a workgroup of 256
// threads, called by all of them after the entries are written and a
// barrier: thread t owns entries 4t..4t+3, the waves scan their threads'
// sums with shuffles, and the four wave totals are added in wave order.  The
// workgroup is synchronised again on return.
__device__ __forceinline__ void block_scan_counts(int32_t *tot, int E) {
  __shared__ int wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int v[4], run = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * tid + i;
    run += (e < E) ? tot[e] : 0;
    v[i] = run;
  }
  int x = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  int before = x - run;
  for (int w = 0; w < wave; ++w) before += wtot[w];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (4 * tid + i < E) tot[4 * tid + i] = before + v[i];
  __syncthreads();
}

// Phase 2 (one workgroup): per-expert exclusive scan over blocks, the
// per-expert counts, and the exclusive scan over experts.
__global__ __launch_bounds__(256) void perm_scan_kernel(const int32_t *__restrict__ blk_count,
                                                         int nblk, int E,
                                                         int32_t *__restrict__ blk_base,
                                                         int32_t *__restrict__ counts,
                                                         int32_t *__restrict__ offsets) {
  __shared__ int32_t tot[1024];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    // eight block counts are read before any is added, so eight loads are
    // in flight instead of one
    int run = 0, b = 0;
    for (; b + 8 <= nblk; b += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = blk_count[(size_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        blk_base[(size_t)(b + u) * E + e] = run;
        run += c[u];
      }
    }
    for (; b < nblk; ++b) {
      blk_base[(size_t)b * E + e] = run;
      run += blk_count[(size_t)b * E + e];
    }
    counts[e] = run;
    tot[e] = run;
  }
  __syncthreads();
  block_scan_counts(tot, E);
  for (int e = tid; e <= E; e += blockDim.x) offsets[e] = (e == 0) ? 0 : tot[e - 1];
}

// Phase 3: every pair computes its row and writes both directions.  The
// block's bitmap columns and its first row per expert are staged in LDS
// first (coalesced), so the ranks read no global memory.
template <int KT>
__global__ __launch_bounds__(256) void perm_scatter_kernel(
    const int32_t *__restrict__ topk_idx, int T, int E, int k, const uint32_t *__restrict__ bits,
    const int32_t *__restrict__ blk_base, const int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_src, int32_t *__restrict__ dest) {
  constexpr int KM = KT > 0 ? KT : kMaxChoices;
  extern __shared__ uint32_t col[];           // [E][kPermWords], then first row [E]
  int32_t *first = (int32_t *)(col + E * kPermWords);
  const int b = blockIdx.x, tid = threadIdx.x;
  const int t = b * kPermBlock + tid;
  int ev[kMaxChoices];
  if (t < T) load_choices<KT>(topk_idx, t, k, ev);
  const uint32_t *bb = bits + (size_t)b * E * kPermWords;
  for (int i = tid; i < E * kPermWords; i += 256) col[i] = bb[i];
  for (int e = tid; e < E; e += 256) first[e] = offsets[e] + blk_base[(size_t)b * E + e];
  __syncthreads();
  if (t >= T) return;
  const int word = tid >> 5;
  const uint32_t below = (1u << (tid & 31)) - 1u;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int f = t * k + j;
    const int e = ev[j];
    if ((KT == 0 && j >= k) || e < 0 || e >= E) continue;
    const uint32_t *c = col + e * kPermWords;
    int rank = __popc(c[word] & below);
    for (int w = 0; w < word; ++w) rank += __popc(c[w]);
    const int r = first[e] + rank;
    sorted_src[r] = f;
    dest[f] = r;
  }
}

// All three phases in one workgroup, for a single token block (T <= 256):
// the bitmap columns stay in LDS, and one launch replaces three.
template <int KT>
__global__ __launch_bounds__(256) void perm_single_kernel(
    const int32_t *__restrict__ topk_idx, int T, int E, int k, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_src, int32_t *__restrict__ dest) {
  constexpr int KM = KT > 0 ? KT : kMaxChoices;
  extern __shared__ uint32_t col[];           // [E][kPermWords], then tot[1024]
  int32_t *tot = (int32_t *)(col + E * kPermWords);
  const int tid = threadIdx.x;
  int ev[kMaxChoices];
  if (tid < T) load_choices<KT>(topk_idx, tid, k, ev);
  for (int i = tid; i < E * kPermWords; i += 256) col[i] = 0u;
  __syncthreads();
  if (tid < T) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int e = ev[j];
      if ((KT > 0 || j < k) && e >= 0 && e < E)
        atomicOr(&col[e * kPermWords + (tid >> 5)], 1u << (tid & 31));
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kPermWords; ++w) c += __popc(col[e * kPermWords + w]);
    counts[e] = c;
    tot[e] = c;
  }
  __syncthreads();
  block_scan_counts(tot, E);
  for (int e = tid; e <= E; e += 256) offsets[e] = (e == 0) ? 0 : tot[e - 1];
  if (tid >= T) return;
  const int word = tid >> 5;
  const uint32_t below = (1u << (tid & 31)) - 1u;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int f = tid * k + j;
    const int e = ev[j];
    if ((KT == 0 && j >= k) || e < 0 || e >= E) continue;
    const uint32_t *c = col + e * kPermWords;
    int rank = __popc(c[word] & below);
    for (int w = 0; w < word; ++w) rank += __popc(c[w]);
    const int r = (e == 0 ? 0 : tot[e - 1]) + rank;
    sorted_src[r] = f;
    dest[f] = r;
  }
}

size_t permute_ws_bytes(int T, int E) {
  size_t nblk = (size_t)(T + kPermBlock - 1) / kPermBlock;
  size_t b = nblk * E * kPermWords * sizeof(uint32_t);
  b = (b + 255) & ~(size_t)255;
  size_t c = nblk * E * sizeof(int32_t);
  c = (c + 255) & ~(size_t)255;
  return b + 2 * c;
}

hipError_t launch_permute(const int32_t *topk_idx, int T, int E, int k, int32_t *counts,
                          int32_t *offsets, int32_t *sorted_src, int32_t *dest, void *ws,
                          hipStream_t stream) {
  const int nblk = (T + kPermBlock - 1) / kPermBlock;
  size_t nb = (size_t)nblk * E * kPermWords * sizeof(uint32_t);
  nb = (nb + 255) & ~(size_t)255;
  size_t nc = (size_t)nblk * E * sizeof(int32_t);
  nc = (nc + 255) & ~(size_t)255;
  uint32_t *bits = (uint32_t *)ws;
  int32_t *blk_count = (int32_t *)((char *)ws + nb);
  int32_t *blk_base = (int32_t *)((char *)ws + nb + nc);
  // k = 4 or 8 with 16-byte aligned rows: vector reads of the choices
  const bool vec = ((uintptr_t)topk_idx & 15) == 0;
  const int kt = vec && (k == 4 || k == 8) ? k : 0;
#define MOE_PERM_K(KERNEL, ...)                                             \
  (kt == 8 ? KERNEL<8> __VA_ARGS__ : kt == 4 ? KERNEL<4> __VA_ARGS__ : KERNEL<0> __VA_ARGS__)
  if (nblk == 1) {
    const size_t lds = (size_t)E * kPermWords * sizeof(uint32_t) + 1024 * sizeof(int32_t);
    MOE_PERM_K(perm_single_kernel, <<<1, 256, lds, stream>>>(topk_idx, T, E, k, counts, offsets,
                                                             sorted_src, dest));
    return hipGetLastError();
  }
  if (nblk > 0) {
    MOE_PERM_K(perm_count_kernel,
               <<<nblk, 256, (size_t)E * kPermWords * sizeof(uint32_t), stream>>>(
                   topk_idx, T, E, k, bits, blk_count));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  perm_scan_kernel<<<1, 256, 0, stream>>>(blk_count, nblk, E, blk_base, counts, offsets);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nblk == 0) return err;
  MOE_PERM_K(perm_scatter_kernel,
             <<<nblk, 256, (size_t)E * (kPermWords + 1) * sizeof(uint32_t), stream>>>(
                 topk_idx, T, E, k, bits, blk_base, offsets, sorted_src, dest));
#undef MOE_PERM_K
  return hipGetLastError();
}

}  // namespace moe
