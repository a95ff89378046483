// Mixture-of-experts block with the experts sharded in place, for one
// tensor-parallel rank on gfx950: routing, grouping of the routed rows by
// expert, and the weighted combine around two grouped GEMMs.
//
// What is computed ("Tensor-parallel all-reduce count per transformer layer
// in MLX shard_linear", Facts: the MoE layers of DeepSeek V3 and Qwen3-MoE
// shard their routed experts in place, keep the router replicated and sum the
// block output once): each token goes to its top-k experts (softmax over the
// router logits, ties to the lower expert index, probabilities renormalised
// over the k chosen), and the rank's partial is
//   y_i[t] = sum_j gate[t, j] * swiglu_shard(x[t]; expert idx[t, j]).
//
// Design:
//  * Routing: one thread per token, k passes of an arg-max over the fp32
//    logits (k <= 16, E <= 1024), exponentials relative to the largest.
//  * Grouping, without a host round trip: per-expert counts (atomics), one
//    workgroup turns them into offsets with every expert's group padded to a
//    whole 128-row tile and writes the tile -> expert table, then each routed
//    (token, slot) takes a row in its expert's group.  Row order inside a
//    group does not affect any value (every output row is its own dot
//    products), so the atomics leave results bitwise reproducible.
//  * The routed rows of x are gathered into the grouped order (padding rows
//    zero), the grouped tiled GEMMs read each tile's expert weights from the
//    table (gate/up with the SwiGLU epilogue, then down to fp32), and the
//    combine adds each token's k rows in slot order with their gates.
#include "tp_kernels.h"
#include "tp_device.h"

namespace tpk {
namespace {

__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                        int* __restrict__ idx, float* __restrict__ gate) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const float* lg = logits + (int64_t)t * E;
  uint32_t taken[MOE_MAX_E / 32];
#pragma unroll
  for (int w = 0; w < MOE_MAX_E / 32; ++w) taken[w] = 0u;
  int sel[MOE_MAX_K];
  float val[MOE_MAX_K];
  for (int j = 0; j < k; ++j) {
    int best = -1;
    float bv = 0.0f;
    for (int e = 0; e < E; ++e) {
      if (taken[e >> 5] >> (e & 31) & 1u) continue;
      const float v = lg[e];
      if (best < 0 || v > bv) {  // strict: equal logits keep the lower index
        best = e;
        bv = v;
      }
    }
    taken[best >> 5] |= 1u << (best & 31);
    sel[j] = best;
    val[j] = bv;
  }
  float w[MOE_MAX_K];
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) {
    w[j] = expf(val[j] - val[0]);
    sum += w[j];
  }
  for (int j = 0; j < k; ++j) {
    idx[(int64_t)t * k + j] = sel[j];
    gate[(int64_t)t * k + j] = w[j] / sum;
  }
}

// (expert indices outside [0, E) are skipped here and in the scatter: such a
// slot contributes nothing)
__global__ __launch_bounds__(256) void moe_count_kernel(const int* __restrict__ idx, int n, int E,
                                                        int* __restrict__ counts) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int e = idx[i];
  if (e >= 0 && e < E) atomicAdd(&counts[e], 1);
}

// One workgroup: padded group offsets, tile -> expert table, cleared cursors
// and padding rows marked empty.
__global__ __launch_bounds__(1024) void moe_plan_kernel(const int* __restrict__ counts, int E, int* __restrict__ offsets,
                                                        int* __restrict__ cursors, int* __restrict__ tile_expert,
                                                        int n_tiles, int* __restrict__ src_row, int rows) {
  __shared__ int s_off[MOE_MAX_E + 1];
  if (threadIdx.x == 0) {
    int o = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e] = o;
      o += (counts[e] + MOE_TILE - 1) / MOE_TILE * MOE_TILE;
    }
    s_off[E] = o;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = s_off[e];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cursors[e] = 0;
  for (int tl = threadIdx.x; tl < n_tiles; tl += blockDim.x) {
    const int r = tl * MOE_TILE;
    int ex = -1;
    if (r < s_off[E]) {  // the expert whose padded group holds row r (binary search)
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= r) lo = mid;
        else hi = mid - 1;
      }
      ex = lo;
    }
    tile_expert[tl] = ex;
  }
  for (int r = threadIdx.x; r < rows; r += blockDim.x) src_row[r] = -1;
}

__global__ __launch_bounds__(256) void moe_scatter_kernel(const int* __restrict__ idx, int n, int k, int E,
                                                          const int* __restrict__ offsets, int* __restrict__ cursors,
                                                          int* __restrict__ src_row, int* __restrict__ pos_of) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int e = idx[i];
  if (e < 0 || e >= E) {
    pos_of[i] = -1;
    return;
  }
  const int pos = offsets[e] + atomicAdd(&cursors[e], 1);
  src_row[pos] = i / k;
  pos_of[i] = pos;
}

// xs[r] = x[src_row[r]] (zero for padding rows); d % 8 == 0, 16-byte rows.
__global__ __launch_bounds__(256) void moe_gather_kernel(const uint4* __restrict__ x, const int* __restrict__ src_row,
                                                         int rows, int d8, uint4* __restrict__ xs) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * d8) return;
  const int r = (int)(i / d8), c = (int)(i % d8);
  const int s = src_row[r];
  xs[i] = s >= 0 ? x[(int64_t)s * d8 + c] : make_uint4(0u, 0u, 0u, 0u);
}

// y[t, c] = sum_j gate[t, j] * zs[pos_of[t, j], c] in slot order (fp32).
template <typename OutT>
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ zs, const int* __restrict__ pos_of,
                                                          const float* __restrict__ gate, int T, int k, int d,
                                                          OutT* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * d) return;
  const int t = (int)(i / d), c = (int)(i % d);
  float s = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int pos = pos_of[(int64_t)t * k + j];
    if (pos >= 0) s += gate[(int64_t)t * k + j] * zs[(int64_t)pos * d + c];
  }
  if constexpr (std::is_same<OutT, float>::value) y[i] = s;
  else y[i] = f2bf(s);
}

unsigned blocks(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t moe_route(const float* logits, int T, int E, int k, int* idx, float* gate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_route_kernel, dim3(blocks(T, 256)), dim3(256), 0, s, logits, T, E, k, idx, gate);
  return hipGetLastError();
}

hipError_t moe_group(const int* idx, int T, int E, int k, const void* x, int d, int rows, int n_tiles, int* counts,
                     int* offsets, int* cursors, int* tile_expert, int* src_row, int* pos_of, void* xs, hipStream_t s) {
  const int n = T * k;
  hipError_t e = zero_fill(counts, (size_t)E * sizeof(int), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_count_kernel, dim3(blocks(n, 256)), dim3(256), 0, s, idx, n, E, counts);
  hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(1024), 0, s, counts, E, offsets, cursors, tile_expert, n_tiles,
                     src_row, rows);
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(blocks(n, 256)), dim3(256), 0, s, idx, n, k, E, offsets, cursors,
                     src_row, pos_of);
  const int64_t units = (int64_t)rows * (d / 8);
  hipLaunchKernelGGL(moe_gather_kernel, dim3(blocks(units, 256)), dim3(256), 0, s, reinterpret_cast<const uint4*>(x),
                     src_row, rows, d / 8, reinterpret_cast<uint4*>(xs));
  return hipGetLastError();
}

hipError_t moe_combine(const float* zs, const int* pos_of, const float* gate, int T, int k, int d, void* y,
                       bool out_f32, hipStream_t s) {
  const int64_t n = (int64_t)T * d;
  if (n == 0) return hipSuccess;
  if (out_f32)
    hipLaunchKernelGGL(moe_combine_kernel<float>, dim3(blocks(n, 256)), dim3(256), 0, s, zs, pos_of, gate, T, k, d,
                       reinterpret_cast<float*>(y));
  else
    hipLaunchKernelGGL(moe_combine_kernel<uint16_t>, dim3(blocks(n, 256)), dim3(256), 0, s, zs, pos_of, gate, T, k, d,
                       reinterpret_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace tpk
