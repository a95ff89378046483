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
//  * Routing: one wave per token, k passes of a wave arg-max over the fp32
//    logits (k <= 16, E <= 1024), exponentials relative to the largest.
//  * Grouping, without a host round trip: one workgroup counts the routed
//    slots per expert in LDS and turns the counts into offsets with every
//    expert's group padded to whole MOE_TILE-row tiles (and the tile -> expert
//    table), then each routed (token, slot) takes a row in its expert's group
//    (per-workgroup LDS counts, one global atomic per workgroup and
//    expert).  Row order inside a group does not affect any value (every
//    output row is its own dot products), so the atomics leave results
//    bitwise reproducible.
//  * The grouped tiled GEMMs read each tile's expert weights from the tile
//    table (gate/up with the SwiGLU epilogue, then down to fp32 rows); the
//    gate/up GEMM reads the routed rows of x through the row table (padding
//    rows load as zeros; an x of 2 GiB or more is first gathered into the
//    grouped order), and the down GEMM stores each row at its (token, slot)
//    position (padding rows are not stored), rounded to bf16 when the block's
//    output is bf16 (an intermediate, like h) and fp32 otherwise.  The
//    combine adds each token's k contiguous rows in slot order with their
//    gates, in fp32.
#include "tp_kernels.h"
#include "tp_device.h"

namespace tpk {
namespace {

constexpr int SCATTER_PER = 512;  // routed slots per scatter workgroup

// (bv, be) <- the better of itself and (ov, oe): larger value, then lower index.
__device__ __forceinline__ void take(float& bv, int& be, float ov, int oe) {
  if (ov > bv || (ov == bv && oe < be)) {
    bv = ov;
    be = oe;
  }
}

// take() with the partner lane's pair read through a DPP permutation.
template <int CTRL>
__device__ __forceinline__ void dpp_take(float& bv, int& be) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oe = __builtin_amdgcn_update_dpp(0, be, CTRL, 0xF, 0xF, false);
  take(bv, be, ov, oe);
}

// One wave per token: lane l holds logits l, l + 64, ... (a NaN logit ranks
// as -inf); each of the k passes takes the wave's arg-max (larger value, then
// lower index) and removes it.
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                        int* __restrict__ idx, float* __restrict__ gate) {
  constexpr int PER = MOE_MAX_E / 64;
  constexpr int NONE = 0x7fffffff;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* lg = logits + (int64_t)t * E;
  const int per = (E + 63) / 64;  // register slots in use (uniform)
  float v[PER];
  uint32_t live = 0;  // bit q: value q of this lane is still a candidate
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    if (q >= per) break;
    const int e = lane + 64 * q;
    const float x = e < E ? lg[e] : -INFINITY;
    v[q] = x != x ? -INFINITY : x;
    if (e < E) live |= 1u << q;
  }
  float my_val = -INFINITY;  // lane j keeps pass j's pick
  int my_sel = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = NONE;
#pragma unroll
    for (int q = 0; q < PER; ++q) {  // indices rise with q: strict > keeps the lower on ties
      if (q >= per) break;
      if ((live >> q & 1u) && (be == NONE || v[q] > bv)) {
        bv = v[q];
        be = lane + 64 * q;
      }
    }
    // butterfly over the wave: every step pairs each lane with a partner
    // whose group has not been merged yet, so all lanes end with the same
    // (value, index); the first four steps are DPP lane permutations (xor 1
    // and xor 2 inside quads, then the half-row and row mirrors)
    dpp_take<0xB1>(bv, be);   // quad_perm [1, 0, 3, 2]
    dpp_take<0x4E>(bv, be);   // quad_perm [2, 3, 0, 1]
    dpp_take<0x141>(bv, be);  // row_half_mirror
    dpp_take<0x140>(bv, be);  // row_mirror
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) take(bv, be, __shfl_xor(bv, off), __shfl_xor(be, off));
    if (lane == j) {
      my_val = bv;
      my_sel = be;
    }
    if ((be & 63) == lane) live &= ~(1u << (be >> 6));
  }
  // gates: exponentials relative to the largest pick, normalised over the k
  const float top = __shfl(my_val, 0);
  const float w = lane < k ? expf(my_val - top) : 0.0f;
  float sum = w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    idx[(int64_t)t * k + lane] = my_sel;
    gate[(int64_t)t * k + lane] = w / sum;
  }
}

// One workgroup plans the grouping: per-expert counts (an LDS histogram of
// idx; indices outside [0, E) are skipped here and in the scatter, so such a
// slot contributes nothing), every expert's group padded to whole tiles
// (exclusive scan), the tile -> expert table, cleared cursors, and the padding
// rows of each group marked empty (every other row of an active tile is
// written by the scatter; tiles past the last group are never read).
__global__ __launch_bounds__(1024) void moe_plan_kernel(const int* __restrict__ idx, int n, int E,
                                                        int* __restrict__ offsets, int* __restrict__ cursors,
                                                        int* __restrict__ tile_expert, int n_tiles,
                                                        int* __restrict__ src_row, int* __restrict__ dst_slot) {
  __shared__ int cnt[MOE_MAX_E];
  __shared__ int s_off[MOE_MAX_E + 1];
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();
  for (int i0 = 0; i0 < n; i0 += 1024 * 16) {  // 16 loads in flight per thread, then the LDS atomics
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u * 1024 + tid;
      v[u] = i < n ? idx[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (v[u] >= 0 && v[u] < E) atomicAdd(&cnt[v[u]], 1);
  }
  __syncthreads();
  // exclusive scan of the padded sizes, one expert per thread (E <= 1024)
  const int c = tid < E ? cnt[tid] : 0;
  const int padded = (c + MOE_TILE - 1) / MOE_TILE * MOE_TILE;
  int incl = padded;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const int start = before + incl - padded;
  if (tid < E) {
    s_off[tid] = start;
    offsets[tid] = start;
    cursors[tid] = 0;
  }
  if (tid == E - 1) {
    s_off[E] = start + padded;
    offsets[E] = start + padded;
  }
  __syncthreads();
  for (int tl = tid; tl < n_tiles; tl += 1024) {
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
  // padding rows: each expert's last (padded - count) rows, one wave per expert
  for (int e = wave; e < E; e += 16) {
    const int first = s_off[e] + cnt[e];
    for (int r = first + lane; r < s_off[e + 1]; r += 64) {
      src_row[r] = -1;
      dst_slot[r] = -1;
    }
  }
}

// Each workgroup (SCATTER_PER entries) counts its entries per expert in LDS,
// reserves one block per expert with a single global atomic, then hands out
// rows inside the block with LDS atomics.
__global__ __launch_bounds__(256) void moe_scatter_kernel(const int* __restrict__ idx, int n, int k, int E,
                                                          const int* __restrict__ offsets, int* __restrict__ cursors,
                                                          int* __restrict__ src_row, int* __restrict__ dst_slot,
                                                          int* __restrict__ pos_of) {
  __shared__ int h[MOE_MAX_E];
  __shared__ int base[MOE_MAX_E];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int lo = blockIdx.x * SCATTER_PER, hi = min(n, lo + SCATTER_PER);
  for (int i = lo + threadIdx.x; i < hi; i += 256) {
    const int e = idx[i];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    base[e] = h[e] ? offsets[e] + atomicAdd(&cursors[e], h[e]) : 0;
    h[e] = 0;
  }
  __syncthreads();
  for (int i = lo + threadIdx.x; i < hi; i += 256) {
    const int e = idx[i];
    if (e < 0 || e >= E) {
      pos_of[i] = -1;
      continue;
    }
    const int pos = base[e] + atomicAdd(&h[e], 1);
    src_row[pos] = i / k;
    dst_slot[pos] = i;
    pos_of[i] = pos;
  }
}

// xs[r] = x[src_row[r]] (zero for padding rows) for the rows of the groups
// (r < *used; later rows are never read); d % 8 == 0, 16-byte rows.
__global__ __launch_bounds__(256) void moe_gather_kernel(const uint4* __restrict__ x, const int* __restrict__ src_row,
                                                         const int* __restrict__ used, int rows, int d8,
                                                         uint4* __restrict__ xs) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)rows * d8) return;
  const int r = (int)(i / d8), c = (int)(i % d8);
  if (r >= *used) return;
  const int s = src_row[r];
  xs[i] = s >= 0 ? x[(int64_t)s * d8 + c] : make_uint4(0u, 0u, 0u, 0u);
}

// y[t, c] = sum_j gate[t, j] * zs[t k + j, c] in slot order (fp32), over
// the slots that were routed (pos_of >= 0); four columns per thread
// (d % 8 == 0).  zs holds fp32 or bf16 rows (ZT).
__device__ __forceinline__ float4 load4(const float* z) { return *reinterpret_cast<const float4*>(z); }
__device__ __forceinline__ float4 load4(const uint16_t* z) {
  const uint2 w = *reinterpret_cast<const uint2*>(z);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xffff0000u));
}

template <typename ZT, typename OutT>
__global__ __launch_bounds__(256) void moe_combine_kernel(const ZT* __restrict__ zs, const int* __restrict__ pos_of,
                                                          const float* __restrict__ gate, int T, int k, int d,
                                                          OutT* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int d4 = d / 4;
  if (i >= (int64_t)T * d4) return;
  const int t = (int)(i / d4), c = (int)(i % d4) * 4;
  float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j = 0; j < k; ++j) {
    if (pos_of[(int64_t)t * k + j] < 0) continue;
    const float g = gate[(int64_t)t * k + j];
    const float4 z = load4(zs + ((int64_t)t * k + j) * d + c);
    s.x += g * z.x;
    s.y += g * z.y;
    s.z += g * z.z;
    s.w += g * z.w;
  }
  if constexpr (std::is_same<OutT, float>::value) {
    *reinterpret_cast<float4*>(y + (int64_t)t * d + c) = s;
  } else {
    uint2 o;
    o.x = f2bf2(s.x, s.y);
    o.y = f2bf2(s.z, s.w);
    *reinterpret_cast<uint2*>(y + (int64_t)t * d + c) = o;
  }
}

unsigned blocks(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t moe_route(const float* logits, int T, int E, int k, int* idx, float* gate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_route_kernel, dim3(blocks(T, 4)), dim3(256), 0, s, logits, T, E, k, idx, gate);
  return hipGetLastError();
}

hipError_t moe_group(const int* idx, int T, int E, int k, const void* x, int d, int rows, int n_tiles, int* offsets,
                     int* cursors, int* tile_expert, int* src_row, int* dst_slot, int* pos_of, void* xs, hipStream_t s) {
  const int n = T * k;
  hipLaunchKernelGGL(moe_plan_kernel, dim3(1), dim3(1024), 0, s, idx, n, E, offsets, cursors, tile_expert, n_tiles,
                     src_row, dst_slot);
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(blocks(n, SCATTER_PER)), dim3(256), 0, s, idx, n, k, E, offsets, cursors,
                     src_row, dst_slot, pos_of);
  if (!xs) return hipGetLastError();  // the GEMM reads x through src_row
  const int64_t units = (int64_t)rows * (d / 8);
  hipLaunchKernelGGL(moe_gather_kernel, dim3(blocks(units, 256)), dim3(256), 0, s, reinterpret_cast<const uint4*>(x),
                     src_row, offsets + E, rows, d / 8, reinterpret_cast<uint4*>(xs));
  return hipGetLastError();
}

hipError_t moe_combine(const void* zs, bool zs_f32, const int* pos_of, const float* gate, int T, int k, int d,
                       void* y, bool out_f32, hipStream_t s) {
  const int64_t n = (int64_t)T * (d / 4);
  if (n == 0) return hipSuccess;
  const dim3 grid(blocks(n, 256));
  if (zs_f32 && out_f32)
    hipLaunchKernelGGL((moe_combine_kernel<float, float>), grid, dim3(256), 0, s, reinterpret_cast<const float*>(zs),
                       pos_of, gate, T, k, d, reinterpret_cast<float*>(y));
  else if (zs_f32)
    hipLaunchKernelGGL((moe_combine_kernel<float, uint16_t>), grid, dim3(256), 0, s,
                       reinterpret_cast<const float*>(zs), pos_of, gate, T, k, d, reinterpret_cast<uint16_t*>(y));
  else if (out_f32)
    hipLaunchKernelGGL((moe_combine_kernel<uint16_t, float>), grid, dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(zs), pos_of, gate, T, k, d, reinterpret_cast<float*>(y));
  else
    hipLaunchKernelGGL((moe_combine_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(zs), pos_of, gate, T, k, d, reinterpret_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace tpk
