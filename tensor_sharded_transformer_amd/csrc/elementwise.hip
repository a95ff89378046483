// Elementwise kernels: activation on owned columns, the sum of the p
// full-shape partials, and a workspace zero-fill.
//
// Activation: "How does tensor parallelism split a transformer feed-forward
// block's two matmuls across devices?", "The nonlinearity is free" (an
// elementwise function of each owned column, no communication).
// Sum of partials: "Tensor Parallelism" notes, first paragraph (Y = sum_i Z_i,
// an all-reduce in a real group) and the MLX shard_linear facts (the bias is
// added once, after the sum).
//
// All three are HBM-bound streams: each thread moves 16-byte vectors, the grid
// is sized to a few waves of workgroups per CU and loops grid-stride.
#include <algorithm>
#include <type_traits>

#include "tp_kernels.h"
#include "tp_device.h"

namespace tpk {

static int stream_grid(int64_t units, int block) {
  int64_t g = (units + block - 1) / block;
  const int64_t cap = 256 * 16;  // 256 CUs x 16 workgroups: enough bytes in flight
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

// ---- activation in place ----------------------------------------------------
__global__ __launch_bounds__(256) void act_bf16_kernel(uint16_t* h, const uint16_t* up, int64_t n, int act, int vec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t nv = vec ? n / 8 : 0;
  for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < nv; v += stride) {
    uint4 hv = reinterpret_cast<const uint4*>(h)[v];
    uint4 uv = make_uint4(0, 0, 0, 0);
    if (act == ACT_SWIGLU) uv = reinterpret_cast<const uint4*>(up)[v];
    uint32_t* hw = reinterpret_cast<uint32_t*>(&hv);
    const uint32_t* uw = reinterpret_cast<const uint32_t*>(&uv);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a0 = bf2f((uint16_t)(hw[q] & 0xffffu)), a1 = bf2f((uint16_t)(hw[q] >> 16));
      if (act == ACT_SWIGLU) {
        const float u0 = bf2f((uint16_t)(uw[q] & 0xffffu)), u1 = bf2f((uint16_t)(uw[q] >> 16));
        a0 = a0 * sigmoidf_(a0) * u0;
        a1 = a1 * sigmoidf_(a1) * u1;
      } else {
        a0 = act_fwd(act, a0);
        a1 = act_fwd(act, a1);
      }
      hw[q] = f2bf2(a0, a1);
    }
    reinterpret_cast<uint4*>(h)[v] = hv;
  }
  // scalar tail (or everything when not 16-byte aligned)
  for (int64_t e = nv * 8 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += stride) {
    float a = bf2f(h[e]);
    if (act == ACT_SWIGLU) a = a * sigmoidf_(a) * bf2f(up[e]);
    else a = act_fwd(act, a);
    h[e] = f2bf(a);
  }
}

__global__ __launch_bounds__(256) void act_f32_kernel(float* h, const float* up, int64_t n, int act) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += stride) {
    float a = h[e];
    if (act == ACT_SWIGLU) a = a * sigmoidf_(a) * up[e];
    else a = act_fwd(act, a);
    h[e] = a;
  }
}

hipError_t act_inplace(void* h, const void* up, int64_t n, bool bf16, int act, hipStream_t s) {
  if (n == 0 || act == ACT_NONE) return hipSuccess;
  if (bf16) {
    const int vec = ((uintptr_t)h % 16 == 0) && (up == nullptr || (uintptr_t)up % 16 == 0);
    hipLaunchKernelGGL(act_bf16_kernel, dim3(stream_grid(vec ? (n + 7) / 8 : n, 256)), dim3(256), 0, s,
                       (uint16_t*)h, (const uint16_t*)up, n, act, vec);
  } else {
    hipLaunchKernelGGL(act_f32_kernel, dim3(stream_grid(n, 256)), dim3(256), 0, s, (float*)h, (const float*)up, n,
                       act);
  }
  return hipGetLastError();
}

// ---- sum of partials ----------------------------------------------------------
constexpr int MAX_P = 64;
struct SumArgs {
  const void* z[MAX_P];
};

template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void partial_sum_kernel(const SumArgs a, int p, const void* bias, void* y,
                                                          int64_t T, int64_t N, int vec) {
  const int64_t n = T * N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // 8 elements per thread per step when every row start is 16-byte aligned
  // for bf16 (32 bytes for f32 in two 16-byte halves).
  if (vec) {
    const int64_t nv = n / 8;
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < nv; v += stride) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
      // the partials in batches of 8: a batch's loads are all issued before
      // the first is added (one memory round trip per batch, not per
      // partial), then added in ascending i
      for (int i0 = 0; i0 < p; i0 += 8) {
        const int nb = p - i0 < 8 ? p - i0 : 8;
        if constexpr (IN_BF16) {
          uint4 w[8];  // unconditional loads (straight-line code); slots past p re-read partial i0
#pragma unroll
          for (int b = 0; b < 8; ++b) w[b] = reinterpret_cast<const uint4*>(a.z[i0 + (b < nb ? b : 0)])[v];
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            if (b < nb) {
              const uint32_t ww[4] = {w[b].x, w[b].y, w[b].z, w[b].w};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                acc[2 * q] += bf2f((uint16_t)(ww[q] & 0xffffu));
                acc[2 * q + 1] += bf2f((uint16_t)(ww[q] >> 16));
              }
            }
          }
        } else {
          float4 w0[8], w1[8];
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const float4* z = reinterpret_cast<const float4*>(a.z[i0 + (b < nb ? b : 0)]);
            w0[b] = z[2 * v];
            w1[b] = z[2 * v + 1];
          }
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            if (b < nb) {
              acc[0] += w0[b].x; acc[1] += w0[b].y; acc[2] += w0[b].z; acc[3] += w0[b].w;
              acc[4] += w1[b].x; acc[5] += w1[b].y; acc[6] += w1[b].z; acc[7] += w1[b].w;
            }
          }
        }
      }
      if (bias) {
        const int64_t col = (v * 8) % N;  // N % 8 == 0 on this path
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (IN_BF16) acc[e] += bf2f(reinterpret_cast<const uint16_t*>(bias)[col + e]);
          else acc[e] += reinterpret_cast<const float*>(bias)[col + e];
        }
      }
      if constexpr (OUT_BF16) {
        uint4 o;
        o.x = f2bf2(acc[0], acc[1]);
        o.y = f2bf2(acc[2], acc[3]);
        o.z = f2bf2(acc[4], acc[5]);
        o.w = f2bf2(acc[6], acc[7]);
        reinterpret_cast<uint4*>(y)[v] = o;
      } else {
        reinterpret_cast<float4*>(y)[2 * v] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        reinterpret_cast<float4*>(y)[2 * v + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
      }
    }
    return;
  }
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += stride) {
    float acc = 0.f;
    for (int i = 0; i < p; ++i) {
      if constexpr (IN_BF16) acc += bf2f(reinterpret_cast<const uint16_t*>(a.z[i])[e]);
      else acc += reinterpret_cast<const float*>(a.z[i])[e];
    }
    if (bias) {
      if constexpr (IN_BF16) acc += bf2f(reinterpret_cast<const uint16_t*>(bias)[e % N]);
      else acc += reinterpret_cast<const float*>(bias)[e % N];
    }
    if constexpr (OUT_BF16) reinterpret_cast<uint16_t*>(y)[e] = f2bf(acc);
    else reinterpret_cast<float*>(y)[e] = acc;
  }
}

hipError_t partial_sum(const void* const* z, int p, const void* bias, void* y, int64_t T, int64_t N, bool in_bf16,
                       bool out_bf16, hipStream_t s) {
  if (T == 0 || N == 0) return hipSuccess;
  SumArgs a{};
  bool aligned = ((uintptr_t)y % 16 == 0) && (N % 8 == 0);
  for (int i = 0; i < p; ++i) {
    a.z[i] = z[i];
    aligned = aligned && ((uintptr_t)z[i] % 16 == 0);
  }
  const int vec = aligned ? 1 : 0;
  const int grid = stream_grid(vec ? (T * N) / 8 : T * N, 256);
  if (in_bf16 && out_bf16)
    hipLaunchKernelGGL((partial_sum_kernel<true, true>), dim3(grid), dim3(256), 0, s, a, p, bias, y, T, N, vec);
  else if (in_bf16)
    hipLaunchKernelGGL((partial_sum_kernel<true, false>), dim3(grid), dim3(256), 0, s, a, p, bias, y, T, N, vec);
  else if (out_bf16)
    hipLaunchKernelGGL((partial_sum_kernel<false, true>), dim3(grid), dim3(256), 0, s, a, p, bias, y, T, N, vec);
  else
    hipLaunchKernelGGL((partial_sum_kernel<false, false>), dim3(grid), dim3(256), 0, s, a, p, bias, y, T, N, vec);
  return hipGetLastError();
}

// ---- sequence-parallel boundary: reduce-scatter share + residual add + RMSNorm -------
// One workgroup per owned row, sized to the row (up to 1024 threads, one
// 8-column group each) so all of a row's loads are in flight together.  Pass 1 sums the p partials (ascending i), the
// bias and the residual in fp32, keeps the row in LDS, writes residual_out and
// accumulates the sum of squares; the block reduces it; pass 2 scales the LDS
// row by 1/sqrt(mean + eps) and norm_w.  8 columns per thread per step (16-byte
// loads) when every row start is 16-byte aligned, else one.
template <typename InT, typename OutT>
__device__ __forceinline__ float ld1(const void* p, int64_t i) {
  if constexpr (std::is_same<InT, uint16_t>::value) return bf2f(reinterpret_cast<const uint16_t*>(p)[i]);
  else return reinterpret_cast<const float*>(p)[i];
}
template <typename T>
__device__ __forceinline__ void st1(void* p, int64_t i, float v) {
  if constexpr (std::is_same<T, uint16_t>::value) reinterpret_cast<uint16_t*>(p)[i] = f2bf(v);
  else reinterpret_cast<float*>(p)[i] = v;
}
// 8 consecutive values from a 16-byte aligned address (bf16: one 16-byte load; f32: two)
template <typename T>
__device__ __forceinline__ void ld8(const void* p, int64_t i, float (&v)[8]) {
  if constexpr (std::is_same<T, uint16_t>::value) {
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + i);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf2f((uint16_t)(ww[q] & 0xffffu));
      v[2 * q + 1] = bf2f((uint16_t)(ww[q] >> 16));
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}
template <typename T>
__device__ __forceinline__ void st8(void* p, int64_t i, const float (&v)[8]) {
  if constexpr (std::is_same<T, uint16_t>::value) {
    uint4 o;
    o.x = f2bf2(v[0], v[1]);
    o.y = f2bf2(v[2], v[3]);
    o.z = f2bf2(v[4], v[5]);
    o.w = f2bf2(v[6], v[7]);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p) + i) = o;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p) + i) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p) + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <typename InT, typename OutT>
__global__ __launch_bounds__(1024) void rs_norm_kernel(const SumArgs a, int p, int64_t row0, const void* bias,
                                                      const void* res_in, const void* norm_w, float eps,
                                                      void* res_out, void* y, int64_t N, int vec) {
  extern __shared__ float srow[];  // the row's fp32 sums
  __shared__ float wsum[16];
  const int nt = blockDim.x;
  const int64_t r = blockIdx.x;    // owned row
  const int64_t zrow = (row0 + r) * N, orow = r * N;
  float ss = 0.f;
  if (vec) {
    for (int64_t c = threadIdx.x * 8; c < N; c += nt * 8) {
      float s[8], t[8];
      ld8<OutT>(res_in, orow + c, s);
      for (int i = 0; i < p; ++i) {
        ld8<InT>(a.z[i], zrow + c, t);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += t[e];
      }
      if (bias) {
        ld8<InT>(bias, c, t);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += t[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        srow[c + e] = s[e];
        ss += s[e] * s[e];
      }
      st8<OutT>(res_out, orow + c, s);
    }
  } else {
    for (int64_t c = threadIdx.x; c < N; c += nt) {
      float s = ld1<OutT, OutT>(res_in, orow + c);
      for (int i = 0; i < p; ++i) s += ld1<InT, InT>(a.z[i], zrow + c);
      if (bias) s += ld1<InT, InT>(bias, c);
      srow[c] = s;
      ss += s * s;
      st1<OutT>(res_out, orow + c, s);
    }
  }
  // block sum of squares: wave shuffles, then the four wave totals in wave order
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();  // also orders the srow writes before pass 2
  float tot = 0.f;
  for (int w = 0; w < nt / 64; ++w) tot += wsum[w];  // in wave order
  const float inv = 1.0f / sqrtf(tot / (float)N + eps);
  if (vec) {
    for (int64_t c = threadIdx.x * 8; c < N; c += nt * 8) {
      float w[8], o[8];
      ld8<OutT>(norm_w, c, w);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = srow[c + e] * inv * w[e];
      st8<OutT>(y, orow + c, o);
    }
  } else {
    for (int64_t c = threadIdx.x; c < N; c += nt) st1<OutT>(y, orow + c, srow[c] * inv * ld1<OutT, OutT>(norm_w, c));
  }
}

hipError_t rs_residual_rmsnorm(const void* const* z, int p, int rank, const void* bias, const void* residual_in,
                               const void* norm_w, float eps, void* residual_out, void* y, int64_t T, int64_t N,
                               bool in_bf16, bool out_bf16, hipStream_t s) {
  const int64_t rows = T / p;
  if (rows == 0 || N == 0) return hipSuccess;
  SumArgs a{};
  bool aligned = N % 8 == 0;
  for (int i = 0; i < p; ++i) {
    a.z[i] = z[i];
    aligned = aligned && (uintptr_t)z[i] % 16 == 0;
  }
  for (const void* q : {residual_in, norm_w, (const void*)residual_out, (const void*)y, bias})
    aligned = aligned && (q == nullptr || (uintptr_t)q % 16 == 0);
  const int vec = aligned ? 1 : 0;
  const size_t lds = (size_t)N * sizeof(float);
  const int64_t groups = vec ? (N + 7) / 8 : N;  // work items of a row
  const int nt = (int)std::min<int64_t>(1024, std::max<int64_t>(64, (groups + 63) / 64 * 64));
  const int64_t row0 = (int64_t)rank * rows;
  if (lds > 48 * 1024) {  // more dynamic LDS than the default limit: raise it for this kernel
    hipError_t e = hipSuccess;
    if (in_bf16 && out_bf16)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(rs_norm_kernel<uint16_t, uint16_t>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    else if (in_bf16)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(rs_norm_kernel<uint16_t, float>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    else if (out_bf16)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(rs_norm_kernel<float, uint16_t>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    else
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(rs_norm_kernel<float, float>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (in_bf16 && out_bf16)
    hipLaunchKernelGGL((rs_norm_kernel<uint16_t, uint16_t>), dim3(rows), dim3(nt), lds, s, a, p, row0, bias,
                       residual_in, norm_w, eps, residual_out, y, N, vec);
  else if (in_bf16)
    hipLaunchKernelGGL((rs_norm_kernel<uint16_t, float>), dim3(rows), dim3(nt), lds, s, a, p, row0, bias,
                       residual_in, norm_w, eps, residual_out, y, N, vec);
  else if (out_bf16)
    hipLaunchKernelGGL((rs_norm_kernel<float, uint16_t>), dim3(rows), dim3(nt), lds, s, a, p, row0, bias,
                       residual_in, norm_w, eps, residual_out, y, N, vec);
  else
    hipLaunchKernelGGL((rs_norm_kernel<float, float>), dim3(rows), dim3(nt), lds, s, a, p, row0, bias, residual_in,
                       norm_w, eps, residual_out, y, N, vec);
  return hipGetLastError();
}

// ---- zero fill --------------------------------------------------------------------
__global__ __launch_bounds__(256) void zero_kernel(char* p, size_t bytes, int vec) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t nv = vec ? bytes / 16 : 0;
  for (size_t v = blockIdx.x * (size_t)blockDim.x + threadIdx.x; v < nv; v += stride)
    reinterpret_cast<uint4*>(p)[v] = make_uint4(0, 0, 0, 0);
  for (size_t e = nv * 16 + blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < bytes; e += stride) p[e] = 0;
}

hipError_t zero_fill(void* ws, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const int vec = ((uintptr_t)ws % 16 == 0) ? 1 : 0;
  const int64_t units = vec ? (int64_t)(bytes / 16) + 1 : (int64_t)bytes;
  hipLaunchKernelGGL(zero_kernel, dim3(stream_grid(units, 256)), dim3(256), 0, s, (char*)ws, bytes, vec);
  return hipGetLastError();
}

// fp8 weight codes (K, N) row-major -> 64-column strip-major: one thread per
// 16-byte piece of a strip row.
__global__ __launch_bounds__(256) void pack_strips_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                          int64_t K, int64_t N) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // piece index in destination order
  const int64_t pieces = K * (N / 16);
  if (i >= pieces) return;
  const int64_t strip = i / (K * 4), rem = i % (K * 4);
  const int64_t k = rem / 4, q = rem % 4;
  const uint4 v = *reinterpret_cast<const uint4*>(src + k * N + strip * 64 + q * 16);
  *reinterpret_cast<uint4*>(dst + i * 16) = v;
}

hipError_t pack_fp8_strips(const void* src, void* dst, int64_t K, int64_t N, hipStream_t s) {
  const int64_t pieces = K * (N / 16);
  if (pieces == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_strips_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(src), reinterpret_cast<uint8_t*>(dst), K, N);
  return hipGetLastError();
}

}  // namespace tpk
