// fp32 GEMM (vector ALU, LDS-tiled) for the fp32 variant of the shard ops.
//
// Same contraction and epilogues as the bf16 MFMA kernels (see
// gemm_bf16.hip); used when the caller asks for fp32 throughout, where bf16
// operand rounding would not meet an fp32 tolerance.  It is a correctness
// path for small fp32 problems, not a tuned one: 64x64 output tiles, each of
// 256 threads owning a 4x4 block, K staged 16 at a time through LDS.
#include "tp_kernels.h"
#include "tp_device.h"

namespace tpk {

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmParams p, int akc, int bkc, int dual) {
  constexpr int TB = 64, TK = 16;
  __shared__ float As[TK][TB + 1];
  __shared__ float Bs[2][TK][TB + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * TB, n0 = blockIdx.x * TB;
  float acc0[4][4], acc1[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) { acc0[i][j] = 0.f; acc1[i][j] = 0.f; }

  const int nseg = (dual || p.K1 == 0) ? 1 : 2;
  for (int seg = 0; seg < nseg; ++seg) {
    const int K = seg ? p.K1 : p.K0;
    const float* A = reinterpret_cast<const float*>(seg ? p.A1 : p.A0);
    const float* B0 = reinterpret_cast<const float*>(seg ? p.B1 : p.B0);
    const float* B1 = reinterpret_cast<const float*>(p.B1);
    for (int k0 = 0; k0 < K; k0 += TK) {
      for (int e = tid; e < TB * TK; e += 256) {
        const int mm = e / TK, kk = e % TK;
        const int gm = m0 + mm, gk = k0 + kk;
        float v = 0.f;
        if (gm < p.M && gk < K) v = akc ? A[(int64_t)gm * p.lda + gk] : A[(int64_t)gk * p.lda + gm];
        As[kk][mm] = v;
      }
      for (int e = tid; e < TB * TK; e += 256) {
        const int kk = e / TB, nn = e % TB;
        const int gn = n0 + nn, gk = k0 + kk;
        float v0 = 0.f, v1 = 0.f;
        if (gn < p.N && gk < K) {
          const int64_t off = bkc ? (int64_t)gn * p.ldb + gk : (int64_t)gk * p.ldb + gn;
          v0 = B0[off];
          if (dual) v1 = B1[off];
        }
        Bs[0][kk][nn] = v0;
        Bs[1][kk][nn] = v1;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < TK; ++kk) {
        float a[4], b0[4], b1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) { b0[j] = Bs[0][kk][tx * 4 + j]; b1[j] = Bs[1][kk][tx * 4 + j]; }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc0[i][j] = fmaf(a[i], b0[j], acc0[i][j]);
            acc1[i][j] = fmaf(a[i], b1[j], acc1[i][j]);
          }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < p.M && n < p.N) epilogue_elem<EPI, float, float>(p, m, n, acc0[i][j], acc1[i][j]);
    }
}

template <int EPI>
static hipError_t launch_f32(const GemmParams& p, int akc, int bkc, int dual, hipStream_t s) {
  dim3 grid((p.N + 63) / 64, (p.M + 63) / 64);
  hipLaunchKernelGGL(gemm_f32_kernel<EPI>, grid, dim3(256), 0, s, p, akc, bkc, dual);
  return hipGetLastError();
}

hipError_t gemm_f32(const GemmParams& p, GemmKind kind, hipStream_t s) {
  switch (kind) {
    case GK_FWD_STORE: return launch_f32<EPI_STORE>(p, 1, 0, 0, s);
    case GK_FWD_ACT: return launch_f32<EPI_ACT>(p, 1, 0, 0, s);
    case GK_FWD_SWIGLU: return launch_f32<EPI_SWIGLU>(p, 1, 0, 1, s);
    case GK_BWD_DH_SWIGLU: return launch_f32<EPI_SWIGLU_BWD>(p, 1, 1, 0, s);
    case GK_BWD_DH_ACT: return launch_f32<EPI_ACT_BWD>(p, 1, 1, 0, s);
    case GK_BWD_DW: return launch_f32<EPI_STORE>(p, 0, 0, 0, s);
    case GK_BWD_DW_DUAL: return launch_f32<EPI_DUAL_STORE>(p, 0, 0, 1, s);
    case GK_BWD_DX: return launch_f32<EPI_STORE>(p, 1, 1, 0, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpk
