// Device-side helpers shared by the tpshard kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tpk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Epilogue kinds of the GEMM kernels.
enum Epi : int {
  EPI_STORE = 0,       // C = acc
  EPI_ACT = 1,         // a = acc (+ bias); C2 <- a (optional); C = act(a)
  EPI_SWIGLU = 2,      // dual: C2 <- g, C3 <- u (optional); C = silu(g) * u
  EPI_DUAL_STORE = 3,  // dual: C = acc0, C2 = acc1
  EPI_SWIGLU_BWD = 4,  // acc = dh; g = S0, u = S1: C = dh*u*silu'(g), C2 = dh*silu(g), C3 = silu(g)*u
  EPI_ACT_BWD = 5,     // acc = dh; a = S0: C = dh*act'(a), C3 = act(a)
};

enum ActKind : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2, ACT_SWIGLU = 3 };

// fp32 -> bf16 with round-to-nearest-even (NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
// Two floats to two bf16 (lo in bits 0-15) with the hardware conversion
// (v_cvt_pk_bf16_f32: round to nearest even, one instruction for the pair).
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// Activations in fp32 (exact erf GELU; silu(g) = g * sigmoid(g)).
// 1 / (1 + e^-g) from the hardware 2^x and reciprocal (v_exp_f32, v_rcp_f32,
// about 1 ulp each, far inside the bf16 rounding of every value it feeds);
// g -> -inf gives 0, g -> +inf gives 1, NaN stays NaN.
__device__ __forceinline__ float sigmoidf_(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896341f));
}
__device__ __forceinline__ float act_fwd(int act, float a) {
  if (act == ACT_RELU) return a > 0.0f ? a : 0.0f;
  if (act == ACT_GELU) return 0.5f * a * (1.0f + erff(a * 0.70710678118654752f));
  return a;
}
__device__ __forceinline__ float act_grad(int act, float a) {
  if (act == ACT_RELU) return a > 0.0f ? 1.0f : 0.0f;
  if (act == ACT_GELU) {
    const float cdf = 0.5f * (1.0f + erff(a * 0.70710678118654752f));
    const float pdf = 0.39894228040143268f * expf(-0.5f * a * a);
    return cdf + a * pdf;
  }
  return 1.0f;
}

// Parameters shared by the bf16 MFMA GEMM and the fp32 GEMM.
//   C[m, n] = sum_k A(m, k) B(k, n)
// A(m, k) is A[m*lda + k] when A is k-contiguous, else A[k*lda + m].
// B(k, n) is B[n*ldb + k] when B is k-contiguous, else B[k*ldb + n].
// Two K segments (seg 0 then seg 1) let dx = dG W1^T + dU Wup^T run as one
// GEMM; in dual mode B0 and B1 are two B matrices over the same K that give
// two accumulators per output element (gate and up).
struct GemmParams {
  const void* A0;
  const void* A1;
  const void* B0;
  const void* B1;
  int64_t lda, ldb;
  int K0, K1;
  int M, N;            // output rows / columns (columns of ONE B in dual mode)
  void* C;
  void* C2;
  void* C3;
  int64_t ldc, ldc2, ldc3;
  const void* S0;
  const void* S1;
  int64_t lds;
  const void* bias;    // per-column bias (EPI_ACT only), may be null
  int act;
  int vecA, vecB;      // 16-byte vector loads allowed for A / B
  int splitk;          // number of K splits (>= 1)
  float* partials;     // split-K fp32 partial tiles
  int* counters;       // split-K arrival counters (zero on entry, left zero)
  void* apk;           // decode kernel: A in MFMA fragment order (workspace)
  int apk_ready;       // decode kernel: apk already holds A (skip the packing pass)
  void* cpk;           // if set: the bf16 output goes here, in the packed A
  int cpk_mt;          //   layout of a decode GEMM with cpk_mt 32-row tiles, instead of to C
  int split_base;      // decode kernel: K splits of a column strip (splitk = split slots per tile) ...
  int slow_first;      //   ... except strips slow_first + 8j (weight bytes of the slow address class),
  int slow_extra;      //   which get slow_extra more
  int b_fp8;           // decode kernel: B0/B1 hold fp8 (OCP e4m3) codes, ldb in elements (= bytes) ...
  const float* bscale0;  //   ... with per-column scales applied to the sums (B0)
  const float* bscale1;  //   (B1)
  const int* tile_expert;   // tiled kernel, grouped mode: expert of each BM-row tile (-1: no rows) ...
  int64_t b_expert_stride;  //   ... whose B0/B1 start this many elements further per expert index
  const int* a_rows;        // tiled kernel, k-contiguous A only: the A row of each output row (-1: a zero
                            //   row), A0 pointing at row 0; A's bytes must stay below 2^31
  const int* c_rows;        // tiled kernel, EPI_STORE: the C row each output row is stored to (-1: not stored)
};

// Calls f(integral_constant<int, I>) for I = 0 .. N-1, so array indices in
// f are compile-time constants (keeps the prefetch ring in registers).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Renumber workgroups so that each XCD gets a contiguous range of ids.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  if (nblk < 8) return bid;
  const int xcd = bid & 7;
  const int idx = bid >> 3;
  const int per = nblk >> 3;
  const int rem = nblk & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// ---- split-K exchange ------------------------------------------------------
// Partial tiles move through the workspace with 16-byte buffer operations
// carrying the agent-scope coherence bit (sc1): they are coherent across the
// XCDs' separate L2 caches without flushing or invalidating them.  The
// buffer's byte bound makes out-of-range reads return 0.
typedef float f32x4v __attribute__((ext_vector_type(4)));
constexpr int CPOL_SC1 = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t splitk_rsrc(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void splitk_store(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4v v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CPOL_SC1);
}
__device__ __forceinline__ f32x4v splitk_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL_SC1);
}

// Split-K exchange for one wave's tile of NACC accumulators (tile t of the
// launch, split `split`): publish this split's partial, take an arrival
// ticket, and if this was the last split to arrive, replace acc by the sum of
// all splits in split order and re-zero the ticket.  Returns false for the
// splits that are not last (they have nothing left to do).  Layout per tile:
// [split][acc][quarter][lane][4 floats], so every store and load is 1 KB
// contiguous per wave.
// A tile may have fewer splits (nsplit) than the p.splitk slots it is laid
// out with.
template <int NACC>
__device__ __forceinline__ bool splitk_exchange(const GemmParams& p, int t, int split, int nsplit, int lane,
                                                f32x16* acc) {
  constexpr uint32_t SPLIT_BYTES = NACC * 16 * 64 * 4;
  const float* base = p.partials + (int64_t)t * p.splitk * NACC * 16 * 64;
  const __amdgpu_buffer_rsrc_t r = splitk_rsrc(base, SPLIT_BYTES * (uint32_t)nsplit);
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4v v = {acc[a][4 * q], acc[a][4 * q + 1], acc[a][4 * q + 2], acc[a][4 * q + 3]};
      splitk_store(r, split * SPLIT_BYTES + ((a * 4 + q) * 64 + lane) * 16, v);
    }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this lane's partial stores are complete
  __builtin_amdgcn_wave_barrier();
  int prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(&p.counters[t], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0);
  if (prev != nsplit - 1) return false;
  // Every split has arrived: load the splits' values in batches of SB splits
  // (all accumulators of a batch issued together, about 32 loads per lane)
  // and add them in split order.
  constexpr int SB = NACC >= 8 ? 1 : 8 / NACC;
  f32x16 sum[NACC];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum[a][e] = 0.0f;
  for (int s0 = 0; s0 < nsplit; s0 += SB) {
    f32x4v v[SB][NACC][4];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int a = 0; a < NACC; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[sb][a][q] = splitk_load(r, (s0 + sb) * SPLIT_BYTES + ((a * 4 + q) * 64 + lane) * 16);
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int a = 0; a < NACC; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sum[a][4 * q] += v[sb][a][q][0];
          sum[a][4 * q + 1] += v[sb][a][q][1];
          sum[a][4 * q + 2] += v[sb][a][q][2];
          sum[a][4 * q + 3] += v[sb][a][q][3];
        }
  }
#pragma unroll
  for (int a = 0; a < NACC; ++a) acc[a] = sum[a];
  if (lane == 0) __hip_atomic_store(&p.counters[t], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}
template <int NACC>
__device__ __forceinline__ bool splitk_exchange(const GemmParams& p, int t, int split, int lane, f32x16* acc) {
  return splitk_exchange<NACC>(p, t, split, p.splitk, lane, acc);
}

// Element stores / loads of the output and side tensors.
template <typename T>
__device__ __forceinline__ void st(void* base, int64_t ld, int m, int n, float v);
template <>
__device__ __forceinline__ void st<uint16_t>(void* base, int64_t ld, int m, int n, float v) {
  reinterpret_cast<uint16_t*>(base)[(int64_t)m * ld + n] = f2bf(v);
}
template <>
__device__ __forceinline__ void st<float>(void* base, int64_t ld, int m, int n, float v) {
  reinterpret_cast<float*>(base)[(int64_t)m * ld + n] = v;
}
template <typename T>
__device__ __forceinline__ float ld_in(const void* base, int64_t ld, int m, int n);
template <>
__device__ __forceinline__ float ld_in<uint16_t>(const void* base, int64_t ld, int m, int n) {
  return bf2f(reinterpret_cast<const uint16_t*>(base)[(int64_t)m * ld + n]);
}
template <>
__device__ __forceinline__ float ld_in<float>(const void* base, int64_t ld, int m, int n) {
  return reinterpret_cast<const float*>(base)[(int64_t)m * ld + n];
}

// The main (bf16) output of the activation epilogues: row-major C, or the
// packed fragment layout of the next decode GEMM's A operand (k = n).
__device__ __forceinline__ void st_main(const GemmParams& p, int m, int n, float v) {
  if (p.cpk) {
    const int64_t chunk = ((int64_t)(n >> 4) * p.cpk_mt + (m >> 5)) * 64 + (m & 31) + ((n >> 3) & 1) * 32;
    reinterpret_cast<uint16_t*>(p.cpk)[chunk * 8 + (n & 7)] = f2bf(v);
  } else {
    st<uint16_t>(p.C, p.ldc, m, n, v);
  }
}

// The epilogue for one output element.  OutT is the type of C (and of the
// C2/C3 side outputs and S0/S1 side inputs, except EPI_STORE's f32 output of
// bf16 inputs, which only writes C).
template <int EPI, typename OutT, typename SideT>
__device__ __forceinline__ void epilogue_elem(const GemmParams& p, int m, int n, float v0, float v1) {
  if constexpr (EPI == EPI_STORE) {
    st<OutT>(p.C, p.ldc, m, n, v0);
  } else if constexpr (EPI == EPI_ACT) {
    float a = v0;
    if (p.bias) a += ld_in<SideT>(p.bias, 0, 0, n);
    if (p.C2) st<SideT>(p.C2, p.ldc2, m, n, a);
    if constexpr (std::is_same<OutT, uint16_t>::value) st_main(p, m, n, act_fwd(p.act, a));
    else st<OutT>(p.C, p.ldc, m, n, act_fwd(p.act, a));
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (p.C2) {
      st<SideT>(p.C2, p.ldc2, m, n, v0);
      st<SideT>(p.C3, p.ldc2, m, n, v1);
    }
    if constexpr (std::is_same<OutT, uint16_t>::value) st_main(p, m, n, v0 * sigmoidf_(v0) * v1);
    else st<OutT>(p.C, p.ldc, m, n, v0 * sigmoidf_(v0) * v1);
  } else if constexpr (EPI == EPI_DUAL_STORE) {
    st<OutT>(p.C, p.ldc, m, n, v0);
    st<OutT>(p.C2, p.ldc2, m, n, v1);
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    const float g = ld_in<SideT>(p.S0, p.lds, m, n);
    const float u = ld_in<SideT>(p.S1, p.lds, m, n);
    const float s = sigmoidf_(g);
    const float sg = g * s;
    st<OutT>(p.C, p.ldc, m, n, v0 * u * (s + sg * (1.0f - s)));
    st<OutT>(p.C2, p.ldc2, m, n, v0 * sg);
    st<OutT>(p.C3, p.ldc3, m, n, sg * u);
  } else if constexpr (EPI == EPI_ACT_BWD) {
    const float a = ld_in<SideT>(p.S0, p.lds, m, n);
    st<OutT>(p.C, p.ldc, m, n, v0 * act_grad(p.act, a));
    st<OutT>(p.C3, p.ldc3, m, n, act_fwd(p.act, a));
  }
}

}  // namespace tpk
