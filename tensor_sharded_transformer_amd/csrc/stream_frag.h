// Device helpers of the weight-streaming (decode-size) GEMM kernels: the
// per-wave weight slab loads and their transposed LDS round trip.
#pragma once
#include "tp_device.h"

namespace tpk {

namespace stream_detail {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One k-step (16 values of k) of weight operands for one wave, as loaded
// from global memory: per matrix, NW instructions of 1 KB, instruction u
// covering rows u*16/NW .. (u+1)*16/NW - 1 and all NW*32 columns, so every
// instruction reads NW*64 contiguous bytes of each of its rows.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int NF>
struct WFrag {
  u32x4 b[NF];
};

// LDS tile of one 32-column fragment: [16 rows][32 columns] bf16 (64-byte
// rows), padded so the NW tiles a row of lanes writes to land on different
// banks.
template <int NW>
constexpr int tile_bytes() { return NW == 1 ? 1024 : 1152; }

// Weight loads of one k-step.  The kernel runs only when the weights allow
// 16-byte loads (rows 16-byte aligned, N a multiple of 8); columns beyond N
// are clamped to the last valid 8-column chunk, whose products only reach
// outputs the epilogue never stores.  In the TAIL step rows at or beyond K
// read as zero.
template <int NW, bool DUAL, bool TAIL>
__device__ __forceinline__ void load_w(WFrag<DUAL ? 2 * NW : NW>& fr, const GemmParams& p, int step, int n0,
                                       int lane) {
  constexpr int RPI = 16 / NW;     // rows per instruction
  constexpr int CPR = NW * 4;      // 16-byte chunks per row
  const int c = lane % CPR;
  const int n = min(n0 + c * 8, p.N - 8);
#pragma unroll
  for (int mat = 0; mat < (DUAL ? 2 : 1); ++mat) {
    const uint16_t* B = reinterpret_cast<const uint16_t*>(mat ? p.B1 : p.B0);
#pragma unroll
    for (int u = 0; u < NW; ++u) {
      const int kb = step * 16 + u * RPI + lane / CPR;
      if (!TAIL || kb < p.K0) fr.b[mat * NW + u] = *reinterpret_cast<const u32x4*>(B + (int64_t)kb * p.ldb + n);
      else fr.b[mat * NW + u] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// fp8 weights (one byte per value, NW == 2) in 64-column strip-major order:
// value (k, n) at byte (n / 64) * 64 K + 64 k + n % 64, so a strip's rows are
// one contiguous run and every cache line feeds a single workgroup.  One
// k-step of one matrix is a single 1 KB instruction: lane l reads row l/4,
// columns 16 (l%4) .. +15 of the strip.  Raw codes stay in registers until
// the k-step is consumed.
template <bool DUAL, bool TAIL>
__device__ __forceinline__ void load_w8(WFrag<DUAL ? 2 : 1>& fr, const GemmParams& p, int step, int n0, int lane) {
  const int kb = step * 16 + (lane >> 2);
  const int64_t off = (int64_t)(n0 >> 6) * 64 * p.K0 + (int64_t)kb * 64 + (lane & 3) * 16;
#pragma unroll
  for (int mat = 0; mat < (DUAL ? 2 : 1); ++mat) {
    const uint8_t* B = reinterpret_cast<const uint8_t*>(mat ? p.B1 : p.B0);
    if (!TAIL || kb < p.K0) fr.b[mat] = *reinterpret_cast<const u32x4*>(B + off);
    else fr.b[mat] = u32x4{0u, 0u, 0u, 0u};
  }
}

// Four fp8 (e4m3) codes -> four bf16 values (exact: every e4m3 value is a
// bf16 value), in two 32-bit words, low code first.
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t* lo, uint32_t* hi) {
  typedef float f32x2_ __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_ __attribute__((ext_vector_type(2)));
  const f32x2_ a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_ b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  *lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2_));
  *hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2_));
}

// LDS position of this lane's 16 bytes of instruction u of matrix `mat`.
template <int NW>
__device__ __forceinline__ int w_lds_off(int mat, int u, int lane) {
  constexpr int RPI = 16 / NW, CPR = NW * 4;
  const int c = lane % CPR;
  const int row = u * RPI + lane / CPR;
  return (mat * NW + c / 4) * tile_bytes<NW>() + row * 64 + (c % 4) * 16;
}

// Activation fragment of the TAIL step straight from global memory, with
// k-values at or beyond K read as zero (rows beyond M clamped).
__device__ __forceinline__ u32x4 load_a_tail(const GemmParams& p, int mt, int step, int lane) {
  const int m = min(mt * 32 + (lane & 31), p.M - 1);
  const int ka = step * 16 + (lane >> 5) * 8;
  const uint16_t* ptr = reinterpret_cast<const uint16_t*>(p.A0) + (int64_t)m * p.lda + ka;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (ka + e < p.K0) w[e >> 1] |= ((uint32_t)ptr[e]) << ((e & 1) * 16);
  return u32x4{w[0], w[1], w[2], w[3]};
}

// ds_read_b64_tr_b16 over a [16 rows][32 columns] bf16 tile (64-byte rows):
// in each group of 16 lanes, lane 4j+q names row r0+j, columns c0+4q..c0+4q+3,
// and lane i receives rows r0..r0+3 of column c0+i.  Two reads give the MFMA
// B operand: lane l gets rows 8(l/32)..8(l/32)+7 of column l%32.
__device__ __forceinline__ bf16x8 read_b_frag(const char* tile, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int c0 = (g & 1) * 16, r0 = (g >> 1) * 8;
  const int off = (r0 + (s >> 2)) * 64 + (c0 + (s & 3) * 4) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off + 4 * 64));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace stream_detail
using namespace stream_detail;

// K range of split `split` in whole 16-value steps.
__device__ __forceinline__ void split_range(int K, int splitk, int split, int* s_begin, int* s_end) {
  const int nsteps = (K + 15) / 16;
  *s_begin = (int)(((int64_t)nsteps * split) / splitk);
  *s_end = (int)(((int64_t)nsteps * (split + 1)) / splitk);
}

}  // namespace tpk
