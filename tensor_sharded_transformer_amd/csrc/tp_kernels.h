// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tp_device.h"

namespace tpk {

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

enum TileShape : int { TILE_256x256 = 0, TILE_128x128 = 1, TILE_64x128 = 2 };

struct GemmPlan {
  int tile = TILE_128x128;
  int splitk = 1;
};

// Which operand layouts / epilogue a GEMM uses (one kernel family each).
enum GemmKind : int {
  GK_FWD_STORE = 0,       // A k-contig, B (K, N) n-contig, C = acc (bf16 or f32)
  GK_FWD_ACT = 1,         // same, C = act(acc + bias), optional pre-activation save
  GK_FWD_SWIGLU = 2,      // dual B (gate, up), C = silu(g) * u, optional [G|U] save
  GK_BWD_DH_SWIGLU = 3,   // A = dy, B = W2^T (k-contig), epilogue -> dG, dU, h
  GK_BWD_DH_ACT = 4,      // A = dy, B = W2^T, epilogue -> dA, h
  GK_BWD_DW = 5,          // A = X^T (m-contig), B (K, N) n-contig, C = acc
  GK_BWD_DW_DUAL = 6,     // A = x^T, dual B (dG, dU) -> dW1, dWup
  GK_BWD_DX = 7,          // A k-contig (two segments), B k-contig (two segments)
};

GemmPlan plan_gemm(int M, int N, int K, bool dual);
// Split-K scratch for a plan: fp32 partial tiles (bytes) and one arrival
// counter per output tile.
void gemm_split_sizes(const GemmPlan& plan, int M, int N, bool dual, size_t* part_bytes, size_t* n_tiles);
hipError_t gemm_bf16(const GemmParams& p, const GemmPlan& plan, GemmKind kind, bool out_f32, hipStream_t s);

// fp32 (SIMT) GEMM with the same parameter block and epilogues.
hipError_t gemm_f32(const GemmParams& p, GemmKind kind, hipStream_t s);

// Elementwise kernels.
hipError_t act_inplace(void* h, const void* up, int64_t n_elems, bool bf16, int act, hipStream_t s);
hipError_t partial_sum(const void* const* z, int p, const void* bias, void* y, int64_t T, int64_t N,
                       bool in_bf16, bool out_bf16, hipStream_t s);
hipError_t zero_fill(void* ws, size_t bytes, hipStream_t s);

}  // namespace tpk
