// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tp_device.h"

// Build-time tuning of the weight-streaming kernel: k-steps of weight loads
// in flight per wave, 32-column fragments per wave, waves (column groups) per
// workgroup.
#ifndef TP_STREAM_DEPTH
#define TP_STREAM_DEPTH 3
#endif
#ifndef TP_STREAM_NW
#define TP_STREAM_NW 1
#endif
#ifndef TP_STREAM_CW
#define TP_STREAM_CW 4
#endif
#ifndef TP_STREAM_TARGET_WGS
#define TP_STREAM_TARGET_WGS 256
#endif
// Packed-activation decode kernel: waves per workgroup (each streams its own
// K sub-range), 32-column fragments per weight matrix and workgroup, k-steps
// of loads in flight per wave; TP_DECODE=0 keeps the LDS-slice kernel.
#ifndef TP_DECODE
#define TP_DECODE 1
#endif
#ifndef TP_DECODE_KW
#define TP_DECODE_KW 4
#endif
#ifndef TP_DECODE_NW
#define TP_DECODE_NW 2
#endif
#ifndef TP_DECODE_DEPTH
#define TP_DECODE_DEPTH 4
#endif
// Extra K splits for the decode kernel's column strips of the slow
// weight-address class (when split-K is on).
#ifndef TP_DECODE_SLOW_EXTRA
#define TP_DECODE_SLOW_EXTRA 4
#endif

// Pipelined tiled kernel (LDS-bound loads, four-stage ring) for the 256x256
// and 128x128 tiles; TP_TILE_PIPE=0 keeps the register-staged two-stage
// kernel for those tiles.
#ifndef TP_TILE_BK
#define TP_TILE_BK 64
#endif
#ifndef TP_TILE_STAGES_256
#define TP_TILE_STAGES_256 2
#endif
#ifndef TP_TILE_STAGES_128
#define TP_TILE_STAGES_128 2
#endif
#ifndef TP_TILE_PIPE
#define TP_TILE_PIPE 1
#endif
// Wave grid of the 256x256 tile (waves along M x along N).
#ifndef TP_TILE_WGM_256
#define TP_TILE_WGM_256 2
#endif
#ifndef TP_TILE_WGN_256
#define TP_TILE_WGN_256 4
#endif
// Wave grid of the 128x128 tile.
#ifndef TP_TILE_WGM_128
#define TP_TILE_WGM_128 2
#endif
#ifndef TP_TILE_WGN_128
#define TP_TILE_WGN_128 2
#endif
// Tiled kernel: choose the tile size by estimated time (0: 256x256 whenever
// it gives a full round).
#ifndef TP_TILE_COST
#define TP_TILE_COST 1
#endif
// M tiles per group of the tiled kernel's tile order (operand panel reuse in L2).
#ifndef TP_TILE_GROUP
#define TP_TILE_GROUP 8
#endif

namespace tpk {

constexpr int STREAM_NW = TP_STREAM_NW;
constexpr int STREAM_CW = TP_STREAM_CW;
constexpr int STREAM_WCOLS = 32 * STREAM_NW * STREAM_CW;  // output columns per workgroup
constexpr int STREAM_TILES_PER_WG = STREAM_CW;            // split-K tiles per workgroup
constexpr int DECODE_KW = TP_DECODE_KW;
constexpr int DECODE_NW = TP_DECODE_NW;
constexpr int DECODE_WCOLS = 32 * DECODE_NW;              // output columns per workgroup
constexpr int STREAM_LDS_MAX = 160 * 1024;                // gfx950 LDS per workgroup
constexpr int STREAM_MAX_M = 64;                          // tokens the streaming kernel serves
constexpr int STREAM_TARGET_WGS = TP_STREAM_TARGET_WGS;   // K is split until about this many workgroups

// LDS bytes the streaming kernel needs for M rows and a K range of `ksteps`
// 16-value steps.
size_t stream_lds_bytes(int M, int ksteps, bool dual);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// TILE_128x128_W8: 128x128 tiles with 8 waves (4x2) instead of 4, for grids
// of at most one tile per CU.
enum TileShape : int { TILE_256x256 = 0, TILE_128x128 = 1, TILE_64x128 = 2, TILE_128x128_W8 = 3 };
enum KernelKind : int { KERNEL_TILED = 0, KERNEL_STREAM = 1, KERNEL_DECODE = 2 };

struct GemmPlan {
  int kernel = KERNEL_TILED;
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

// fwd_layout: A k-contiguous and B (K, N) n-contiguous (the forward GEMMs),
// the only layout the weight-streaming kernel serves; vec_ok: both operands
// allow 16-byte loads (its other precondition); allow_split: a workspace for
// split-K partials is available.
GemmPlan plan_gemm(int M, int N, int K, bool dual, bool fwd_layout, bool vec_ok, bool allow_split);
// Workspace a plan needs: split-K fp32 partial tiles (bytes), one arrival
// counter per exchange tile, and the packed activation fragments of the
// decode kernel (bytes).
void gemm_split_sizes(const GemmPlan& plan, int M, int N, int K, bool dual, size_t* part_bytes, size_t* n_tiles,
                      size_t* pack_bytes);
hipError_t gemm_bf16(const GemmParams& p, const GemmPlan& plan, GemmKind kind, bool out_f32, hipStream_t s);
hipError_t gemm_stream(const GemmParams& p, const GemmPlan& plan, GemmKind kind, bool out_f32, hipStream_t s);
// Decode kernel (packs p.A0 into p.apk first), its packed-A bytes and its
// split-K exchange tiles.
size_t decode_pack_bytes(int M, int K);
size_t decode_tiles(int M, int N);
hipError_t gemm_decode(const GemmParams& p, const GemmPlan& plan, GemmKind kind, bool out_f32, hipStream_t s);
// The pipelined tiled kernel, for plans and operands it supports.
bool gemm_tile_supported(const GemmParams& p, const GemmPlan& plan, GemmKind kind);
hipError_t gemm_tile(const GemmParams& p, const GemmPlan& plan, GemmKind kind, bool out_f32, hipStream_t s);

// fp32 (SIMT) GEMM with the same parameter block and epilogues.
hipError_t gemm_f32(const GemmParams& p, GemmKind kind, hipStream_t s);

// Elementwise kernels.
hipError_t act_inplace(void* h, const void* up, int64_t n_elems, bool bf16, int act, hipStream_t s);
hipError_t partial_sum(const void* const* z, int p, const void* bias, void* y, int64_t T, int64_t N,
                       bool in_bf16, bool out_bf16, hipStream_t s);
// Rows [rank*T/p, +T/p) of sum_i z[i] (+ bias) + residual -> residual_out, and
// their RMSNorm (scale norm_w) -> y.  N <= RS_NORM_MAX_N.
constexpr int64_t RS_NORM_MAX_N = 32768;
hipError_t rs_residual_rmsnorm(const void* const* z, int p, int rank, const void* bias, const void* residual_in,
                               const void* norm_w, float eps, void* residual_out, void* y, int64_t T, int64_t N,
                               bool in_bf16, bool out_bf16, hipStream_t s);
hipError_t zero_fill(void* ws, size_t bytes, hipStream_t s);
// fp8 codes (K, N) row-major -> 64-column strip-major (N % 64 == 0, both 16-byte aligned).
hipError_t pack_fp8_strips(const void* src, void* dst, int64_t K, int64_t N, hipStream_t s);

// Mixture of experts (experts sharded in place): routing, grouping of the
// routed rows into 128-row tiles per expert, weighted combine.
constexpr int MOE_MAX_E = 1024;
constexpr int MOE_MAX_K = 16;
constexpr int MOE_TILE = 256;  // rows per expert-group tile (the grouped GEMMs' BM)
hipError_t moe_route(const float* logits, int T, int E, int k, int* idx, float* gate, hipStream_t s);
// (xs == nullptr: no gathered copy of x, the GEMM reads x through src_row)
hipError_t moe_group(const int* idx, int T, int E, int k, const void* x, int d, int rows, int n_tiles, int* offsets,
                     int* cursors, int* tile_expert, int* src_row, int* dst_slot, int* pos_of, void* xs, hipStream_t s);
hipError_t moe_combine(const void* zs, bool zs_f32, const int* pos_of, const float* gate, int T, int k, int d,
                       void* y, bool out_f32, hipStream_t s);

// Local grouped-query attention over a rank's heads: qkv (T, (n_q + 2 n_kv)
// * 128) bf16 rows [Q | K | V], out (T, n_q * 128) bf16; both 16-byte
// aligned.  head_dim is fixed at attention_head_dim().
int attention_head_dim();
hipError_t gqa_attention_fwd(const void* qkv, void* out, int T, int n_q, int n_kv, bool causal, float scale,
                             hipStream_t s);

}  // namespace tpk
