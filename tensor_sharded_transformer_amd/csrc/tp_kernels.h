// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tp_device.h"

namespace tpk {

// Weight-streaming kernel with the activation slice in LDS (decode-size calls
// made without a workspace): k-steps of weight loads in flight per wave,
// 32-column fragments per wave, waves (column groups) per workgroup.
constexpr int STREAM_DEPTH = 3;
constexpr int STREAM_NW = 1;
constexpr int STREAM_CW = 4;
constexpr int STREAM_WCOLS = 32 * STREAM_NW * STREAM_CW;  // output columns per workgroup
constexpr int STREAM_TILES_PER_WG = STREAM_CW;            // split-K tiles per workgroup
constexpr int STREAM_LDS_MAX = 160 * 1024;                // gfx950 LDS per workgroup
constexpr int STREAM_MAX_M = 64;                          // tokens the streaming kernels serve
constexpr int STREAM_TARGET_WGS = 256;                    // K is split until about this many workgroups
// Packed-activation decode kernel (row-major weights, a workspace given):
// waves per workgroup (each streams its own K sub-range), 32-column fragments
// per weight matrix and workgroup, k-steps of loads in flight per wave, and
// the extra K splits of the column strips of the slow weight-address class.
constexpr int DECODE_KW = 4;
constexpr int DECODE_NW = 2;
constexpr int DECODE_DEPTH = 4;
constexpr int DECODE_SLOW_EXTRA = 4;
constexpr int DECODE_WCOLS = 32 * DECODE_NW;              // output columns per workgroup
// Pipelined tiled kernel: k per LDS stage, ring stages, wave grids (waves
// along M x along N) of the 256x256 and 128x128 tiles, M tiles per group of
// the tile order (operand panel reuse in L2).
constexpr int TILE_BK = 64;
constexpr int TILE_STAGES = 2;
constexpr int TILE_WGM_256 = 2, TILE_WGN_256 = 4;
constexpr int TILE_WGM_128 = 2, TILE_WGN_128 = 2;
constexpr int TILE_GROUP = 8;
// Packed-weight decode kernel: waves per workgroup, k-blocks of loads in
// flight per wave.
constexpr int PACKED_KW = 4;
constexpr int PACKED_DEPTH = 4;
// waves per workgroup of the bf16 dual (gate/up) launches: 8 streams the
// fused gate/up GEMM 28.4 -> 27.7 us at T=64 (down, QKV and the fp8 launches
// measured slower with 8)
constexpr int PACKED_KW_DUAL = 8;

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
// Column walk of the tiled kernel (one workgroup per 256-row tile walks every
// column tile; A held in LDS): forward store GEMMs with K <= 128 and a bf16
// output whose stored byte offsets (rows below c_max_row) stay below 2^31.
bool gemm_walk_supported(const GemmParams& p, int64_t c_max_row);
hipError_t gemm_walk(const GemmParams& p, hipStream_t s);

// Packed-weight decode GEMM (gemm_packed.hip): weights stored once in 1 KB
// MFMA B-fragment chunks (16-column strips of 32-row k-blocks; fp8 codes: of
// 64-row k-pairs), activations packed alike (32-column k-blocks of 16-row
// tiles), M <= 64.
struct PackedParams {
  const void* A;         // packed activations: nkb k-blocks x mt tiles (fp8 weights: nkb even)
  const void* B0;        // packed weights (nstrips strips x nkb k-blocks, or nkb / 2 k-pairs of fp8 codes)
  const void* B1;        // second packed weights (dual: gate and up), or null
  int M, N, K;           // output rows and columns, contraction length
  int mt;                // 16-row tiles of the packed activations
  int nkb;               // 32-row k-blocks of both packed operands
  int nstrips;           // 16-column strips of the weights
  int splitk;            // workgroups along K per strip group
  float* partials;       // split-K fp32 partial tiles
  int* counters;         // split-K arrival counters (zero on entry, left zero)
  void* C;               // row-major output (bf16 or f32)
  int64_t ldc;
  int vec_out;           // C allows 16-byte stores (aligned, ldc a multiple of 8)
  void* cpk;             // if set: the bf16 output goes here in the packed-activation layout
  int cpk_mt;            //   of a GEMM with this many 16-row tiles
  const uint16_t* bias;  // per-column bias (EPI_ACT), may be null
  int act;
  const float* bscale0;  // fp8 weights: per-column scales of B0 / B1, applied to the sums
  const float* bscale1;
  // If set, the activation fragments are read straight from row-major x
  // (M, K) with rows of xlda elements (K a multiple of 32, of 64 with fp8
  // codes; x and its rows 16-byte aligned; rows past M read as zeros)
  // instead of A
  const uint16_t* xrm;
  int64_t xlda;
  // With xrm (bf16 weights, K a multiple of 64, rows 16-byte aligned): load
  // x in whole 128-byte lines and pass it through LDS into the fragments
  int xstage;
};
struct PackedPlan {
  int ns = 1;              // strips per workgroup
  int splitk = 1;          // workgroups along K
  int kw = PACKED_KW;      // waves per workgroup
};
int packed_mt(int M);
// staged: the plan of a launch that stages row-major x through LDS (two
// strips per workgroup from 64 strips on, so that every such launch has at
// least two weight fragments per k-block)
PackedPlan plan_packed(int M, int N, int K, bool split_ok, bool f8 = false, bool dual = false, bool staged = false);
size_t packed_act_bytes(int M, int K);
size_t packed_units(int M, int N, const PackedPlan& pl);
size_t packed_partial_bytes(int M, int N, bool dual, const PackedPlan& pl);
inline size_t packed_weight_bytes(int64_t K, int64_t N) { return (size_t)((N + 15) / 16) * ((K + 31) / 32) * 1024; }
inline size_t packed_fp8_weight_bytes(int64_t K, int64_t N) { return (size_t)((N + 15) / 16) * ((K + 63) / 64) * 1024; }
// nkb: k-blocks to write (at least (K + 31) / 32; those past K are zeros)
hipError_t pack_act16(const void* x, int64_t lda, int M, int K, bool vec, void* out, hipStream_t s, int nkb = 0);
hipError_t pack_weight16(const void* w, int64_t ldw, int K, int N, bool vec, void* out, hipStream_t s);
hipError_t pack_weight8(const void* w, int64_t ldw, int K, int N, bool vec, void* out, hipStream_t s);
// f8: B0/B1 hold packed fp8 codes (p.nkb even, p.bscale0/1 set)
hipError_t gemm_packed(const PackedParams& p, const PackedPlan& pl, GemmKind kind, bool out_f32, hipStream_t s,
                       bool f8 = false);

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
