// bf16 MFMA GEMM for gfx950 (CDNA4): the column-parallel and row-parallel
// matmuls of one tensor-parallel rank, their fused epilogues, and the shard
// backward's GEMMs.
//
// What is computed (see "Tensor Parallelism" notes, first paragraph, and
// "How does tensor parallelism split a transformer feed-forward block's two
// matmuls across devices?", "Column split, then row split"):
//   C[m, n] = epilogue( sum_k A(m, k) B(k, n) )   with fp32 accumulation.
//
// Design (one workgroup = one BM x BN output tile, or one K-split of it):
//  * v_mfma_f32_32x32x16_bf16: each wave owns a (BM/WGM) x (BN/WGN) block of
//    32x32 accumulator tiles.
//  * Both operands are staged through LDS in a [row][k] layout (row = m for
//    A, n for B) with BK = 64 bf16 (128 B) per row, so every MFMA fragment is
//    one 16-byte ds_read.  The 16-byte chunk index inside a row is XOR-swizzled
//    with (row ^ row>>3) & 7, which keeps both the fragment reads (32
//    consecutive rows, same chunk) and the transposed-staging writes (rows 8
//    apart) spread over distinct banks.
//  * Operands whose memory layout is k-contiguous are copied 16 bytes at a
//    time; operands stored with m or n contiguous (the (in, out) weights, and
//    the transposed operands of the weight gradients) are loaded as 8x8 bf16
//    blocks and transposed in registers with v_perm_b32 before the LDS write.
//  * Two LDS stages: the next K tile is fetched into registers while the
//    current one feeds the MFMAs, then written to the other stage; one
//    barrier per K tile.
//  * Workgroup ids are renumbered so each XCD (ids are dealt round-robin to
//    the 8 XCDs) works on a contiguous, M-grouped range of tiles and shares
//    operand panels in its own L2.
//  * Optional split-K: each split writes its fp32 tile to a workspace in
//    register order; the last split to arrive (agent-scope ticket) sums all
//    splits in ascending order, so the result does not depend on timing, then
//    runs the epilogue and re-zeroes the ticket.
#include <type_traits>

#include "tp_kernels.h"
#include "tp_device.h"

namespace tpk {

constexpr int BK = 64;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive bf16 starting at src, masked to `valid` elements.
__device__ __forceinline__ u32x4 load8_masked(const uint16_t* src, int valid) {
  u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < valid) w[e >> 1] |= ((uint32_t)src[e]) << ((e & 1) * 16);
  }
  return w;
}

// A tile of R rows x BK k-values read from a k-contiguous matrix src[row*ld + k].
// In dual mode rows [0, R/2) come from src0 and [R/2, R) from src1.  The
// unmasked form is used for tiles that lie entirely inside the matrix with
// 16-byte aligned rows; the masked form zero-fills past the edges.
template <int R, int NT, bool DUAL>
struct TileKC {
  static constexpr int TOTAL = R * (BK / 8);
  static constexpr int PER = (TOTAL + NT - 1) / NT;
  u32x4 v[PER];

  template <bool MASKED>
  __device__ __forceinline__ void load(const uint16_t* src0, const uint16_t* src1, int64_t ld, int r0, int rows,
                                       int k0, int klen, bool vec, int tid) {
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int id = tid + c * NT;
      if (TOTAL % NT != 0 && id >= TOTAL) break;
      int row = id >> 3;
      const int kc = id & 7;
      const uint16_t* src = src0;
      if (DUAL && row >= R / 2) { src = src1; row -= R / 2; }
      const int gr = r0 + row;
      const int gk = k0 + kc * 8;
      if constexpr (!MASKED) {
        v[c] = *reinterpret_cast<const u32x4*>(src + (int64_t)gr * ld + gk);
      } else if (gr < rows && gk < klen) {
        const uint16_t* ptr = src + (int64_t)gr * ld + gk;
        if (vec && gk + 8 <= klen) v[c] = *reinterpret_cast<const u32x4*>(ptr);
        else v[c] = load8_masked(ptr, klen - gk);
      } else {
        v[c] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int id = tid + c * NT;
      if (TOTAL % NT != 0 && id >= TOTAL) break;
      *reinterpret_cast<u32x4*>(lds + lds_off(id >> 3, id & 7)) = v[c];
    }
  }
};

// A tile of R rows x BK k-values read from a row-contiguous matrix
// src[k*ld + row] (8x8 blocks, transposed in registers).
template <int R, int NT, bool DUAL>
struct TileRC {
  static constexpr int RB = R / 8;
  static constexpr int TOTAL = RB * (BK / 8);
  static constexpr int PER = (TOTAL + NT - 1) / NT;
  u32x4 v[PER][8];

  template <bool MASKED>
  __device__ __forceinline__ void load(const uint16_t* src0, const uint16_t* src1, int64_t ld, int r0, int rows,
                                       int k0, int klen, bool vec, int tid) {
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int id = tid + c * NT;
      if (TOTAL % NT != 0 && id >= TOTAL) break;
      int rb = id % RB;
      const int kb = id / RB;
      const uint16_t* src = src0;
      if (DUAL && rb >= RB / 2) { src = src1; rb -= RB / 2; }
      const int gr = r0 + rb * 8;
      const int valid_r = rows - gr;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gk = k0 + kb * 8 + j;
        if constexpr (!MASKED) {
          v[c][j] = *reinterpret_cast<const u32x4*>(src + (int64_t)gk * ld + gr);
        } else if (gk < klen && valid_r > 0) {
          const uint16_t* ptr = src + (int64_t)gk * ld + gr;
          if (vec && valid_r >= 8) v[c][j] = *reinterpret_cast<const u32x4*>(ptr);
          else v[c][j] = load8_masked(ptr, valid_r);
        } else {
          v[c][j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int id = tid + c * NT;
      if (TOTAL % NT != 0 && id >= TOTAL) break;
      const int rb = id % RB;
      const int kb = id / RB;
      // v[c][j] holds k = 8kb + j, rows 8rb .. 8rb+7 (two rows per dword).
      // Output row i needs k = 8kb .. 8kb+7 at row 8rb + i.
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = i >> 1;
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        u32x4 o;
        o[0] = __builtin_amdgcn_perm(v[c][1][q], v[c][0][q], sel);
        o[1] = __builtin_amdgcn_perm(v[c][3][q], v[c][2][q], sel);
        o[2] = __builtin_amdgcn_perm(v[c][5][q], v[c][4][q], sel);
        o[3] = __builtin_amdgcn_perm(v[c][7][q], v[c][6][q], sel);
        *reinterpret_cast<u32x4*>(lds + lds_off(rb * 8 + i, kb)) = o;
      }
    }
  }
};

template <int R, int NT, bool KC, bool DUAL>
using Tile = typename std::conditional<KC, TileKC<R, NT, DUAL>, TileRC<R, NT, DUAL>>::type;

template <int BM, int BN, int WGM, int WGN, bool AKC, bool BKC, bool DUAL, int EPI, typename OutT>
__global__ __launch_bounds__(WGM* WGN * 64) void gemm_bf16_kernel(const GemmParams p) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM;
  constexpr int WN = BN / WGN;
  constexpr int TM = WM / 32;
  constexpr int TN = WN / 32;
  constexpr int BNH = DUAL ? BN / 2 : BN;  // output columns per tile
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(!DUAL || (TN % 2 == 0), "dual mode needs gate and up fragments per wave");
  constexpr int STAGE = (BM + BN) * BK * 2;  // bytes per LDS stage
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN;
  const int wn = wave % WGN;

  // ---- tile / split assignment -------------------------------------------
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BNH - 1) / BNH;
  const int ntiles = tiles_m * tiles_n;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int split = id / ntiles;
  const int t = id - split * ntiles;
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int g = t / per_group;
  const int first_m = g * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tin = t - g * per_group;
  const int tm = first_m + tin % gsz;
  const int tn = tin / gsz;
  const int m0 = tm * BM;
  const int n0 = tn * BNH;

  const int nk0 = (p.K0 + BK - 1) / BK;
  const int nk1 = (p.K1 + BK - 1) / BK;
  const int nk = nk0 + nk1;
  const int kt_begin = (int)(((int64_t)nk * split) / p.splitk);
  const int kt_end = (int)(((int64_t)nk * (split + 1)) / p.splitk);

  Tile<BM, NT, AKC, false> ta;
  Tile<BN, NT, BKC, DUAL> tb;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // B fragment row inside the LDS B tile for fragment column j.
  auto brow = [&](int j) -> int {
    if constexpr (DUAL) {
      constexpr int TNH = TN / 2;
      return (j < TNH ? 0 : BN / 2) + wn * (WN / 2) + (j % TNH) * 32;
    } else {
      return wn * WN + j * 32;
    }
  };

  // The K loop, compiled twice: without any masking for tiles that lie
  // entirely inside the operands (the common case), and with edge masking.
  auto kloop = [&](auto masked_tag) {
    constexpr bool MK = decltype(masked_tag)::value;
    auto load_tiles = [&](int kt) {
      const bool s1 = kt >= nk0;
      const int k0 = (s1 ? kt - nk0 : kt) * BK;
      const int klen = s1 ? p.K1 : p.K0;
      const uint16_t* a = reinterpret_cast<const uint16_t*>(s1 ? p.A1 : p.A0);
      const uint16_t* b0 = reinterpret_cast<const uint16_t*>(s1 ? p.B1 : p.B0);
      const uint16_t* b1 = reinterpret_cast<const uint16_t*>(p.B1);
      ta.template load<MK>(a, a, p.lda, m0, p.M, k0, klen, p.vecA, tid);
      tb.template load<MK>(b0, b1, p.ldb, n0, p.N, k0, klen, p.vecB, tid);
    };
    // MFMA operands are double-buffered in registers: the LDS reads of
    // substep s+1 are issued before the MFMAs of substep s, and the next K
    // tile (fetched from global memory at the top of the step) is written to
    // the other LDS stage halfway through the step.
    bf16x8 af[2][TM];
    bf16x8 bfr[2][TN];
    auto read_frags = [&](const char* la, int s, int buf) {
      const char* lb = la + BM * BK * 2;
      const int chunk = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[buf][i] = *reinterpret_cast<const bf16x8*>(la + lds_off(wm * WM + i * 32 + (lane & 31), chunk));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[buf][j] = *reinterpret_cast<const bf16x8*>(lb + lds_off(brow(j) + (lane & 31), chunk));
    };
    auto mma = [&](int buf) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfr[buf][j], acc[i][j], 0, 0, 0);
    };
    if (kt_begin < kt_end) {
      load_tiles(kt_begin);
      ta.store(smem, tid);
      tb.store(smem + BM * BK * 2, tid);
    }
    __syncthreads();
    if (kt_begin < kt_end) read_frags(smem, 0, 0);
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      const int cur = (kt - kt_begin) & 1;
      const bool more = kt + 1 < kt_end;
      const char* la = smem + cur * STAGE;
      char* nxt = smem + (cur ^ 1) * STAGE;
      if (more) load_tiles(kt + 1);
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        if (s + 1 < BK / 16) read_frags(la, s + 1, (s + 1) & 1);
        mma(s & 1);
        if (s == 1 && more) {
          ta.store(nxt, tid);
          tb.store(nxt + BM * BK * 2, tid);
        }
      }
      __syncthreads();
      if (more) read_frags(nxt, 0, 0);
    }
  };
  const bool interior = p.vecA && p.vecB && m0 + BM <= p.M && n0 + BNH <= p.N && p.K0 % BK == 0 && p.K1 % BK == 0;
  if (interior) kloop(std::false_type{});
  else kloop(std::true_type{});

  // ---- split-K ---------------------------------------------------------------
  // Each wave's accumulators are one exchange tile; see splitk_exchange (the
  // epilogue below has no barrier, so the waves may leave independently).
  if (p.splitk > 1) {
    if (!splitk_exchange<TM * TN>(p, t * (NT / 64) + wave, split, lane, &acc[0][0])) return;
  }

  // ---- epilogue -----------------------------------------------------------
  const int mrow = m0 + wm * WM + 4 * (lane >> 5);
  if constexpr (DUAL) {
    constexpr int TNH = TN / 2;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TNH; ++j) {
        const int n = n0 + wn * (WN / 2) + j * 32 + (lane & 31);
        if (n >= p.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mrow + i * 32 + 8 * (r >> 2) + (r & 3);
          if (m < p.M) epilogue_elem<EPI, OutT, uint16_t>(p, m, n, acc[i][j][r], acc[i][j + TNH][r]);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 32 + (lane & 31);
        if (n >= p.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mrow + i * 32 + 8 * (r >> 2) + (r & 3);
          if (m < p.M) epilogue_elem<EPI, OutT, uint16_t>(p, m, n, acc[i][j][r], 0.0f);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Launch configurations.
// ---------------------------------------------------------------------------
struct Cfg {
  int bm, bn;  // bn counts combined (gate+up) columns in dual mode
  int splitk;
};

template <int BM, int BN, int WGM, int WGN, bool AKC, bool BKC, bool DUAL, int EPI, typename OutT>
static hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
  constexpr int BNH = DUAL ? BN / 2 : BN;
  const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BNH - 1) / BNH);
  const int grid = tiles * p.splitk;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, AKC, BKC, DUAL, EPI, OutT>), dim3(grid), dim3(WGM * WGN * 64),
                     0, s, p);
  return hipGetLastError();
}

template <bool AKC, bool BKC, bool DUAL, int EPI, typename OutT>
static hipError_t launch_shape(GemmParams p, const GemmPlan& plan, hipStream_t s) {
  p.splitk = plan.splitk;
  switch (plan.tile) {
    case TILE_256x256: return launch_cfg<256, 256, 2, 2, AKC, BKC, DUAL, EPI, OutT>(p, s);
    case TILE_128x128:
    case TILE_128x128_W8: return launch_cfg<128, 128, 2, 2, AKC, BKC, DUAL, EPI, OutT>(p, s);
    case TILE_64x128: return launch_cfg<64, 128, 2, 2, AKC, BKC, DUAL, EPI, OutT>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Kernel, tile shape and K-split for an (M, N, K) problem on 256 CUs.
GemmPlan plan_gemm(int M, int N, int K, bool dual, bool fwd_layout, bool vec_ok, bool allow_split) {
  GemmPlan plan;
  constexpr int CUS = 256;
  const int nsteps = (K + 15) / 16;
  const bool decode_shape = M <= STREAM_MAX_M && fwd_layout && vec_ok && N >= 8;
  if (decode_shape && allow_split) {
    // Decode-sized forward GEMM with a workspace: packed-activation weight
    // streaming.  Split K across workgroups (a power of two) until about one
    // workgroup per CU, keeping at least 8 k-steps per wave.
    plan.kernel = KERNEL_DECODE;
    const int strips = (N + DECODE_WCOLS - 1) / DECODE_WCOLS;
    int split = 1;
    while (strips * split * 2 <= CUS && nsteps / (split * 2) >= DECODE_KW * 8) split *= 2;
    plan.splitk = split;
    return plan;
  }
  const bool stream_fits = allow_split || stream_lds_bytes(M, nsteps, dual) <= (size_t)STREAM_LDS_MAX;
  if (decode_shape && stream_fits) {
    // Weight streaming with the activation slice in LDS.  Split K across
    // workgroups (a power of two) until about one workgroup per CU while
    // keeping at least 16 k-steps of 16 per split, then further if the
    // split's activation slice would not fit in LDS.
    plan.kernel = KERNEL_STREAM;
    const int strips = (N + STREAM_WCOLS - 1) / STREAM_WCOLS;
    int split = 1;
    while (strips * split * 2 <= STREAM_TARGET_WGS && nsteps / (split * 2) >= 16) split *= 2;
    while (stream_lds_bytes(M, (nsteps + split - 1) / split, dual) > (size_t)STREAM_LDS_MAX) split *= 2;
    plan.splitk = allow_split ? split : 1;
    return plan;
  }
  auto tiles_for = [&](int bm, int bn) {
    const int bnh = dual ? bn / 2 : bn;
    return ((M + bm - 1) / bm) * ((N + bnh - 1) / bnh);
  };
  plan.kernel = KERNEL_TILED;
  if (M <= 128) {
    plan.tile = TILE_64x128;
    const int tiles = tiles_for(64, 128);
    const int nk = (K + BK - 1) / BK;
    int split = 1;
    while (tiles * split < CUS && split * 2 <= nk && split < 8) split *= 2;
    plan.splitk = allow_split ? split : 1;
    return plan;
  }
  // Tile size by estimated time: rounds of 256 CUs times the time of one
  // round.  A round of 256x256 tiles (8 waves) has 4x the work of a round of
  // 128x128 ones (4 waves) and measures ~2.2x as long at K ~ 4096 (107 vs
  // 48 us: the small tiles load twice the bytes per flop through the shared
  // L2-to-CU path), so 256x256 wins once it needs fewer than 1/2.2 of the
  // rounds (attention-projection backward dW_qkv, 640 -> 160 tiles: 121 ->
  // ~100 us).
  const int r256 = (tiles_for(256, 256) + CUS - 1) / CUS;
  const int r128 = (tiles_for(128, 128) + CUS - 1) / CUS;
  plan.tile = r256 * 22 < r128 * 10 ? TILE_256x256 : TILE_128x128;
  plan.splitk = 1;
  if (plan.tile == TILE_128x128 && tiles_for(128, 128) <= CUS) {
    // At most one 128x128 tile per CU: with a workspace, split K in two so
    // each CU runs two 4-wave workgroups (twice the loads in flight; the
    // fp32 partial tiles meet in the workspace); without one, give the single
    // workgroup 8 waves so every SIMD has two to interleave (measured on the
    // 224-tile shard-backward dh GEMM: 80 -> 68 us).
    if (allow_split && (K + 63) / 64 >= 32) plan.splitk = 2;
    else if (tiles_for(128, 128) < CUS) plan.tile = TILE_128x128_W8;
  }
  return plan;
}

void gemm_split_sizes(const GemmPlan& plan, int M, int N, int K, bool dual, size_t* part_bytes, size_t* n_tiles,
                      size_t* pack_bytes) {
  *part_bytes = 0;
  *n_tiles = 0;
  *pack_bytes = 0;
  if (plan.kernel == KERNEL_DECODE) {
    *pack_bytes = decode_pack_bytes(M, K);
    if (plan.splitk <= 1) return;
    const size_t tiles = decode_tiles(M, N);
    // split slots per tile: the plan's splits plus the slow-class strips' extra ones
    *part_bytes = tiles * (plan.splitk + DECODE_SLOW_EXTRA) * (dual ? 2 : 1) * 16 * 64 * sizeof(float);
    *n_tiles = tiles;
    return;
  }
  if (plan.splitk <= 1) return;
  if (plan.kernel == KERNEL_STREAM) {
    const size_t tiles = (size_t)(N + STREAM_WCOLS - 1) / STREAM_WCOLS * STREAM_TILES_PER_WG;
    const int mt = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
    const size_t per = (size_t)mt * (dual ? 2 : 1) * STREAM_NW * 16 * 64;  // floats per column-group tile
    *part_bytes = tiles * plan.splitk * per * sizeof(float);
    *n_tiles = tiles;
    return;
  }
  // the 64x128 and 128x128 tiles (4 waves) split K: every split publishes
  // its fp32 tile; one arrival counter per wave (the register-staged kernel
  // takes a ticket per wave, the pipelined one per workgroup)
  const int bm = plan.tile == TILE_64x128 ? 64 : 128, bn = 128, waves = 4;
  const int bnh = dual ? bn / 2 : bn;
  const size_t tiles = (size_t)((M + bm - 1) / bm) * ((N + bnh - 1) / bnh);
  *part_bytes = tiles * plan.splitk * (size_t)bm * bn * sizeof(float);
  *n_tiles = tiles * waves;
}

hipError_t gemm_bf16(const GemmParams& p, const GemmPlan& plan, GemmKind kind, bool out_f32, hipStream_t s) {
  if (plan.kernel == KERNEL_STREAM) return gemm_stream(p, plan, kind, out_f32, s);
  if (plan.kernel == KERNEL_DECODE) return gemm_decode(p, plan, kind, out_f32, s);
  if (gemm_tile_supported(p, plan, kind)) return gemm_tile(p, plan, kind, out_f32, s);
  switch (kind) {
    case GK_FWD_STORE:
      return out_f32 ? launch_shape<true, false, false, EPI_STORE, float>(p, plan, s)
                     : launch_shape<true, false, false, EPI_STORE, uint16_t>(p, plan, s);
    case GK_FWD_ACT: return launch_shape<true, false, false, EPI_ACT, uint16_t>(p, plan, s);
    case GK_FWD_SWIGLU: return launch_shape<true, false, true, EPI_SWIGLU, uint16_t>(p, plan, s);
    case GK_BWD_DH_SWIGLU: return launch_shape<true, true, false, EPI_SWIGLU_BWD, uint16_t>(p, plan, s);
    case GK_BWD_DH_ACT: return launch_shape<true, true, false, EPI_ACT_BWD, uint16_t>(p, plan, s);
    case GK_BWD_DW: return launch_shape<false, false, false, EPI_STORE, uint16_t>(p, plan, s);
    case GK_BWD_DW_DUAL: return launch_shape<false, false, true, EPI_DUAL_STORE, uint16_t>(p, plan, s);
    case GK_BWD_DX: return launch_shape<true, true, false, EPI_STORE, uint16_t>(p, plan, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpk
