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
#include "tp_kernels.h"
#include "tp_device.h"

namespace tpk {

constexpr int BK = 64;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * 128 + ((chunk ^ swz(row)) << 4); }

// 8 consecutive bf16 starting at src[idx..idx+8), masked to `valid` elements.
__device__ __forceinline__ uint4 load8_masked(const uint16_t* src, int valid) {
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < valid) w[e >> 1] |= ((uint32_t)src[e]) << ((e & 1) * 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// A tile of R rows x BK k-values read from a k-contiguous matrix src[row*ld + k].
// In dual mode rows [0, R/2) come from src0 and [R/2, R) from src1.
template <int R, int NT, bool DUAL>
struct TileKC {
  static constexpr int TOTAL = R * (BK / 8);
  static constexpr int PER = (TOTAL + NT - 1) / NT;
  uint4 v[PER];

  __device__ __forceinline__ void load(const uint16_t* src0, const uint16_t* src1, int64_t ld, int r0,
                                       int rows, int k0, int klen, bool vec, int tid) {
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
      if (gr < rows && gk < klen) {
        const uint16_t* ptr = src + (int64_t)gr * ld + gk;
        if (vec && gk + 8 <= klen) v[c] = *reinterpret_cast<const uint4*>(ptr);
        else v[c] = load8_masked(ptr, klen - gk);
      } else {
        v[c] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const int id = tid + c * NT;
      if (TOTAL % NT != 0 && id >= TOTAL) break;
      *reinterpret_cast<uint4*>(lds + lds_off(id >> 3, id & 7)) = v[c];
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
  uint4 v[PER][8];

  __device__ __forceinline__ void load(const uint16_t* src0, const uint16_t* src1, int64_t ld, int r0,
                                       int rows, int k0, int klen, bool vec, int tid) {
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
        if (gk < klen && valid_r > 0) {
          const uint16_t* ptr = src + (int64_t)gk * ld + gr;
          if (vec && valid_r >= 8) v[c][j] = *reinterpret_cast<const uint4*>(ptr);
          else v[c][j] = load8_masked(ptr, valid_r);
        } else {
          v[c][j] = make_uint4(0u, 0u, 0u, 0u);
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
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&v[c][0]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = i >> 1;
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        uint4 o;
        o.x = __builtin_amdgcn_perm(w[1 * 4 + q], w[0 * 4 + q], sel);
        o.y = __builtin_amdgcn_perm(w[3 * 4 + q], w[2 * 4 + q], sel);
        o.z = __builtin_amdgcn_perm(w[5 * 4 + q], w[4 * 4 + q], sel);
        o.w = __builtin_amdgcn_perm(w[7 * 4 + q], w[6 * 4 + q], sel);
        *reinterpret_cast<uint4*>(lds + lds_off(rb * 8 + i, kb)) = o;
      }
    }
  }
};

template <int R, int NT, bool KC, bool DUAL>
using Tile = typename std::conditional<KC, TileKC<R, NT, DUAL>, TileRC<R, NT, DUAL>>::type;

// Renumber workgroups so that each XCD gets a contiguous range of ids.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  if (nblk < 8) return bid;
  const int xcd = bid & 7;
  const int idx = bid >> 3;
  const int per = nblk >> 3;
  const int rem = nblk & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

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
  __shared__ int s_last;

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

  auto load_tiles = [&](int kt) {
    const bool s1 = kt >= nk0;
    const int k0 = (s1 ? kt - nk0 : kt) * BK;
    const int klen = s1 ? p.K1 : p.K0;
    const uint16_t* a = reinterpret_cast<const uint16_t*>(s1 ? p.A1 : p.A0);
    const uint16_t* b0 = reinterpret_cast<const uint16_t*>(s1 ? p.B1 : p.B0);
    const uint16_t* b1 = reinterpret_cast<const uint16_t*>(p.B1);
    ta.load(a, a, p.lda, m0, p.M, k0, klen, p.vecA, tid);
    tb.load(b0, b1, p.ldb, n0, p.N, k0, klen, p.vecB, tid);
  };

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

  if (kt_begin < kt_end) {
    load_tiles(kt_begin);
    ta.store(smem, tid);
    tb.store(smem + BM * BK * 2, tid);
  }
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int cur = (kt - kt_begin) & 1;
    const bool more = kt + 1 < kt_end;
    if (more) load_tiles(kt + 1);
    const char* la = smem + cur * STAGE;
    const char* lb = la + BM * BK * 2;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int chunk = 2 * s + (lane >> 5);
      bf16x8 af[TM];
      bf16x8 bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(la + lds_off(wm * WM + i * 32 + (lane & 31), chunk));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(lb + lds_off(brow(j) + (lane & 31), chunk));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      char* nxt = smem + (cur ^ 1) * STAGE;
      ta.store(nxt, tid);
      tb.store(nxt + BM * BK * 2, tid);
    }
    __syncthreads();
  }

  // ---- split-K: publish, and let the last arriving split finish ----------
  if (p.splitk > 1) {
    constexpr int NV = TM * TN * 4;  // float4 per lane
    float4* mine = reinterpret_cast<float4*>(p.partials) + ((int64_t)t * p.splitk + split) * NV * NT;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          mine[((i * TN + j) * 4 + q) * NT + tid] =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(&p.counters[t], 1);
      s_last = (prev == p.splitk - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const float4* all = reinterpret_cast<const float4*>(p.partials) + (int64_t)t * p.splitk * NV * NT;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
          for (int s = 0; s < p.splitk; ++s) {
            float4 v;
            if (s == split) {
              v = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            } else {
              v = all[((int64_t)s * NV + (i * TN + j) * 4 + q) * NT + tid];
            }
            sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
          }
          acc[i][j][4 * q] = sum.x; acc[i][j][4 * q + 1] = sum.y;
          acc[i][j][4 * q + 2] = sum.z; acc[i][j][4 * q + 3] = sum.w;
        }
    if (tid == 0) atomicExch(&p.counters[t], 0);
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
    case TILE_128x128: return launch_cfg<128, 128, 2, 2, AKC, BKC, DUAL, EPI, OutT>(p, s);
    case TILE_64x128: return launch_cfg<64, 128, 2, 2, AKC, BKC, DUAL, EPI, OutT>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Tile shape and K-split for an (M, N, K) problem on 256 CUs.
GemmPlan plan_gemm(int M, int N, int K, bool dual) {
  GemmPlan plan;
  const int ncols = dual ? 2 * N : N;  // combined columns
  auto tiles_for = [&](int bm, int bn) {
    const int bnh = dual ? bn / 2 : bn;
    return ((M + bm - 1) / bm) * ((N + bnh - 1) / bnh);
  };
  (void)ncols;
  if (M <= 128) {
    // Decode-sized: stream the weights once, split K so enough workgroups are
    // in flight to keep HBM busy.
    plan.tile = TILE_64x128;
    const int tiles = tiles_for(64, 128);
    const int nk = (K + BK - 1) / BK;
    int split = 1;
    while (tiles * split < 512 && split * 2 <= nk && split < 16) split *= 2;
    plan.splitk = split;
    return plan;
  }
  if (tiles_for(256, 256) >= 256) {
    plan.tile = TILE_256x256;
  } else {
    plan.tile = TILE_128x128;
  }
  plan.splitk = 1;
  return plan;
}

void gemm_split_sizes(const GemmPlan& plan, int M, int N, bool dual, size_t* part_bytes, size_t* n_tiles) {
  *part_bytes = 0;
  *n_tiles = 0;
  if (plan.splitk <= 1) return;
  int bm = 64, bn = 128;
  if (plan.tile == TILE_256x256) { bm = 256; bn = 256; }
  if (plan.tile == TILE_128x128) { bm = 128; bn = 128; }
  const int bnh = dual ? bn / 2 : bn;
  const size_t tiles = (size_t)((M + bm - 1) / bm) * ((N + bnh - 1) / bnh);
  *part_bytes = tiles * plan.splitk * (size_t)bm * bn * sizeof(float);
  *n_tiles = tiles;
}

hipError_t gemm_bf16(const GemmParams& p, const GemmPlan& plan, GemmKind kind, bool out_f32, hipStream_t s) {
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
