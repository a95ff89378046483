// bf16 MFMA GEMM for gfx950 (CDNA4) with a deep global-load pipeline: the
// prefill-sized column-parallel and row-parallel matmuls of one
// tensor-parallel rank and the shard backward's GEMMs.
//
// What is computed (see "Tensor Parallelism" notes, first paragraph, and
// "How does tensor parallelism split a transformer feed-forward block's two
// matmuls across devices?", "Column split, then row split"):
//   C[m, n] = epilogue( sum_k A(m, k) B(k, n) )   with fp32 accumulation.
//
// Design (one workgroup of WGM x WGN waves = one BM x BN output tile):
//  * v_mfma_f32_32x32x16_bf16; each wave owns a (BM/WGM) x (BN/WGN) block of
//    32x32 accumulator tiles.
//  * K advances in tiles of 64.  Operand tiles go from global memory straight
//    into LDS (buffer_load_dwordx4 ... lds, no staging registers) through a
//    ring of STAGES separate LDS arrays; the loads of tile kt+STAGES-1 are
//    issued while tile kt feeds the MFMAs.  Because each stage is its own LDS
//    object, the compiler orders a fragment read only after the loads into
//    that stage, not after every load in flight.
//  * Operands keep their memory layout in LDS.  A k-contiguous operand is a
//    [rows][64] tile (128-byte rows) read as MFMA fragments with ds_read_b128;
//    an m- or n-contiguous operand (the (in, out) weights, the transposed
//    operands of the weight gradients) is a [64][cols] tile in sub-tiles of at
//    most 128 columns, read with ds_read_b64_tr_b16, which transposes 16-bit
//    elements on the way out of LDS.  Both layouts XOR-swizzle 16-byte chunks
//    (measured conflict-free on gfx950); the swizzle is applied on the global
//    side of the load: each lane fetches the chunk that belongs at its fixed
//    LDS slot.
//  * Edges: each lane's buffer offset is replaced by an out-of-range value
//    when its 16-byte chunk lies outside the matrix; the buffer unit then
//    writes zeros to LDS.  No separate masked loop.
//  * One barrier per k-tile.  The MFMAs of a tile's last substep run after
//    that barrier, interleaved with the next tile's first fragment reads, and
//    every MFMA block is interleaved with the LDS reads of the next block.
//  * Workgroup ids are renumbered so each XCD works on a contiguous, M-grouped
//    range of tiles and shares operand panels in its own L2.
#include <type_traits>

#include "tp_kernels.h"
#include "tp_device.h"

namespace tpk {
namespace {

constexpr int TBK = TILE_BK;            // k per LDS stage
constexpr int NSUB = TBK / 16;          // MFMA k-substeps per stage
constexpr int KC_CHUNKS = TBK / 8;      // 16-byte chunks per k-contiguous row
constexpr uint32_t OOB = 0x80000000u;   // buffer offset past the record bound

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// Chunk swizzle of a k-contiguous [rows][64] tile (128-byte rows):
// conflict-free ds_read_b128 of 32 consecutive rows, one chunk each
// (measured on gfx950: row bits 0-2 and 3).
static_assert(TBK == 64, "the swizzles below are for 128-byte rows");
__device__ __forceinline__ int kc_swz(int row) { return (row ^ (row >> 3)) & 7; }
// Chunk swizzle of a [32][SW] sub-tile (SW = 128: 16 chunks per row,
// SW = 64: 8): conflict-free ds_read_b64_tr_b16 of four k-rows x 32 columns.
template <int SW>
__device__ __forceinline__ int mn_swz(int krow) {
  if constexpr (SW == 128) return ((krow & 1) * 10) ^ ((krow & 2) * 2);
  else return 2 * (krow & 3);
}

// Scheduling recipe for one block: NM MFMAs, each followed by its share of
// NR LDS reads, NW LDS writes and NV global loads, so the wave issues memory
// instructions while the matrix core works instead of in bursts between MFMAs.
template <int NM, int NR, int NW, int NV>
__device__ __forceinline__ void interleave() {
  static_for<0, NM>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    constexpr int r = (i + 1) * NR / NM - i * NR / NM;
    constexpr int w = (i + 1) * NW / NM - i * NW / NM;
    constexpr int v = (i + 1) * NV / NM - i * NV / NM;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // DS read
    if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(0x200, w, 0);  // DS write
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);  // VMEM read
  });
}

// One operand's tile of R rows (k-contiguous) or R columns (m/n-contiguous)
// by TBK k-values.  Each of the NT threads issues NL 16-byte loads per
// stage; load c of thread tid fills LDS slot c*NT + tid.  Every wave-wide
// load lies inside one source matrix, so its buffer descriptor is uniform.
template <int R, bool KC, bool DUAL, int NT>
struct OpTile {
  static constexpr int NL = R * TBK / (8 * NT);              // loads per thread per stage
  static_assert(R * TBK % (8 * NT) == 0, "whole loads per thread");
  static constexpr int BYTES = R * TBK * 2;                  // LDS bytes per stage
  static constexpr int SW = KC ? 0 : (DUAL ? (R / 2 < 128 ? R / 2 : 128) : (R < 128 ? R : 128));
  static_assert(KC || SW == 64 || SW == 128, "sub-tile width");
  static_assert(R % 64 == 0, "tile extent");
  static constexpr int SUB_SLOTS = KC ? 0 : TBK * SW / 8;    // 16-byte slots per sub-tile

  uint32_t voff[NL];  // byte offset from the (source, k-tile) base
  int kidx[NL];       // k position checked against the k-tile's valid length (INT_MAX: masked)

  // Which source matrix (0 / 1) load c reads: the second half of a dual tile.
  static constexpr int src_of(int c) {
    if constexpr (!DUAL) return 0;
    else if constexpr (KC) return c * NT >= (R / 2) * KC_CHUNKS ? 1 : 0;
    else return ((c * NT) / SUB_SLOTS) >= (R / SW) / 2 ? 1 : 0;
  }

  // r0: first row (KC) or column (MN) of the tile in each source;
  // extent: rows (KC) or columns (MN) of each source; ld in elements.
  __device__ __forceinline__ void setup(int tid, int r0, int extent, int64_t ld) {
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      const int slot = c * NT + tid;
      if constexpr (KC) {
        int row = slot / KC_CHUNKS;
        if (DUAL && row >= R / 2) row -= R / 2;
        const int chunk = (slot % KC_CHUNKS) ^ kc_swz(slot / KC_CHUNKS);
        voff[c] = (uint32_t)(row * ld * 2 + chunk * 16);
        kidx[c] = r0 + row < extent ? chunk * 8 : INT_MAX;
      } else {
        const int st = slot / SUB_SLOTS;                // sub-tile
        const int within = slot % SUB_SLOTS;
        const int krow = within / (SW / 8);
        const int chunk = (within % (SW / 8)) ^ mn_swz<SW>(krow);
        const int col = (DUAL ? st % ((R / SW) / 2) : st) * SW + chunk * 8;
        voff[c] = (uint32_t)(krow * ld * 2 + col * 2);
        kidx[c] = r0 + col < extent ? krow : INT_MAX;
      }
    }
  }

  // k-contiguous rows named by a table: row r of the tile reads source row
  // rows[r0 + r] (offsets from the source's row 0; -1 masks the row).
  __device__ __forceinline__ void setup_rows(int tid, int r0, int extent, int64_t ld, const int* rows) {
    static_assert(KC && !DUAL, "row tables index k-contiguous single operands");
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      const int slot = c * NT + tid;
      const int row = slot / KC_CHUNKS;
      const int chunk = (slot % KC_CHUNKS) ^ kc_swz(row);
      const int src = r0 + row < extent ? rows[r0 + row] : -1;
      voff[c] = (uint32_t)(max(src, 0) * ld * 2 + chunk * 16);
      kidx[c] = src >= 0 ? chunk * 8 : INT_MAX;
    }
  }

  // Issue one k-tile's loads straight into LDS.  base0/base1: the sources
  // at (tile origin, k-tile start); kvalid: k-values of the k-tile inside the
  // matrix (<= 0: every load masked); lds: this operand's tile in the stage.
  __device__ __forceinline__ void issue(const void* base0, const void* base1, int kvalid, char* lds,
                                        int wave) const {
    const __amdgpu_buffer_rsrc_t r0 = rsrc_at(base0);
    const __amdgpu_buffer_rsrc_t r1 = rsrc_at(base1);
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      const uint32_t off = kidx[c] < kvalid ? voff[c] : OOB;
      lds_void* dst = (lds_void*)(lds + (c * NT + wave * 64) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src_of(c) ? r1 : r0, dst, 16, off, 0, 0, 0);
    }
  }

  // The same k-tile through registers (single source): fetch loads this
  // thread's chunks (masked ones read as zeros), put writes them to the LDS
  // slots issue() would fill.
  __device__ __forceinline__ void fetch(const void* base, int kvalid, u32x4 (&r)[NL]) const {
    static_assert(!DUAL, "one source");
    const __amdgpu_buffer_rsrc_t rs = rsrc_at(base);
#pragma unroll
    for (int c = 0; c < NL; ++c)
      r[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, kidx[c] < kvalid ? voff[c] : OOB, 0, 0));
  }
  __device__ __forceinline__ void put(char* lds, int tid, const u32x4 (&r)[NL]) const {
#pragma unroll
    for (int c = 0; c < NL; ++c) *reinterpret_cast<u32x4*>(lds + (c * NT + tid) * 16) = r[c];
  }
};

// Lane-constant part of the LDS byte offset of an MFMA fragment whose 32
// rows (KC) or columns (MN) start at `first` inside the operand tile.
// KC: o0 = row start, o1 = the lane's chunk for substep 0 (substep s reads
// chunk o1 ^ 2s).  MN: o0 = the offset for substep 0.
template <int R, bool KC, bool DUAL>
__device__ __forceinline__ void frag_offsets(int first, int lane, int* o0, int* o1) {
  if constexpr (KC) {
    const int row = first + (lane & 31);
    *o0 = row * (TBK * 2);
    *o1 = (lane >> 5) ^ kc_swz(row);
  } else {
    constexpr int SW = OpTile<R, KC, DUAL, 256>::SW;
    const int g = lane >> 4, i = lane & 15;
    const int col = first + (g & 1) * 16 + 4 * (i & 3);
    const int st = col / SW, cc = col % SW;
    const int krow = (g >> 1) * 8 + (i >> 2);        // plus 16*substep + 4*read
    *o0 = st * (TBK * SW * 2) + krow * (SW * 2) + (((cc >> 3) ^ mn_swz<SW>(krow)) << 4) + (cc & 7) * 2;
    *o1 = *o0;
  }
}

template <int R, bool KC, bool DUAL>
__device__ __forceinline__ bf16x8 read_frag(const char* tile, int o0, int o1, int s) {
  if constexpr (KC) {
    return *reinterpret_cast<const bf16x8*>(tile + o0 + ((o1 ^ (2 * s)) << 4));
  } else {
    constexpr int SW = OpTile<R, KC, DUAL, 256>::SW;
    const char* p = tile + o0 + s * 16 * (SW * 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * SW * 2));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
}

// s_waitcnt vmcnt(N), other counters untouched, then s_barrier.  Written as
// one asm statement with a memory clobber so no LDS access moves across it;
// the wait covers this wave's own LDS-bound loads, the barrier everyone's.
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  if constexpr (N == 0) __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) __asm__ volatile("s_waitcnt vmcnt(8)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 16) __asm__ volatile("s_waitcnt vmcnt(16)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 24) __asm__ volatile("s_waitcnt vmcnt(24)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4) __asm__ volatile("s_waitcnt vmcnt(4)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 12) __asm__ volatile("s_waitcnt vmcnt(12)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 32) __asm__ volatile("s_waitcnt vmcnt(32)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 48) __asm__ volatile("s_waitcnt vmcnt(48)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 63) __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // LDS only
  else static_assert(N == 0, "add the vmcnt value here");
}

template <int BM, int BN, bool AKC, bool BKC, bool DUAL, int NT>
struct TileCfg {
  using TA = OpTile<BM, AKC, false, NT>;
  using TB = OpTile<BN, BKC, DUAL, NT>;
  static constexpr int STAGE = TA::BYTES + TB::BYTES;
  static constexpr int LPS = TA::NL + TB::NL;  // loads per thread per stage
};

// WGM x WGN waves; wave (wm, wn) owns rows [wm*BM/WGM, +BM/WGM) and
// columns [wn*BN/WGN, +BN/WGN) of the tile (per source in dual mode).
template <int BM, int BN, int WGM, int WGN, int STAGES, bool AKC, bool BKC, bool DUAL, int EPI, typename OutT>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_tile_kernel(const GemmParams p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int BNH = DUAL ? BN / 2 : BN;  // output columns per tile
  static_assert(TM >= 1 && TN >= 1, "at least one 32x32 fragment per wave");
  static_assert(!DUAL || (TN % 2 == 0), "dual mode needs gate and up fragments per wave");
  using Cfg = TileCfg<BM, BN, AKC, BKC, DUAL, NT>;
  using TA = typename Cfg::TA;
  using TB = typename Cfg::TB;
  constexpr int STAGE = Cfg::STAGE;
  constexpr int LPS = Cfg::LPS;
  static_assert(STAGES >= 2 && STAGES <= 5, "the ring is two to five LDS arrays");
  static_assert(NSUB % 2 == 0, "fragment buffers alternate per substep");
  // One LDS object per stage (see the header comment).
  __shared__ __attribute__((aligned(1024))) char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[STAGE];
  __shared__ __attribute__((aligned(1024))) char st3[STAGES > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char st4[STAGES > 4 ? STAGE : 16];
  auto stage = [&](auto ic) -> char* {
    constexpr int i = decltype(ic)::value % STAGES;
    if constexpr (i == 0) return st0;
    else if constexpr (i == 1) return st1;
    else if constexpr (i == 2) return st2;
    else if constexpr (i == 3) return st3;
    else return st4;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN;
  const int wn = wave % WGN;

  // ---- tile and K-split assignment (XCD-contiguous, M-grouped) -------------
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BNH - 1) / BNH;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int split = id / (tiles_m * tiles_n);
  const int t = id - split * (tiles_m * tiles_n);
  constexpr int GROUP = TILE_GROUP;
  const int per_group = GROUP * tiles_n;
  const int g = t / per_group;
  const int first_m = g * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tin = t - g * per_group;
  const int m0 = (first_m + tin % gsz) * BM;
  const int n0 = (tin / gsz) * BNH;

  const int nk0 = (p.K0 + TBK - 1) / TBK;
  const int nk = nk0 + (p.K1 + TBK - 1) / TBK;
  // this split's k-tiles (both K segments counted together)
  const int kt_begin = (int)((int64_t)nk * split / p.splitk);
  const int kt_end = (int)((int64_t)nk * (split + 1) / p.splitk);

  // grouped mode: this M tile's expert selects the weights (a tile with no
  // routed rows has nothing to do; the whole workgroup leaves together)
  const uint16_t* gB0 = reinterpret_cast<const uint16_t*>(p.B0);
  const uint16_t* gB1 = reinterpret_cast<const uint16_t*>(p.B1);
  if (p.tile_expert) {
    const int ex = p.tile_expert[m0 / BM];
    if (ex < 0) return;
    gB0 += ex * p.b_expert_stride;
    if (gB1) gB1 += ex * p.b_expert_stride;
  }

  TA ta;
  TB tb;
  if constexpr (AKC) {
    if (p.a_rows) ta.setup_rows(tid, m0, p.M, p.lda, p.a_rows);
    else ta.setup(tid, m0, p.M, p.lda);
  } else {
    ta.setup(tid, m0, p.M, p.lda);
  }
  tb.setup(tid, n0, p.N, p.ldb);

  // Issue the LDS-bound loads of k-tile kt into stage array st.  Tiles past
  // the end are issued too, fully masked (no memory access, zeros in LDS), so
  // every step issues the same number of loads and the wait counts are exact.
  auto issue = [&](int kt, char* st) {
    const bool s1 = kt >= nk0;
    const int k0 = (s1 ? kt - nk0 : kt) * TBK;
    const int kvalid = kt >= kt_end ? 0 : (s1 ? p.K1 : p.K0) - k0;
    const uint16_t* a = reinterpret_cast<const uint16_t*>(s1 ? p.A1 : p.A0);
    const uint16_t* b0 = s1 ? gB1 : gB0;
    const uint16_t* b1 = gB1;
    const int64_t ao =
        kvalid <= 0 ? 0 : (AKC ? (p.a_rows ? 0 : (int64_t)m0 * p.lda) + k0 : (int64_t)k0 * p.lda + m0);
    const int64_t bo = kvalid <= 0 ? 0 : (BKC ? (int64_t)n0 * p.ldb + k0 : (int64_t)k0 * p.ldb + n0);
    ta.issue(a + ao, a + ao, kvalid, st, wave);
    tb.issue(b0 + bo, b1 + bo, kvalid, st + TA::BYTES, wave);
  };

  // Fragment offsets (lane-constant) inside a stage.
  int ao0[TM], ao1[TM], bo0[TN], bo1[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) frag_offsets<BM, AKC, false>(wm * WM + i * 32, lane, &ao0[i], &ao1[i]);
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    int first;
    if constexpr (DUAL) {
      constexpr int TNH = TN / 2;
      first = (j < TNH ? 0 : BN / 2) + wn * (WN / 2) + (j % TNH) * 32;
    } else {
      first = wn * WN + j * 32;
    }
    frag_offsets<BN, BKC, DUAL>(first, lane, &bo0[j], &bo1[j]);
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  bf16x8 af[2][TM];
  bf16x8 bf[2][TN];
  auto read_frags = [&](const char* st, int s, int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i) af[buf][i] = read_frag<BM, AKC, false>(st, ao0[i], ao1[i], s);
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[buf][j] = read_frag<BN, BKC, DUAL>(st + TA::BYTES, bo0[j], bo1[j], s);
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bf[buf][j], acc[i][j], 0, 0, 0);
  };

  // ---- main loop -------------------------------------------------------------
  // Tile t lives in stage t % STAGES.  Step kt: issue tile kt+STAGES-1 into the stage tile
  // kt-1 used (every wave finished reading it before the barrier that ended
  // step kt-1); block 0 = MFMAs of tile kt-1's second substep + fragment reads
  // of tile kt's first; block 1 = MFMAs of tile kt's first substep + reads of
  // its second; then wait for this wave's loads of tile kt+1 and barrier.
  // The loop is unrolled by STAGES so every stage array is a constant.
  static_for<0, STAGES - 1>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    issue(kt_begin + i, stage(ic));
  });
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) af[1][i][e] = (__bf16)0.0f;
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) bf[1][j][e] = (__bf16)0.0f;
  wait_loads_barrier<(STAGES - 2) * LPS>();
  constexpr int NMF = TM * TN;                                  // MFMAs per block
  constexpr int NRD = TM * (AKC ? 1 : 2) + TN * (BKC ? 1 : 2);  // LDS reads per block
  const int nk_pad = (kt_end - kt_begin + STAGES - 1) / STAGES * STAGES;
  for (int kt0 = 0; kt0 < nk_pad; kt0 += STAGES) {
    static_for<0, STAGES>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      const int kt = kt_begin + kt0 + u;
      const char* cur = stage(uc);
      issue(kt + STAGES - 1, stage(std::integral_constant<int, u + STAGES - 1>{}));
      // block b: MFMAs of the substep before b (block 0: the previous tile's
      // last one) while the fragments of substep b are read.
      static_for<0, NSUB>([&](auto bc) __attribute__((always_inline)) {
        constexpr int b = decltype(bc)::value;
        read_frags(cur, b, b & 1);
        mma((b + 1) & 1);
        interleave<NMF, NRD, 0, b == 0 ? LPS : 0>();
        __builtin_amdgcn_sched_barrier(0);
      });
      wait_loads_barrier<(STAGES - 2) * LPS>();
    });
  }
  mma(1);

  // ---- split-K ---------------------------------------------------------------
  // Every wave publishes its accumulators ([split][acc][quarter][lane][4], 1 KB
  // per wave instruction); the workgroup takes one arrival ticket for its
  // tile, so all its waves either leave together or, in the last split to
  // arrive, add the splits in split order and go on to the epilogue.
  if (p.splitk > 1) {
    constexpr int NACC = TM * TN;
    constexpr uint32_t WAVE_BYTES = NACC * 16 * 64 * 4;
    __shared__ int ticket;
    const float* base = p.partials + ((int64_t)t * (NT / 64) + wave) * p.splitk * (WAVE_BYTES / 4);
    const __amdgpu_buffer_rsrc_t r = splitk_rsrc(base, WAVE_BYTES * (uint32_t)p.splitk);
    static_for<0, NACC>([&](auto ac) __attribute__((always_inline)) {
      constexpr int a = decltype(ac)::value;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4v v = {acc[a / TN][a % TN][4 * q], acc[a / TN][a % TN][4 * q + 1], acc[a / TN][a % TN][4 * q + 2],
                          acc[a / TN][a % TN][4 * q + 3]};
        splitk_store(r, split * WAVE_BYTES + ((a * 4 + q) * 64 + lane) * 16, v);
      }
    });
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are complete
    __syncthreads();
    if (tid == 0) ticket = __hip_atomic_fetch_add(&p.counters[t], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (ticket != p.splitk - 1) return;
    static_for<0, NACC>([&](auto ac) __attribute__((always_inline)) {
      constexpr int a = decltype(ac)::value;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a / TN][a % TN][e] = 0.0f;
    });
    for (int sp = 0; sp < p.splitk; ++sp) {
      static_for<0, NACC>([&](auto ac) __attribute__((always_inline)) {
        constexpr int a = decltype(ac)::value;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4v v = splitk_load(r, sp * WAVE_BYTES + ((a * 4 + q) * 64 + lane) * 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[a / TN][a % TN][4 * q + e] += v[e];
        }
      });
    }
    if (tid == 0) __hip_atomic_store(&p.counters[t], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue --------------------------------------------------------------
  // Accumulator register r of tile (i, j) is row 8(r/4) + 4(lane/32) + r%4,
  // column lane%32 of that 32x32 tile.  Fully unrolled so every accumulator
  // index is a compile-time constant.
  const int mrow = m0 + wm * WM + 4 * (lane >> 5);
  constexpr int TNO = DUAL ? TN / 2 : TN;  // output fragments per wave row

  // Common case (a bf16 output with nothing else to write): each 32x32 tile
  // goes through a per-wave LDS patch so the global stores are 16 bytes per
  // lane along rows (two per tile) instead of 16 two-byte stores.
  if constexpr (std::is_same<OutT, uint16_t>::value && (EPI == EPI_STORE || EPI == EPI_ACT || EPI == EPI_SWIGLU)) {
    if (!p.C2 && !p.cpk && (!p.c_rows || EPI == EPI_STORE) && p.N % 8 == 0 && p.ldc % 8 == 0 &&
        ((uintptr_t)p.C & 15) == 0) {
      wait_loads_barrier<0>();                // every stage is idle (masked tail loads included)
      constexpr int PITCH = 80;               // bytes per patch row: 64 + 16 of padding
      static_assert(NT / 64 * 32 * PITCH <= STAGE, "patches fit in stage 0");
      char* patch = st0 + wave * 32 * PITCH;
      static_for<0, TM>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        int crow[2];                          // destination rows of this lane's two stores
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int m = m0 + wm * WM + i * 32 + q * 16 + (lane >> 2);
          crow[q] = m >= p.M ? -1 : (p.c_rows ? p.c_rows[m] : m);
        }
        static_for<0, TNO>([&](auto jc) __attribute__((always_inline)) {
          constexpr int j = decltype(jc)::value;
          const int ncol = n0 + wn * (DUAL ? WN / 2 : WN) + j * 32;
          const int n = ncol + (lane & 31);
          float bias = 0.0f;
          if constexpr (EPI == EPI_ACT) {
            if (p.bias && n < p.N) bias = bf2f(reinterpret_cast<const uint16_t*>(p.bias)[n]);
          }
          auto value = [&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            if constexpr (EPI == EPI_STORE) return acc[i][j][r];
            else if constexpr (EPI == EPI_ACT) return act_fwd(p.act, acc[i][j][r] + bias);
            else return acc[i][j][r] * sigmoidf_(acc[i][j][r]) * acc[i][j + TNO][r];
          };
          // registers r and r + 1 (r even) are neighbouring rows: one
          // conversion for the pair, then a 2-byte write each
          static_for<0, 8>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = 2 * decltype(rc)::value;
            const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const uint32_t two = f2bf2(value(std::integral_constant<int, r>{}), value(std::integral_constant<int, r + 1>{}));
            *reinterpret_cast<uint16_t*>(patch + row * PITCH + (lane & 31) * 2) = (uint16_t)two;
            *reinterpret_cast<uint16_t*>(patch + (row + 1) * PITCH + (lane & 31) * 2) = (uint16_t)(two >> 16);
          });
          // one wave's LDS operations complete in order: the reads see the writes
          static_for<0, 2>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            const int row = q * 16 + (lane >> 2);
            const int cc = (lane & 3) * 8;
            const u32x4 v = *reinterpret_cast<const u32x4*>(patch + row * PITCH + cc * 2);
            if (crow[q] >= 0 && ncol + cc < p.N)
              *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.C) + (int64_t)crow[q] * p.ldc + ncol + cc) = v;
          });
        });
      });
      return;
    }
  }
  // Backward activation epilogues (dh times the activation's derivative, read
  // from the saved pre-activations, plus the recomputed activation): the
  // fp32 accumulators go through a per-wave LDS patch 16 rows at a time, so
  // each lane owns 8 consecutive columns of one row and every side load and
  // output store is 16 bytes (instead of five 2-byte accesses per element).
  if constexpr (std::is_same<OutT, uint16_t>::value && !DUAL && (EPI == EPI_SWIGLU_BWD || EPI == EPI_ACT_BWD)) {
    const bool two_sides = EPI == EPI_SWIGLU_BWD;
    if (!p.c_rows && p.N % 8 == 0 && p.ldc % 8 == 0 && p.ldc3 % 8 == 0 && p.lds % 8 == 0 &&
        (!two_sides || p.ldc2 % 8 == 0) &&
        (((uintptr_t)p.C | (uintptr_t)p.C3 | (uintptr_t)p.S0 | (two_sides ? (uintptr_t)p.C2 | (uintptr_t)p.S1 : 0)) &
         15) == 0) {
      wait_loads_barrier<0>();
      constexpr int PITCH = 144;              // 32 fp32 columns + 16 bytes of padding
      static_assert(NT / 64 * 16 * PITCH <= STAGE, "patches fit in stage 0");
      char* patch = st0 + wave * 16 * PITCH;
      const int prow = lane >> 2;             // this lane's patch row
      const int pcol = (lane & 3) * 8;        // and first of its 8 columns
      static_for<0, TM>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        static_for<0, TN>([&](auto jc) __attribute__((always_inline)) {
          constexpr int j = decltype(jc)::value;
          const int n = n0 + wn * WN + j * 32 + pcol;
          static_for<0, 2>([&](auto hc) __attribute__((always_inline)) {
            constexpr int h = decltype(hc)::value;
            // accumulator registers 8h .. 8h+7 are rows 16h .. 16h+15 of the fragment
            static_for<0, 8>([&](auto rc) __attribute__((always_inline)) {
              constexpr int r = 8 * h + decltype(rc)::value;
              const int row = 8 * ((r >> 2) & 1) + 4 * (lane >> 5) + (r & 3);
              *reinterpret_cast<float*>(patch + row * PITCH + (lane & 31) * 4) = acc[i][j][r];
            });
            // one wave's LDS operations complete in order: the reads see the writes
            const u32x4 d0 = *reinterpret_cast<const u32x4*>(patch + prow * PITCH + pcol * 4);
            const u32x4 d1 = *reinterpret_cast<const u32x4*>(patch + prow * PITCH + pcol * 4 + 16);
            const int m = m0 + wm * WM + i * 32 + 16 * h + prow;
            if (m < p.M && n < p.N) {
              float dh[8];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                dh[e] = __uint_as_float(d0[e]);
                dh[4 + e] = __uint_as_float(d1[e]);
              }
              const u32x4 sa = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.S0) + (int64_t)m * p.lds + n);
              u32x4 sb = {0, 0, 0, 0};
              if (two_sides) sb = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.S1) + (int64_t)m * p.lds + n);
              u32x4 o0, o2, o3;
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                float v0[2], v2[2] = {0.0f, 0.0f}, v3[2];
#pragma unroll
                for (int hw = 0; hw < 2; ++hw) {
                  const int e = 2 * w + hw;
                  const float a = bf2f((uint16_t)(sa[w] >> (16 * hw)));
                  if constexpr (EPI == EPI_SWIGLU_BWD) {
                    const float u = bf2f((uint16_t)(sb[w] >> (16 * hw)));
                    const float s = sigmoidf_(a);
                    const float sg = a * s;
                    v0[hw] = dh[e] * u * (s + sg * (1.0f - s));
                    v2[hw] = dh[e] * sg;
                    v3[hw] = sg * u;
                  } else {
                    v0[hw] = dh[e] * act_grad(p.act, a);
                    v3[hw] = act_fwd(p.act, a);
                  }
                }
                // neighbouring columns: one conversion per pair
                o0[w] = f2bf2(v0[0], v0[1]);
                o2[w] = f2bf2(v2[0], v2[1]);
                o3[w] = f2bf2(v3[0], v3[1]);
              }
              *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.C) + (int64_t)m * p.ldc + n) = o0;
              if (two_sides) *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.C2) + (int64_t)m * p.ldc2 + n) = o2;
              *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.C3) + (int64_t)m * p.ldc3 + n) = o3;
            }
          });
        });
      });
      return;
    }
  }
  // fp32 rows (partials): the same per-wave patch, 16-byte stores of 128-byte
  // row pieces, rows optionally remapped through c_rows.
  if constexpr (std::is_same<OutT, float>::value && EPI == EPI_STORE && !DUAL && NT / 64 * 32 * 144 <= STAGE) {
    if (!p.C2 && !p.cpk && p.N % 4 == 0 && p.ldc % 4 == 0 && ((uintptr_t)p.C & 15) == 0) {
      wait_loads_barrier<0>();
      constexpr int PITCH = 144;              // 128 + 16 bytes of padding
      static_assert(NT / 64 * 32 * PITCH <= STAGE, "patches fit in stage 0");
      char* patch = st0 + wave * 32 * PITCH;
      static_for<0, TM>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        int crow[4];                          // destination rows of this lane's four stores
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + wm * WM + i * 32 + q * 8 + (lane >> 3);
          crow[q] = m >= p.M ? -1 : (p.c_rows ? p.c_rows[m] : m);
        }
        static_for<0, TNO>([&](auto jc) __attribute__((always_inline)) {
          constexpr int j = decltype(jc)::value;
          const int ncol = n0 + wn * WN + j * 32;
          static_for<0, 16>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            *reinterpret_cast<float*>(patch + row * PITCH + (lane & 31) * 4) = acc[i][j][r];
          });
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = q * 8 + (lane >> 3);
            const int cc = (lane & 7) * 4;
            const u32x4 v = *reinterpret_cast<const u32x4*>(patch + row * PITCH + cc * 4);
            if (crow[q] >= 0 && ncol + cc < p.N)
              *reinterpret_cast<u32x4*>(reinterpret_cast<float*>(p.C) + (int64_t)crow[q] * p.ldc + ncol + cc) = v;
          }
        });
      });
      return;
    }
  }
  static_for<0, TM>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    static_for<0, TNO>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      const int n = n0 + wn * (DUAL ? WN / 2 : WN) + j * 32 + (lane & 31);
      if (n < p.N) {
        static_for<0, 16>([&](auto rc) __attribute__((always_inline)) {
          constexpr int r = decltype(rc)::value;
          const int m = mrow + i * 32 + 8 * (r >> 2) + (r & 3);
          const int mo = m < p.M && p.c_rows ? p.c_rows[m] : m;
          if (m < p.M && mo >= 0) {
            if constexpr (DUAL) epilogue_elem<EPI, OutT, uint16_t>(p, mo, n, acc[i][j][r], acc[i][j + TNO][r]);
            else epilogue_elem<EPI, OutT, uint16_t>(p, mo, n, acc[i][j][r], 0.0f);
          }
        });
      }
    });
  });
}

// Column walk for a short contraction (K <= NKT * 64) with a bf16 output:
// the grouped down GEMM of the MoE block, whose K is one rank's slice of an
// expert's hidden size.  There a BM x BN tile does only BM * BN * K * 2
// flops per BM * BN * 2 bytes it stores, so a workgroup per tile pays its
// start-up (operand loads, pipeline fill) for very little work.  Here one
// workgroup owns a BM-row tile and walks every BN-column tile of N: the A rows
// (all of K) are loaded into LDS once, and per column tile only B is loaded,
// the MFMAs run over the k-substeps that hold data, and the tile is stored
// through a per-wave LDS patch as 16-byte row pieces.  The next column tile's
// B is loaded into registers while the current tile's MFMAs run and written
// to LDS after them, and the stores drain while the next tile computes
// (buffer stores: a masked lane gets an out-of-range offset instead of a
// branch).
// Grouped mode and row tables as in gemm_tile_kernel (tile_expert, a_rows,
// c_rows).
// NS: 16-value k-substeps run per column tile (K0 <= 16 * NS; substeps past K0
// read zeros).
template <int BM, int BN, int WGM, int WGN, int NS>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_walk_kernel(const GemmParams p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int NKT = (NS + NSUB - 1) / NSUB;  // k-tiles of 64 held in LDS
  static_assert(NS >= 2 && NS % 2 == 0 && NKT <= 2, "two to eight substeps, an even number");
  using TA = OpTile<BM, true, false, NT>;
  using TB = OpTile<BN, false, false, NT>;
  constexpr int PITCH = 80;                   // bytes per patch row: 64 + 16 of padding
  constexpr int NRD = TM + TN * 2;            // LDS fragment reads per substep
  __shared__ __attribute__((aligned(1024))) char sa0[TA::BYTES];
  __shared__ __attribute__((aligned(1024))) char sa1[NKT > 1 ? TA::BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char sb0[TB::BYTES];
  __shared__ __attribute__((aligned(1024))) char sb1[NKT > 1 ? TB::BYTES : 16];
  __shared__ __attribute__((aligned(16))) char patches[NT / 64 * 32 * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN;
  const int wn = wave % WGN;
  const int mt = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = mt * BM;
  const uint16_t* gB = reinterpret_cast<const uint16_t*>(p.B0);
  if (p.tile_expert) {
    const int ex = p.tile_expert[mt];
    if (ex < 0) return;
    gB += ex * p.b_expert_stride;
  }

  TA ta;
  TB tb;
  if (p.a_rows) ta.setup_rows(tid, m0, p.M, p.lda, p.a_rows);
  else ta.setup(tid, m0, p.M, p.lda);
  auto issue_a = [&](int kt, char* st) {
    const int kvalid = p.K0 - kt * TBK;
    const uint16_t* a = reinterpret_cast<const uint16_t*>(p.A0);
    if (kvalid > 0) a += (p.a_rows ? 0 : (int64_t)m0 * p.lda) + kt * TBK;
    ta.issue(a, a, kvalid, st, wave);
  };
  auto issue_b = [&](int kt, int n0, char* st) {
    const int kvalid = p.K0 - kt * TBK;
    const uint16_t* b = gB;
    if (kvalid > 0) b += (int64_t)kt * TBK * p.ldb + n0;
    tb.issue(b, b, kvalid, st, wave);
  };

  int ao0[TM], ao1[TM], bo0[TN], bo1[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) frag_offsets<BM, true, false>(wm * WM + i * 32, lane, &ao0[i], &ao1[i]);
#pragma unroll
  for (int j = 0; j < TN; ++j) frag_offsets<BN, false, false>(wn * WN + j * 32, lane, &bo0[j], &bo1[j]);

  // byte offsets of the destination rows of this lane's two stores per
  // 32-row fragment (the same for every column tile; below 2^31, which the
  // host checks); OOB: not stored
  uint32_t crow[TM][2];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int m = m0 + wm * WM + i * 32 + q * 16 + (lane >> 2);
      const int r = m >= p.M ? -1 : (p.c_rows ? p.c_rows[m] : m);
      crow[i][q] = r < 0 ? OOB : (uint32_t)r * (uint32_t)(p.ldc * 2);
    }
  const __amdgpu_buffer_rsrc_t cr = __builtin_amdgcn_make_buffer_rsrc(p.C, 0, 0x7FFFFFFF, 0x00020000);
  char* patch = patches + wave * 32 * PITCH;

  tb.setup(tid, 0, p.N, p.ldb);
  issue_a(0, sa0);
  if constexpr (NKT > 1) issue_a(1, sa1);
  issue_b(0, 0, sb0);
  if constexpr (NKT > 1) issue_b(1, 0, sb1);
  wait_loads_barrier<0>();
  // the same wait, visible to the compiler: with the LDS-bound loads known to
  // be complete it puts no wait for them before the loop's fragment reads
  // (one that would also wait for the stores queued behind them)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  const int tiles_n = (p.N + BN - 1) / BN;
  f32x16 acc[TM][TN];
  bf16x8 af[2][TM];
  bf16x8 bf[2][TN];
  u32x4 breg[NKT][TB::NL];  // the next column tile's B, in flight during this tile's MFMAs
  for (int tn = 0; tn < tiles_n; ++tn) {
    const int n0 = tn * BN;
    const bool more = tn + 1 < tiles_n;
    if (more) {
      tb.setup(tid, n0 + BN, p.N, p.ldb);
      static_for<0, NKT>([&](auto kc) __attribute__((always_inline)) {
        constexpr int kt = decltype(kc)::value;
        const int kvalid = p.K0 - kt * TBK;
        const uint16_t* b = gB;
        if (kvalid > 0) b += (int64_t)kt * TBK * p.ldb + n0 + BN;
        tb.fetch(b, kvalid, breg[kt]);
      });
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // substep s reads its fragments while the MFMAs of substep s - 1 run
    static_for<0, NS>([&](auto sc) __attribute__((always_inline)) {
      constexpr int st = decltype(sc)::value;
      constexpr int buf = st & 1;
      const char* sa = st / NSUB == 0 ? sa0 : sa1;
      const char* sb = st / NSUB == 0 ? sb0 : sb1;
#pragma unroll
      for (int i = 0; i < TM; ++i) af[buf][i] = read_frag<BM, true, false>(sa, ao0[i], ao1[i], st % NSUB);
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[buf][j] = read_frag<BN, false, false>(sb, bo0[j], bo1[j], st % NSUB);
      if constexpr (st > 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf ^ 1][i], bf[buf ^ 1][j], acc[i][j], 0, 0, 0);
        interleave<TM * TN, NRD, 0, 0>();
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    constexpr int lb = (NS - 1) & 1;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[lb][i], bf[lb][j], acc[i][j], 0, 0, 0);

    // every wave has read this tile's B: put the next one in its place
    wait_loads_barrier<63>();
    if (more) {
      tb.put(sb0, tid, breg[0]);
      if constexpr (NKT > 1) tb.put(sb1, tid, breg[NKT - 1]);
    }

    // epilogue: accumulator register r of fragment (i, j) is row
    // 8(r/4) + 4(lane/32) + r%4, column lane%32; through the patch each lane
    // stores 16 bytes of one row (8 columns)
    static_for<0, TM>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      static_for<0, TN>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        const int ncol = n0 + wn * WN + j * 32;
        // registers r and r + 1 (r even) are neighbouring rows: one conversion
        // for the pair, then a 2-byte write each
        static_for<0, 8>([&](auto rc) __attribute__((always_inline)) {
          constexpr int r = 2 * decltype(rc)::value;
          const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const uint32_t two = f2bf2(acc[i][j][r], acc[i][j][r + 1]);
          *reinterpret_cast<uint16_t*>(patch + row * PITCH + (lane & 31) * 2) = (uint16_t)two;
          *reinterpret_cast<uint16_t*>(patch + (row + 1) * PITCH + (lane & 31) * 2) = (uint16_t)(two >> 16);
        });
        // one wave's LDS operations complete in order: the reads see the writes
        static_for<0, 2>([&](auto qc) __attribute__((always_inline)) {
          constexpr int q = decltype(qc)::value;
          const int row = q * 16 + (lane >> 2);
          const int cc = (lane & 3) * 8;
          const u32x4 v = *reinterpret_cast<const u32x4*>(patch + row * PITCH + cc * 2);
          const uint32_t off = crow[i][q] == OOB || ncol + cc >= p.N ? OOB : crow[i][q] + (uint32_t)(ncol + cc) * 2;
          __builtin_amdgcn_raw_buffer_store_b128(v, cr, off, 0, 0);
        });
      });
    });
    // the next tile's B is in LDS for every wave (the stores keep draining)
    wait_loads_barrier<63>();
  }
}

template <int BM, int BN, int WGM, int WGN, int NS>
hipError_t launch_walk(const GemmParams& p, hipStream_t s) {
  const int grid = (p.M + BM - 1) / BM;
  hipLaunchKernelGGL((gemm_walk_kernel<BM, BN, WGM, WGN, NS>), dim3(grid), dim3(64 * WGM * WGN), 0, s, p);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int STAGES, bool AKC, bool BKC, bool DUAL, int EPI, typename OutT>
hipError_t launch_tile(const GemmParams& p, hipStream_t s) {
  constexpr int BNH = DUAL ? BN / 2 : BN;
  const int grid = ((p.M + BM - 1) / BM) * ((p.N + BNH - 1) / BNH) * p.splitk;
  hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, WGM, WGN, STAGES, AKC, BKC, DUAL, EPI, OutT>), dim3(grid),
                     dim3(64 * WGM * WGN), 0, s, p);
  return hipGetLastError();
}

template <bool AKC, bool BKC, bool DUAL, int EPI, typename OutT>
hipError_t launch_tile_shape(const GemmParams& p, int tile, hipStream_t s) {
  switch (tile) {
    case TILE_256x256:
      return launch_tile<256, 256, TILE_WGM_256, TILE_WGN_256, TILE_STAGES, AKC, BKC, DUAL, EPI, OutT>(p, s);
    case TILE_128x128:
      return launch_tile<128, 128, TILE_WGM_128, TILE_WGN_128, TILE_STAGES, AKC, BKC, DUAL, EPI, OutT>(p, s);
    case TILE_128x128_W8: return launch_tile<128, 128, 4, 2, TILE_STAGES, AKC, BKC, DUAL, EPI, OutT>(p, s);
    default: return hipErrorInvalidValue;
  }
}

bool aligned16(const void* q) { return q == nullptr || ((uintptr_t)q & 15) == 0; }

}  // namespace

// The pipelined kernel needs every 16-byte chunk it loads to be aligned
// and either wholly inside or wholly outside the matrix.
bool gemm_tile_supported(const GemmParams& p, const GemmPlan& plan, GemmKind kind) {
  if (plan.kernel != KERNEL_TILED) return false;
  if (plan.splitk > 1 && (p.tile_expert || p.a_rows || p.c_rows)) return false;
  if (plan.tile != TILE_256x256 && plan.tile != TILE_128x128 && plan.tile != TILE_128x128_W8) return false;
  if (!p.vecA || !p.vecB) return false;
  if (p.lda % 8 || p.ldb % 8 || p.K0 % 8 || p.K1 % 8) return false;
  if (p.lda > (1 << 21) || p.ldb > (1 << 21)) return false;  // per-lane offsets stay below 2^31
  if (!aligned16(p.A0) || !aligned16(p.A1) || !aligned16(p.B0) || !aligned16(p.B1)) return false;
  const bool akc = !(kind == GK_BWD_DW || kind == GK_BWD_DW_DUAL);
  const bool bkc = kind == GK_BWD_DH_SWIGLU || kind == GK_BWD_DH_ACT || kind == GK_BWD_DX;
  if (!akc && p.M % 8) return false;
  if (p.a_rows && (!akc || p.A1 || p.K1)) return false;
  if (p.c_rows && (kind != GK_FWD_STORE || p.C2 || p.cpk)) return false;
  if (!bkc && p.N % 8) return false;
  return true;
}

// The column walk: a forward store GEMM (A k-contiguous, B (K, N)
// n-contiguous) with a bf16 output, K <= 128, every stored byte offset below
// 2^31 (c_max_row: the largest output row plus one).
bool gemm_walk_supported(const GemmParams& p, int64_t c_max_row) {
  GemmPlan plan;
  plan.kernel = KERNEL_TILED;
  plan.tile = TILE_256x256;
  if (!gemm_tile_supported(p, plan, GK_FWD_STORE)) return false;
  if (p.A1 || p.K1 || p.B1 || p.C2 || p.cpk || p.K0 < 1 || p.K0 > 2 * TBK) return false;
  if (p.ldc % 8 || p.ldc < p.N || ((uintptr_t)p.C & 15)) return false;
  return c_max_row * p.ldc * 2 < (int64_t)OOB - 64;
}

hipError_t gemm_walk(const GemmParams& p, hipStream_t s) {
  if (p.K0 <= 32) return launch_walk<256, 256, TILE_WGM_256, TILE_WGN_256, 2>(p, s);
  if (p.K0 <= 64) return launch_walk<256, 256, TILE_WGM_256, TILE_WGN_256, 4>(p, s);
  if (p.K0 <= 96) return launch_walk<256, 256, TILE_WGM_256, TILE_WGN_256, 6>(p, s);
  return launch_walk<256, 256, TILE_WGM_256, TILE_WGN_256, 8>(p, s);
}

hipError_t gemm_tile(const GemmParams& p, const GemmPlan& plan, GemmKind kind, bool out_f32, hipStream_t s) {
  const int t = plan.tile;
  switch (kind) {
    case GK_FWD_STORE:
      return out_f32 ? launch_tile_shape<true, false, false, EPI_STORE, float>(p, t, s)
                     : launch_tile_shape<true, false, false, EPI_STORE, uint16_t>(p, t, s);
    case GK_FWD_ACT: return launch_tile_shape<true, false, false, EPI_ACT, uint16_t>(p, t, s);
    case GK_FWD_SWIGLU: return launch_tile_shape<true, false, true, EPI_SWIGLU, uint16_t>(p, t, s);
    case GK_BWD_DH_SWIGLU: return launch_tile_shape<true, true, false, EPI_SWIGLU_BWD, uint16_t>(p, t, s);
    case GK_BWD_DH_ACT: return launch_tile_shape<true, true, false, EPI_ACT_BWD, uint16_t>(p, t, s);
    case GK_BWD_DW: return launch_tile_shape<false, false, false, EPI_STORE, uint16_t>(p, t, s);
    case GK_BWD_DW_DUAL: return launch_tile_shape<false, false, true, EPI_DUAL_STORE, uint16_t>(p, t, s);
    case GK_BWD_DX: return launch_tile_shape<true, true, false, EPI_STORE, uint16_t>(p, t, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpk
