// Weight-streaming bf16 GEMM for decode-sized token counts (M <= 64) on
// gfx950.
//
// At decode size a rank's matmuls read every weight byte once and do only
// 2*M flops per weight element (M = tokens), so the time is the time to
// stream the (in, out) weight matrix from HBM ("Tensor Parallelism" notes,
// fourth paragraph: one decode token costs weight bytes / HBM bandwidth).
// This kernel is built around keeping HBM busy rather than around MFMA reuse:
//
//  * A workgroup owns CW column groups of NW*32 output columns (gate and up
//    columns together in dual mode), one per wave, and one K range; K is
//    split across workgroups until there is about one workgroup per CU.  The
//    waves walk the same weight rows side by side, so each workgroup reads
//    CW*NW*64 contiguous bytes of every weight row it touches.
//  * The activations of the workgroup's K range (all M rows) are copied once
//    into LDS with direct global->LDS 16-byte loads (whole contiguous rows),
//    with 16 bytes of padding per row so the fragment reads of 32
//    consecutive rows hit distinct banks.  The waves then read their MFMA A
//    operands from LDS instead of each re-reading x from L2.
//  * Weights are (in, out), n-contiguous, while the MFMA wants 8 consecutive
//    k of one column per lane: each wave copies each 16-row weight slab
//    (16-byte loads) into a private 1 KB-per-32-columns LDS tile and reads
//    the operand back with ds_read_b64_tr_b16, which hands every lane 4
//    consecutive rows of one column (two reads per operand).  Rows are 64
//    bytes, so both the copy-in and the transposed reads are conflict-free.
//  * DEPTH k-steps of weight loads stay in flight per wave; the main loop
//    has no workgroup barrier.
//  * When K is split across workgroups, each column group's fp32 partial
//    goes through a workspace with relaxed agent-scope atomics (coherent
//    across the XCDs' L2s) and the last-arriving workgroup adds the splits in
//    split order, so results are bitwise reproducible.
#include <type_traits>

#include "tp_kernels.h"
#include "tp_device.h"
#include "stream_frag.h"

namespace tpk {

template <int MT, int NW, bool DUAL, int DEPTH, int CW, int EPI, typename OutT>
__global__ __launch_bounds__(CW * 64) void gemm_stream_kernel(const GemmParams p) {
  constexpr int NF = DUAL ? 2 * NW : NW;
  constexpr int GCOLS = NW * 32;     // output columns of one column group (one wave)
  constexpr int WCOLS = CW * GCOLS;  // output columns of the workgroup
  constexpr int MP = MT * 32;        // rows of x held in LDS
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int TB = tile_bytes<NW>();
  char* wt = smem;                   // [CW][NF][TB] weight tiles
  char* xs = smem + CW * NF * TB;    // [MP][xrow] activation slice

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nstrips = (p.N + WCOLS - 1) / WCOLS;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int split = id / nstrips;
  const int strip = id - split * nstrips;
  const int n0 = strip * WCOLS + wave * GCOLS;

  int s_begin, s_end;
  split_range(p.K0, p.splitk, split, &s_begin, &s_end);
  const int full_end = min(s_end, p.K0 / 16);   // steps lying entirely inside K
  const int nfull = max(full_end - s_begin, 0);
  const int xrow = nfull * 32 + 16;             // bytes per LDS row of x (+16 padding)

  f32x16 acc[MT][NF];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  WFrag<NF> fr[DEPTH];
  if (nfull > 0) {
    // Weight prefetch first, then the activation slice straight into LDS:
    // MP rows x nfull*16 values, 1 KB per wave instruction.
    static_for<0, DEPTH>([&](auto d) { load_w<NW, DUAL, false>(fr[d], p, min(s_begin + (int)d, full_end - 1), n0, lane); });
    const int rowbytes = nfull * 32;
    const int chunks = (rowbytes + 1023) / 1024;
    const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A0) + s_begin * 16;
    for (int c = wave; c < MP * chunks; c += CW) {
      const int r = c / chunks, q = c - r * chunks;
      const int byte = q * 1024 + lane * 16;
      if (byte < rowbytes) {
        const uint16_t* src = A + (int64_t)min(r, p.M - 1) * p.lda + byte / 2;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(xs + r * xrow + q * 1024), 16, 0,
                                         0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the slice has landed
    __syncthreads();
  }

  // Copy a step's weight slab into this wave's tiles, read the B operands
  // back transposed, read the A operands from the x slice, run the MFMAs.
  // LDS operations of one wave complete in order, so the transposed reads see
  // the writes without a barrier.
  char* my = wt + wave * NF * TB;
  const char* xlane = xs + (lane & 31) * xrow + (lane >> 5) * 16;
  // TAIL: the A operands come from global memory with k >= K zeroed.
  auto mma = [&](const WFrag<NF>& f, int s, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
#pragma unroll
    for (int mat = 0; mat < (DUAL ? 2 : 1); ++mat)
#pragma unroll
      for (int u = 0; u < NW; ++u) *reinterpret_cast<u32x4*>(my + w_lds_off<NW>(mat, u, lane)) = f.b[mat * NW + u];
    bf16x8 bv[NF];
#pragma unroll
    for (int j = 0; j < NF; ++j) bv[j] = read_b_frag(my + j * TB, lane);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      u32x4 a;
      if constexpr (TAIL) a = load_a_tail(p, i, s, lane);
      else a = *reinterpret_cast<const u32x4*>(xlane + i * 32 * xrow + (s - s_begin) * 32);
      const bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
      for (int j = 0; j < NF; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[j], acc[i][j], 0, 0, 0);
    }
  };

  if (nfull > 0) {
    for (int s = s_begin; s < full_end; s += DEPTH) {
      static_for<0, DEPTH>([&](auto d) {
        if (s + (int)d < full_end) mma(fr[d], s + (int)d, std::false_type{});
        load_w<NW, DUAL, false>(fr[d], p, min(s + DEPTH + (int)d, full_end - 1), n0, lane);
      });
    }
  }
  if (s_end > full_end && s_end > s_begin) {  // the partial last k-step of K
    WFrag<NF> ft;
    load_w<NW, DUAL, true>(ft, p, s_end - 1, n0, lane);
    mma(ft, s_end - 1, std::true_type{});
  }

  // ---- split-K across workgroups: each column group is its own tile ---------
  // (one wave per tile from here on; no block barriers below)
  if (p.splitk > 1) {
    const int t = strip * CW + wave;
    if (!splitk_exchange<MT * NF>(p, t, split, lane, &acc[0][0])) return;
  }

  // ---- epilogue --------------------------------------------------------------
  const int mrow = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int n = n0 + j * 32 + (lane & 31);
      if (n >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = i * 32 + mrow + 8 * (r >> 2) + (r & 3);
        if (m < p.M) epilogue_elem<EPI, OutT, uint16_t>(p, m, n, acc[i][j][r], DUAL ? acc[i][j + NW][r] : 0.0f);
      }
    }
}

// LDS bytes the streaming kernel needs for an M-row, K-range-of-`ksteps` launch.
size_t stream_lds_bytes(int M, int ksteps, bool dual) {
  const int mt = M <= 32 ? 1 : 2;
  const int nf = (dual ? 2 : 1) * STREAM_NW;
  return (size_t)STREAM_CW * nf * tile_bytes<STREAM_NW>() + (size_t)mt * 32 * (ksteps * 32 + 16);
}

template <int MT, bool DUAL, int EPI, typename OutT>
static hipError_t launch_stream_mt(const GemmParams& p, const GemmPlan& plan, hipStream_t s) {
  auto kern = gemm_stream_kernel<MT, STREAM_NW, DUAL, STREAM_DEPTH, STREAM_CW, EPI, OutT>;
  const int threads = 64 * STREAM_CW;
  const int nstrips = (p.N + STREAM_WCOLS - 1) / STREAM_WCOLS;
  const int nsteps = (p.K0 + 15) / 16;
  const int max_steps = (nsteps + plan.splitk - 1) / plan.splitk;  // longest split
  const size_t lds = stream_lds_bytes(p.M, max_steps, DUAL);
  static bool attr_set = false;  // one-time opt-in to LDS above 64 KB
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, STREAM_LDS_MAX);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (lds > (size_t)STREAM_LDS_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3(nstrips * plan.splitk), dim3(threads), lds, s, p);
  return hipGetLastError();
}

template <bool DUAL, int EPI, typename OutT>
hipError_t launch_stream(const GemmParams& p, const GemmPlan& plan, hipStream_t s) {
  if (p.M <= 32) return launch_stream_mt<1, DUAL, EPI, OutT>(p, plan, s);
  if (p.M <= STREAM_MAX_M) return launch_stream_mt<2, DUAL, EPI, OutT>(p, plan, s);
  return hipErrorInvalidValue;
}

// The streaming kernel serves the forward layouts (x k-contiguous, weights
// (in, out)); everything else uses the tiled kernel.
hipError_t gemm_stream(const GemmParams& p, const GemmPlan& plan, GemmKind kind, bool out_f32, hipStream_t s) {
  switch (kind) {
    case GK_FWD_STORE:
      return out_f32 ? launch_stream<false, EPI_STORE, float>(p, plan, s)
                     : launch_stream<false, EPI_STORE, uint16_t>(p, plan, s);
    case GK_FWD_ACT: return launch_stream<false, EPI_ACT, uint16_t>(p, plan, s);
    case GK_FWD_SWIGLU: return launch_stream<true, EPI_SWIGLU, uint16_t>(p, plan, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpk
