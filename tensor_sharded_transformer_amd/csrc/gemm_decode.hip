// Weight-streaming bf16 GEMM for decode-sized token counts (M <= 64), with the
// activations pre-packed in MFMA fragment order.
//
// At decode size one rank's matmul reads every weight byte once and does
// only 2*M flops per weight element, so its time is the time to stream the
// (in, out) weight shard from HBM ("Tensor Parallelism" notes, fourth
// paragraph: a decode token costs weight bytes / HBM bandwidth).  Design:
//
//  * A first pass rewrites x (M x K, row-major) so that the A operand of one
//    32x32x16 MFMA (32 rows x 16 k) is 1 KB of contiguous memory in lane
//    order; the streaming kernel then reads each A fragment with one fully
//    coalesced 16-byte load per lane, straight from L2 (x is small and every
//    workgroup re-reads it), and needs no activation copy in LDS.
//  * A workgroup owns NW*32 output columns (gate and up columns together in
//    dual mode, NW*64 contiguous bytes of every weight row) and one K range;
//    its KW waves stream disjoint K sub-ranges of that range, each with DEPTH
//    k-steps of weight and activation loads in flight and no barrier.  K is
//    split across workgroups only until there is about one workgroup per CU,
//    which keeps the cross-workgroup partials small.
//  * Weights are n-contiguous while the MFMA wants 8 consecutive k of one
//    column per lane: each wave copies each 16-row slab into a private LDS
//    tile and reads the operand back with ds_read_b64_tr_b16.
//  * fp8 weights (OCP e4m3 codes with per-column scales) travel the same
//    way at half the bytes: a k-step of one matrix is one 16-byte load per
//    lane, decoded to bf16 in registers (exact) just before the LDS copy;
//    the scales multiply the summed tile before the epilogue.
//  * The waves' accumulators meet in LDS; each wave then owns one output
//    fragment (gate and up together), sums it over the waves in wave order,
//    and takes it through the split-K exchange (last-arriving workgroup adds
//    the splits in split order), so results are bitwise reproducible.
#include <type_traits>

#include "tp_kernels.h"
#include "tp_device.h"
#include "stream_frag.h"

namespace tpk {

namespace {

constexpr int KW = DECODE_KW;
constexpr int NW = DECODE_NW;
constexpr int DEPTH = DECODE_DEPTH;

// Packed A: fragment (step s, m-tile i) is 64 lanes x 16 bytes at
// ((s * MT + i) * 64 + lane) * 16; lane l holds row 32i + l%32, k values
// 16s + 8(l/32) .. +7.  Rows >= M and k >= K are zero.
template <int MT>
__global__ __launch_bounds__(256) void pack_a_kernel(const uint16_t* __restrict__ x, int64_t lda, int M, int K,
                                                     int nsteps, u32x4* __restrict__ out) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  if (gid >= nsteps * MT * 64) return;
  const int lane = gid & 63;
  const int f = gid >> 6;
  const int i = f % MT;
  const int s = f / MT;
  const int m = i * 32 + (lane & 31);
  const int k = s * 16 + (lane >> 5) * 8;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (m < M && k < K) v = *reinterpret_cast<const u32x4*>(x + (int64_t)m * lda + k);
  out[gid] = v;
}

template <int MT, bool DUAL>
constexpr int decode_lds_bytes() {
  constexpr int NF = DUAL ? 2 * NW : NW;
  return KW * NF * tile_bytes<NW>() + KW * MT * NF * 16 * 64 * 4;
}

// One k-step of A (MT fragments) from the packed array.
template <int MT>
__device__ __forceinline__ void load_a(const u32x4* apk, int step, int lane, u32x4 (&a)[MT]) {
#pragma unroll
  for (int i = 0; i < MT; ++i) a[i] = apk[(step * MT + i) * 64 + lane];
}

// Registers of one k-step of weights: NW 16-byte chunks per matrix (bf16),
// one (fp8 codes).
template <bool DUAL, bool F8>
using WRegs = WFrag<F8 ? (DUAL ? 2 : 1) : (DUAL ? 2 * NW : NW)>;

// One k-step of MFMAs: the wave's weight slab goes through its private LDS
// tiles (written row-major, read back transposed) into the B operands; fp8
// codes are decoded to bf16 on the way in.
template <int MT, bool DUAL, bool F8>
__device__ __forceinline__ void mma_step(char* my, int lane, const WRegs<DUAL, F8>& f, const u32x4 (&a)[MT],
                                         f32x16 (&acc)[MT][DUAL ? 2 * NW : NW]) {
  constexpr int NF = DUAL ? 2 * NW : NW;
  constexpr int TB = tile_bytes<NW>();
  if constexpr (F8) {
    static_assert(NW == 2, "fp8 k-step layout assumes 64-column strips");
    // lane: row lane/4, columns 16 (lane%4) .. +15 = bf16 chunks 2 (lane%4) and 2 (lane%4) + 1
    const int row = lane >> 2, c0 = (lane & 3) * 2;
#pragma unroll
    for (int mat = 0; mat < (DUAL ? 2 : 1); ++mat) {
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) fp8x4_to_bf16x4(f.b[mat][q], &w[2 * q], &w[2 * q + 1]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = c0 + h;
        *reinterpret_cast<u32x4*>(my + (mat * NW + c / 4) * TB + row * 64 + (c % 4) * 16) =
            u32x4{w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]};
      }
    }
  } else {
#pragma unroll
    for (int mat = 0; mat < (DUAL ? 2 : 1); ++mat)
#pragma unroll
      for (int u = 0; u < NW; ++u) *reinterpret_cast<u32x4*>(my + w_lds_off<NW>(mat, u, lane)) = f.b[mat * NW + u];
  }
  bf16x8 bv[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) bv[j] = read_b_frag(my + j * TB, lane);
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const bf16x8 av = __builtin_bit_cast(bf16x8, a[i]);
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[j], acc[i][j], 0, 0, 0);
  }
}

// The last, partial k-step of K (packed A is zero past K; weight rows past K
// read as zero).
template <bool DUAL, bool F8, bool TAIL>
__device__ __forceinline__ void load_wregs(WRegs<DUAL, F8>& f, const GemmParams& p, int step, int n0, int lane) {
  if constexpr (F8) load_w8<DUAL, TAIL>(f, p, step, n0, lane);
  else load_w<NW, DUAL, TAIL>(f, p, step, n0, lane);
}

template <int MT, bool DUAL, bool F8>
__device__ __forceinline__ void tail_step(const GemmParams& p, int n0, int step, int lane, char* my,
                                          f32x16 (&acc)[MT][DUAL ? 2 * NW : NW]) {
  WRegs<DUAL, F8> ft;
  u32x4 at[MT];
  load_wregs<DUAL, F8, true>(ft, p, step, n0, lane);
  load_a<MT>(reinterpret_cast<const u32x4*>(p.apk), step, lane, at);
  mma_step<MT, DUAL, F8>(my, lane, ft, at, acc);
}

// Main loop of one wave over k-steps [w_begin, w_end): a ring of DEPTH steps
// of weight and activation loads in flight.  The weights of the first DEPTH
// steps are requested before `ready()` returns (it may wait for the packed
// activations to be published); the activations only after.
//
// Each wave walks its steps from a rotated start, so the workgroups of a
// launch do not all read the same weight rows at the same time (with
// power-of-two row strides that lockstep concentrates on few DRAM banks).
template <int MT, bool DUAL, bool F8, typename Ready>
__device__ __forceinline__ void ring_loop(const GemmParams& p, int n0, int w_begin, int w_end, int rot_seed, int lane,
                                          char* my, f32x16 (&acc)[MT][DUAL ? 2 * NW : NW], Ready&& ready) {
  const u32x4* apk = reinterpret_cast<const u32x4*>(p.apk);
  constexpr int RD = DEPTH;  // (fp8: 8 steps in flight measured no faster than 4)
  const int full_end = min(w_end, p.K0 / 16);  // steps whose weight rows all lie inside K
  const int nw = full_end - w_begin;
  if (nw > 0) {
    const int rot = rot_seed % nw;
    auto phys = [&](int it) {
      const int q = min(it, nw - 1) + rot;
      return w_begin + (q >= nw ? q - nw : q);
    };
    WRegs<DUAL, F8> fr[RD];
    u32x4 fa[RD][MT];
    static_for<0, RD>([&](auto d) { load_wregs<DUAL, F8, false>(fr[d], p, phys(d), n0, lane); });
    ready();
    static_for<0, RD>([&](auto d) { load_a<MT>(apk, phys(d), lane, fa[d]); });
    for (int it = 0; it < nw; it += RD) {
      static_for<0, RD>([&](auto d) {
        if (it + (int)d < nw) mma_step<MT, DUAL, F8>(my, lane, fr[d], fa[d], acc);
        const int st = phys(it + RD + (int)d);
        load_wregs<DUAL, F8, false>(fr[d], p, st, n0, lane);
        load_a<MT>(apk, st, lane, fa[d]);
      });
    }
  } else {
    ready();
  }
  if (w_end > full_end && w_end > w_begin) tail_step<MT, DUAL, F8>(p, n0, w_end - 1, lane, my, acc);
}

// After a workgroup's main loops: the waves' accumulators meet in LDS, wave u
// owns output fragment u (gate and up together) and sums it over the waves
// in wave order, takes it through the split-K exchange (the last-arriving
// split adds the splits in split order, so results are bitwise
// reproducible) and stores it.
template <int MT, bool DUAL, bool F8, int EPI, typename OutT>
__device__ __forceinline__ void decode_finish(const GemmParams& p, int strip, int split, int nsplit, int lane, int wave,
                                              char* my, float* red, f32x16 (&acc)[MT][DUAL ? 2 * NW : NW]) {
  constexpr int NF = DUAL ? 2 * NW : NW;
  constexpr int NACC = MT * NF;
  constexpr int UNITS = MT * NW;
  constexpr int TB = tile_bytes<NW>();
  const int n0 = strip * (NW * 32);
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[(((wave * NACC) + i * NF + j) * 16 + r) * 64 + lane] = acc[i][j][r];
  __syncthreads();
  if (wave >= UNITS) return;
  const int ui = wave / NW;  // m-tile
  const int uj = wave % NW;  // column fragment
  constexpr int NOUT = DUAL ? 2 : 1;
  f32x16 out[NOUT];
#pragma unroll
  for (int o = 0; o < NOUT; ++o) {
    const int a = ui * NF + uj + o * NW;
#pragma unroll
    for (int r = 0; r < 16; ++r) out[o][r] = 0.0f;
#pragma unroll
    for (int w = 0; w < KW; ++w)
#pragma unroll
      for (int r = 0; r < 16; ++r) out[o][r] += red[(((w * NACC) + a) * 16 + r) * 64 + lane];
  }

  if (nsplit > 1) {
    if (!splitk_exchange<NOUT>(p, strip * UNITS + wave, split, nsplit, lane, out)) return;
  }
  if constexpr (F8) {  // per-column scales of the fp8 weights (lane % 32 is the tile column)
    const int nc = min(n0 + uj * 32 + (lane & 31), p.N - 1);
    const float s0 = p.bscale0[nc];
    const float s1 = DUAL ? p.bscale1[nc] : 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      out[0][r] *= s0;
      if constexpr (DUAL) out[NOUT - 1][r] *= s1;
    }
  }

  // Common case (a bf16 output and nothing else to write): the 32x32 tile
  // goes through this wave's LDS weight tile (idle now) so the global stores
  // are 16 bytes per lane (two per tile), row-major or packed.
  if constexpr (std::is_same<OutT, uint16_t>::value && (EPI == EPI_STORE || EPI == EPI_ACT || EPI == EPI_SWIGLU)) {
    if (!p.C2 && p.N % 8 == 0 && (p.cpk || (p.ldc % 8 == 0 && ((uintptr_t)p.C & 15) == 0))) {
      constexpr int PITCH = 64;
      static_assert(32 * PITCH <= NF * TB, "patch fits in the wave's weight tiles");
      const int ncol = n0 + uj * 32;
      const int nl = ncol + (lane & 31);
      float bias = 0.0f;
      if constexpr (EPI == EPI_ACT) {
        if (p.bias && nl < p.N) bias = bf2f(reinterpret_cast<const uint16_t*>(p.bias)[nl]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v;
        if constexpr (EPI == EPI_STORE) v = out[0][r];
        else if constexpr (EPI == EPI_ACT) v = act_fwd(p.act, out[0][r] + bias);
        else v = out[0][r] * sigmoidf_(out[0][r]) * out[NOUT - 1][r];
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        *reinterpret_cast<uint16_t*>(my + row * PITCH + (lane & 31) * 2) = f2bf(v);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = q * 16 + (lane >> 2);
        const int cc = (lane & 3) * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(my + row * PITCH + cc * 2);
        const int m = ui * 32 + row;
        const int nn = ncol + cc;
        if (m < p.M && nn < p.N) {
          if (p.cpk) {
            const int64_t chunk = ((int64_t)(nn >> 4) * p.cpk_mt + (m >> 5)) * 64 + (m & 31) + ((nn >> 3) & 1) * 32;
            reinterpret_cast<u32x4*>(p.cpk)[chunk] = v;
          } else {
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.C) + (int64_t)m * p.ldc + nn) = v;
          }
        }
      }
      return;
    }
  }
  const int n = n0 + uj * 32 + (lane & 31);
  if (n >= p.N) return;
  const int mrow = ui * 32 + 4 * (lane >> 5);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = mrow + 8 * (r >> 2) + (r & 3);
    if (m < p.M) epilogue_elem<EPI, OutT, uint16_t>(p, m, n, out[0][r], DUAL ? out[NOUT - 1][r] : 0.0f);
  }
}

template <int MT, bool DUAL>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[MT][DUAL ? 2 * NW : NW]) {
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < (DUAL ? 2 * NW : NW); ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// The k-steps of wave `wave` in split `split` of `nsplit`.
__device__ __forceinline__ void wave_range(const GemmParams& p, int nsplit, int split, int wave, int* w_begin,
                                           int* w_end) {
  int s_begin, s_end;
  split_range(p.K0, nsplit, split, &s_begin, &s_end);
  *w_begin = s_begin + (s_end - s_begin) * wave / KW;
  *w_end = s_begin + (s_end - s_begin) * (wave + 1) / KW;
}

// Workgroup tile i of a decode GEMM: split_base K splits of every column
// strip (each XCD gets a contiguous block of those), then the extra splits of
// the slow-class strips.
__device__ __forceinline__ void decode_tile(const GemmParams& p, int nstrips, int i, int* strip, int* split,
                                            int* nsplit) {
  const int base_tiles = nstrips * p.split_base;
  if (i < base_tiles) {
    const int id = xcd_remap(i, base_tiles);
    *split = id / nstrips;
    *strip = id - *split * nstrips;
  } else {
    const int e = i - base_tiles;
    *strip = p.slow_first + 8 * (e / p.slow_extra);
    *split = p.split_base + e % p.slow_extra;
  }
  *nsplit = p.split_base + (p.slow_extra > 0 && (*strip & 7) == p.slow_first ? p.slow_extra : 0);
}

template <int MT, bool DUAL, bool F8, int EPI, typename OutT>
__global__ __launch_bounds__(KW * 64) void gemm_decode_kernel(const GemmParams p) {
  constexpr int NF = DUAL ? 2 * NW : NW;
  constexpr int TB = tile_bytes<NW>();
  __shared__ __attribute__((aligned(16))) char smem[decode_lds_bytes<MT, DUAL>()];
  // Every parameter the kernel reads, loaded in one batch up front: each
  // dependent round trip to the argument buffer costs about a microsecond.
  __asm__ volatile("" ::"s"(p.B0), "s"(p.B1), "s"(p.apk), "s"(p.ldb), "s"(p.N), "s"(p.K0), "s"(p.M),
                   "s"(p.splitk), "s"(p.partials), "s"(p.counters), "s"(p.C), "s"(p.ldc), "s"(p.cpk),
                   "s"(p.cpk_mt), "s"(p.split_base), "s"(p.slow_first), "s"(p.slow_extra));
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nstrips = (p.N + NW * 32 - 1) / (NW * 32);
  int strip, split, nsplit;
  decode_tile(p, nstrips, blockIdx.x, &strip, &split, &nsplit);
  int w_begin, w_end;
  wave_range(p, nsplit, split, wave, &w_begin, &w_end);
  char* my = smem + wave * NF * TB;
  float* red = reinterpret_cast<float*>(smem + KW * NF * TB);
  f32x16 acc[MT][NF];
  zero_acc<MT, DUAL>(acc);
  ring_loop<MT, DUAL, F8>(p, strip * NW * 32, w_begin, w_end, strip * 7 + wave * 3, lane, my, acc, [] {});
  decode_finish<MT, DUAL, F8, EPI, OutT>(p, strip, split, nsplit, lane, wave, my, red, acc);
}

// Column strips whose weight bytes have address bits 7..9 equal to 3 stream
// about 30% slower than the others on this chip (measured per wave, for the
// (d, 3584) gate/up and (3584, d) down shards alike): with split-K on, they
// get extra K splits.  Fills split_base/slow_first/slow_extra/splitk and
// returns the number of workgroups.
constexpr uintptr_t SLOW_CLASS = 3;

int decode_split(GemmParams& p, const GemmPlan& plan) {
  const int nstrips = (p.N + DECODE_WCOLS - 1) / DECODE_WCOLS;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(p.B0), b1 = p.B1 ? reinterpret_cast<uintptr_t>(p.B1) : b0;
  p.split_base = plan.splitk;
  p.slow_first = (int)((SLOW_CLASS - (b0 >> 7)) & 7);
  const int nslow = p.slow_first < nstrips ? (nstrips - p.slow_first + 7) / 8 : 0;
  // only while the grid stays within one workgroup per CU, and for splits of
  // at most 4 (finer splits already keep the slow strips' tiles short)
  const bool extra = !p.b_fp8 && plan.splitk > 1 && plan.splitk <= 4 && ((b0 ^ b1) >> 7 & 7) == 0 && nslow > 0 &&
                     nstrips * plan.splitk + nslow * DECODE_SLOW_EXTRA <= 256;
  p.slow_extra = extra ? DECODE_SLOW_EXTRA : 0;
  p.splitk = plan.splitk + p.slow_extra;
  return nstrips * plan.splitk + (extra ? nslow * p.slow_extra : 0);
}

template <int MT, bool DUAL, int EPI, typename OutT>
hipError_t launch_decode_mt(const GemmParams& p, const GemmPlan& plan, hipStream_t s) {
  if (!p.apk_ready && p.K0 > 0) {  // (an empty contraction has nothing to pack)
    const int nsteps = (p.K0 + 15) / 16;
    const int npk = nsteps * MT * 64;
    hipLaunchKernelGGL(pack_a_kernel<MT>, dim3((npk + 255) / 256), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(p.A0), p.lda, p.M, p.K0, nsteps,
                       reinterpret_cast<u32x4*>(p.apk));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  GemmParams pd = p;
  const int nwg = decode_split(pd, plan);
  if (p.b_fp8)
    hipLaunchKernelGGL((gemm_decode_kernel<MT, DUAL, true, EPI, OutT>), dim3(nwg), dim3(KW * 64), 0, s, pd);
  else
    hipLaunchKernelGGL((gemm_decode_kernel<MT, DUAL, false, EPI, OutT>), dim3(nwg), dim3(KW * 64), 0, s, pd);
  return hipGetLastError();
}

template <bool DUAL, int EPI, typename OutT>
hipError_t launch_decode(const GemmParams& p, const GemmPlan& plan, hipStream_t s) {
  if (!p.apk) return hipErrorInvalidValue;
  if (p.M <= 32) return launch_decode_mt<1, DUAL, EPI, OutT>(p, plan, s);
  if (p.M <= STREAM_MAX_M) return launch_decode_mt<2, DUAL, EPI, OutT>(p, plan, s);
  return hipErrorInvalidValue;
}

}  // namespace

size_t decode_pack_bytes(int M, int K) {
  const int mt = M <= 32 ? 1 : 2;
  return (size_t)((K + 15) / 16) * mt * 64 * 16;
}

// Split-K exchange tiles of a decode launch: one per output fragment.
size_t decode_tiles(int M, int N) {
  const int mt = M <= 32 ? 1 : 2;
  return (size_t)((N + DECODE_WCOLS - 1) / DECODE_WCOLS) * mt * DECODE_NW;
}

hipError_t gemm_decode(const GemmParams& p, const GemmPlan& plan, GemmKind kind, bool out_f32, hipStream_t s) {
  switch (kind) {
    case GK_FWD_STORE:
      return out_f32 ? launch_decode<false, EPI_STORE, float>(p, plan, s)
                     : launch_decode<false, EPI_STORE, uint16_t>(p, plan, s);
    case GK_FWD_ACT: return launch_decode<false, EPI_ACT, uint16_t>(p, plan, s);
    case GK_FWD_SWIGLU: return launch_decode<true, EPI_SWIGLU, uint16_t>(p, plan, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpk
