// Weight-streaming bf16 GEMM for decode-sized token counts (M <= 64) over
// weights stored once in MFMA fragment order.
//
// At decode size a rank's matmul reads every weight byte once for only 2*M
// flops per weight, so its time is the time to stream the weight shard from
// HBM ("Tensor Parallelism" notes, fourth paragraph: a decode token costs
// weight bytes / HBM bandwidth).  With (in, out) row-major weights a
// workgroup that owns a few output columns reads short pieces of many rows,
// so the K range has to be split across workgroups and their partial sums
// exchanged.  Here the weights are rearranged once, ahead of the decode steps,
// into the order the matrix cores consume them:
//
//  * Packed weights W (K, N): 1 KB chunks, one per (32-row k-block b,
//    16-column strip s), k-block-major: chunk (s, b) sits at index
//    b * nstrips + s, and lane l's 16 bytes are W[32b + 8(l/16) + j][16s + l%16],
//    j = 0..7, which is exactly the B operand of v_mfma_f32_16x16x32_bf16.
//    Entries outside K x N are zero.  Every workgroup walks the k-blocks in
//    the same order, so at any moment the workgroups of a launch read
//    neighbouring chunks of one contiguous region (the access pattern of a
//    copy), which keeps the HBM channels evenly loaded.
//  * Packed activations X (M, K): chunk (k-block b, 16-row tile i) at index
//    b * mt + i, lane l holding X[16i + l%16][32b + 8(l/16) + j] (the A
//    operand); rows >= M and k >= K are zero.  A packing pass writes it (x is
//    small and every workgroup reads all of it from L2); the SwiGLU epilogue
//    of the column GEMM writes h straight into it for the row GEMM.  When a
//    launch reads few activation bytes in all (K a multiple of 32), the
//    packing launch costs more than it saves, and the fragments are read
//    from row-major x instead (16 bytes of one row per lane; two k-blocks
//    share each 128-byte line of a row).  Larger launches with two or more
//    weight fragments per k-block load row-major x in whole lines (8 rows x
//    64 columns per load) and turn them into the same fragments through the
//    wave's LDS slot, a 64-row k-pair per ring step.
//
// A workgroup owns NS strips (NS * 16 output columns, gate and up together in
// dual mode) and a K range.  Its KW waves each stream a contiguous share of
// that range with DEPTH k-blocks of loads in flight, straight into the MFMA
// operand registers (no LDS on the way).  A CU keeps only so many loads in
// flight, and the activation chunks (L2 hits) take their share of them:
// per k-block a workgroup reads 128 bytes of activations per k for 32 * NS
// (dual: 64 * NS) bytes of weights, so the planner takes two strips per
// workgroup and splits K across workgroups until the grid fills the CUs,
// which halves the activation loads per weight byte of the one-strip,
// whole-K arrangement.  At the end the waves' accumulators meet in LDS and
// are summed in wave order; with K split, each wave publishes all of its
// output tiles at once, takes one arrival ticket, and the last split to
// arrive adds the splits in split order.  Each output tile then goes through
// an LDS patch so the stores are 16 bytes per lane.  Every sum has a fixed
// order, so results are bitwise reproducible.
//
// fp8 weights (OCP e4m3 codes, one fp32 scale per output column) use the
// same scheme at half the bytes: a chunk covers a 64-row k-pair of a strip,
// lane l's 16 bytes being the codes of k-block 2p (bytes 0..7) and 2p + 1
// (bytes 8..15) at rows 8(l/16) + j, column l%16 -- one load feeds two MFMAs
// once the codes are widened to bf16 in registers (exact: every e4m3 value is
// a bf16 value).  A ring step is then a k-pair, with twice the activation
// chunks; the scales multiply the finished sums in the epilogue.
#include <type_traits>

#include "tp_kernels.h"
#include "tp_device.h"

namespace tpk {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int DEPTH = PACKED_DEPTH;     // k-blocks of loads in flight per wave
constexpr int PATCH = 1280;             // bytes of a wave's store patch (16 fp32 rows of 80 bytes)

// Fragments per wave that meet in LDS per reduction pass (at most four, so
// the reduction area stays at 64 KiB per 4 waves; a strip's gate and up
// fragments go together).  Each extra pass costs two barriers on the
// launch's critical path.
template <int WF>
constexpr int pass_frags() {
  return WF <= 4 ? WF : 4;
}
// Per wave: its reduction slot (one pass of PF fragments per tile), which
// during the main loop also holds the wave's x staging (XM_STAGED: the 16-row
// tiles of one 64-row k-pair, MT x 2 KB).
template <int MT, int PF, int XM>
constexpr int packed_slot_bytes() {
  return XM == 2 && PF < 2 ? MT * 2048 : MT * PF * 1024;
}
template <int MT, int PF, int KW, int XM>
constexpr int packed_lds_bytes() {
  return KW * packed_slot_bytes<MT, PF, XM>() + KW * PATCH;  // cross-wave reduction (one pass) + per-wave store patch
}

// One k-block of one wave: NF weight fragments and MT activation fragments.
template <int MT, int NF>
struct KStep {
  u32x4 b[NF];
  u32x4 a[MT];
};

template <int MT, int NF>
__device__ __forceinline__ void load_step(KStep<MT, NF>& r, const u32x4* const (&bp)[NF], const u32x4* ap, int kb,
                                          int64_t kb_stride) {
#pragma unroll
  for (int f = 0; f < NF; ++f) r.b[f] = bp[f][kb * kb_stride];
#pragma unroll
  for (int i = 0; i < MT; ++i) r.a[i] = ap[((int64_t)kb * MT + i) * 64];
}

// The same with the activation fragments read from row-major x: lane l of
// tile i holds row 16 i + l % 16, columns 32 b + 8 (l / 16) .. + 7 (16 bytes)
// of k-block b (ring step kb; with fp8 codes a ring step is the k-pair 2 kb,
// 2 kb + 1, tiles of k-block 2 kb first); rows past M (row_ok false) hold
// zeros.
template <int MT, int NF, bool F8>
__device__ __forceinline__ void load_step_rm(KStep<F8 ? 2 * MT : MT, NF>& r, const u32x4* const (&bp)[NF],
                                             const uint16_t* xl, int64_t lda16, const bool (&row_ok)[MT], int kb,
                                             int64_t kb_stride) {
  constexpr int AT = F8 ? 2 * MT : MT;
#pragma unroll
  for (int f = 0; f < NF; ++f) r.b[f] = bp[f][kb * kb_stride];
#pragma unroll
  for (int c = 0; c < AT; ++c) {
    const int i = c % MT, b = (F8 ? 2 * kb : kb) + c / MT;
    r.a[c] = row_ok[i] ? *reinterpret_cast<const u32x4*>(xl + i * lda16 + b * 32) : u32x4{0u, 0u, 0u, 0u};
  }
}

// One k-pair (k-blocks 2 kp, 2 kp + 1) with the activations as whole 128-byte
// lines of row-major x: load c brings rows 8 c .. 8 c + 7 (lane l: row
// 8 c + l / 8, columns 64 kp + 8 (l % 8) .. + 7), rows past M as zeros;
// weights r.b[h * NF + f] for k-block 2 kp + h.
template <int MT, int NF>
__device__ __forceinline__ void load_pair_x(KStep<2 * MT, 2 * NF>& r, const u32x4* const (&bp)[NF],
                                            const uint16_t* xs, int64_t lda8, const bool (&line_ok)[2 * MT], int kp,
                                            int64_t kb_stride) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int f = 0; f < NF; ++f) r.b[h * NF + f] = bp[f][(int64_t)(2 * kp + h) * kb_stride];
#pragma unroll
  for (int c = 0; c < 2 * MT; ++c)
    r.a[c] = line_ok[c] ? *reinterpret_cast<const u32x4*>(xs + c * lda8 + kp * 64) : u32x4{0u, 0u, 0u, 0u};
}

// The staged k-pair through the wave's LDS slot: the lines go in with row R's
// eight 16-byte pieces rotated by R % 8 (piece q of row R at R * 128 +
// 16 (q ^ R % 8)), so that both the line writes and the fragment reads of
// eight consecutive rows hit eight different bank groups; the fragments read
// back are exactly the packed-activation chunks (lane l: row 16 i + l % 16,
// columns 32 h + 8 (l / 16) .. + 7 of the pair).
template <int MT, int NF>
__device__ __forceinline__ void mma_pair_staged(const KStep<2 * MT, 2 * NF>& r, char* stg, int lane,
                                                f32x4 (&acc)[MT][NF]) {
#pragma unroll
  for (int c = 0; c < 2 * MT; ++c) {
    const int row = 8 * c + (lane >> 3);
    *reinterpret_cast<u32x4*>(stg + row * 128 + (((lane & 7) ^ (lane >> 3)) << 4)) = r.a[c];
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 af[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int row = 16 * i + (lane & 15);
      af[i] = *reinterpret_cast<const u32x4*>(stg + row * 128 + (((4 * h + (lane >> 4)) ^ (lane & 7)) << 4));
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int f = 0; f < NF; ++f)
        acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                           __builtin_bit_cast(bf16x8, r.b[h * NF + f]), acc[i][f], 0,
                                                           0, 0);
  }
}

// Four fp8 codes -> four bf16 values in two words, low code first.
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  typedef float f32x2_ __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_ __attribute__((ext_vector_type(2)));
  const f32x2_ a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_ b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2_));
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2_));
}

// One k-pair of fp8 weights: r.a holds the MT tiles of k-block 2p, then of 2p + 1.
template <int MT, int NF>
__device__ __forceinline__ void mma_step_f8(const KStep<2 * MT, NF>& r, f32x4 (&acc)[MT][NF]) {
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    u32x4 b[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t w0, w1, w2, w3;
      e4m3x4_to_bf16(r.b[f][2 * h], w0, w1);
      e4m3x4_to_bf16(r.b[f][2 * h + 1], w2, w3);
      b[h] = u32x4{w0, w1, w2, w3};
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < MT; ++i)
        acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.a[h * MT + i]),
                                                           __builtin_bit_cast(bf16x8, b[h]), acc[i][f], 0, 0, 0);
  }
}

template <int MT, int NF>
__device__ __forceinline__ void mma_step(const KStep<MT, NF>& r, f32x4 (&acc)[MT][NF]) {
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const bf16x8 av = __builtin_bit_cast(bf16x8, r.a[i]);
#pragma unroll
    for (int f = 0; f < NF; ++f)
      acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, r.b[f]), acc[i][f], 0, 0, 0);
  }
}

// Split-K exchange of the NU x NB 16x16 tiles one wave owns (ticket t of the
// launch: workgroup group and wave, the same for every split): publish this
// split's tiles, take one arrival ticket; the last split to arrive replaces
// v by the sum over all splits in split order and re-zeroes the ticket.
// Per ticket: [split][tile][lane][4 floats], 1 KB per tile.
template <int NT>
__device__ __forceinline__ bool packed_exchange(const PackedParams& p, int t, int split, int lane, f32x4 (&v)[NT]) {
  constexpr uint32_t SPLIT_BYTES = NT * 1024;
  const float* base = p.partials + (int64_t)t * p.splitk * NT * 256;
  const __amdgpu_buffer_rsrc_t r = splitk_rsrc(base, SPLIT_BYTES * (uint32_t)p.splitk);
#pragma unroll
  for (int a = 0; a < NT; ++a) splitk_store(r, split * SPLIT_BYTES + a * 1024 + lane * 16, v[a]);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this lane's partial stores are complete
  __builtin_amdgcn_wave_barrier();
  int prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(&p.counters[t], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0);
  if (prev != p.splitk - 1) return false;
  f32x4 sum[NT];
#pragma unroll
  for (int a = 0; a < NT; ++a) sum[a] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int sp = 0; sp < p.splitk; ++sp) {
    f32x4 tl[NT];
#pragma unroll
    for (int a = 0; a < NT; ++a) tl[a] = splitk_load(r, sp * SPLIT_BYTES + a * 1024 + lane * 16);
#pragma unroll
    for (int a = 0; a < NT; ++a) sum[a] += tl[a];
  }
#pragma unroll
  for (int a = 0; a < NT; ++a) v[a] = sum[a];
  if (lane == 0) __hip_atomic_store(&p.counters[t], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// The epilogue value of one accumulator element.
template <int EPI>
__device__ __forceinline__ float epi_value(const PackedParams& p, int n, float g, float u) {
  if constexpr (EPI == EPI_SWIGLU) {
    return g * sigmoidf_(g) * u;
  } else if constexpr (EPI == EPI_ACT) {
    const float b = (p.bias && n < p.N) ? bf2f(p.bias[n]) : 0.0f;
    return act_fwd(p.act, g + b);
  } else {
    return g;
  }
}

// Stores one 16x16 output tile (rows 16i.., columns 16gs..) of this wave:
// lane l holds rows 4(l/16) + j, column l%16 (j = 0..3) in v[j].
template <int EPI, typename OutT>
__device__ __forceinline__ void store_tile(const PackedParams& p, int i, int gs, int lane, char* patch,
                                           const float (&v)[4]) {
  const int col = lane & 15;
  const int r0 = 4 * (lane >> 4);
  const int n0 = gs * 16;
  if constexpr (std::is_same<OutT, float>::value) {
    // fp32 rows: patch [16][16] floats (64-byte rows + 16 of padding), then
    // lane l stores row l/4, columns 4(l%4) .. +3
    constexpr int PITCH = 80;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<float*>(patch + (r0 + j) * PITCH + col * 4) = v[j];
    const int row = lane >> 2, c4 = (lane & 3) * 4;
    const f32x4 t = *reinterpret_cast<const f32x4*>(patch + row * PITCH + c4 * 4);
    const int m = i * 16 + row, n = n0 + c4;
    if (m < p.M) {
      float* c = reinterpret_cast<float*>(p.C) + (int64_t)m * p.ldc + n;
      if (p.vec_out && n + 4 <= p.N) {
        *reinterpret_cast<f32x4*>(c) = t;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < p.N) c[e] = t[e];
      }
    }
  } else {
    // bf16: patch [16][16] (32-byte rows + 16 of padding); lanes 0..31 each
    // take 8 columns of one row
    constexpr int PITCH = 48;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint16_t*>(patch + (r0 + j) * PITCH + col * 2) = f2bf(v[j]);
    if (lane < 32) {
      const int row = lane & 15, q = lane >> 4;
      const u32x4 t = *reinterpret_cast<const u32x4*>(patch + row * PITCH + q * 16);
      if (p.cpk) {
        // the next GEMM's packed activations: k-block gs/2, tile i, lanes of
        // column half gs%2 (rows past M and columns past N hold zeros here)
        const int64_t chunk = (int64_t)(gs >> 1) * p.cpk_mt + i;
        reinterpret_cast<u32x4*>(p.cpk)[chunk * 64 + row + 16 * (2 * (gs & 1) + q)] = t;
        if ((p.nstrips & 1) && gs == p.nstrips - 1)  // the k-block's other half has no strip: zeros
          reinterpret_cast<u32x4*>(p.cpk)[chunk * 64 + row + 16 * (2 + q)] = u32x4{0u, 0u, 0u, 0u};
      } else {
        const int m = i * 16 + row, n = n0 + q * 8;
        if (m < p.M) {
          uint16_t* c = reinterpret_cast<uint16_t*>(p.C) + (int64_t)m * p.ldc + n;
          if (p.vec_out && n + 8 <= p.N) {
            *reinterpret_cast<u32x4*>(c) = t;
          } else {
            const uint16_t* h = reinterpret_cast<const uint16_t*>(&t);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (n + e < p.N) c[e] = h[e];
          }
        }
      }
    }
  }
}

// XM: where the activation fragments come from: 0 the packed copy (A), 1
// row-major x read straight into the fragments (16 half lines per load), 2
// row-major x in whole lines staged through LDS (bf16 weights, k-pairs).
template <int MT, int NS, bool DUAL, int EPI, typename OutT, bool F8, int XM, int KW>
__global__ __launch_bounds__(KW * 64) void packed_gemm_kernel(const PackedParams params) {
  constexpr bool RM = XM == 1;
  constexpr bool ST = XM == 2;
  static_assert(!(ST && F8), "staged row-major activations serve bf16 weights");
  constexpr int AT = F8 ? 2 * MT : MT;       // activation chunks per ring step (fp8: a k-pair)
  constexpr int NB = DUAL ? 2 : 1;           // weight matrices
  constexpr int WF = NS * NB;                // weight fragments per k-block (all streamed by every wave)
  constexpr int PF = pass_frags<WF>();       // fragments per wave per reduction pass
  constexpr int NPASS = WF / PF;
  static_assert(WF % PF == 0 && PF % NB == 0, "passes hold whole strips");
  constexpr int SLOT = packed_slot_bytes<MT, PF, XM>();
  __shared__ __attribute__((aligned(16))) char smem[packed_lds_bytes<MT, PF, KW, XM>()];
  // Every parameter, requested in one batch at the start and held in SGPRs:
  // a kernel argument first read after the main loop would be a scalar load
  // queued behind the loop's memory traffic, on the launch's critical path.
  PackedParams p = params;
  __asm__ volatile("" ::"s"(p.A), "s"(p.B0), "s"(p.B1), "s"(p.nkb), "s"(p.nstrips), "s"(p.splitk));
  __asm__ volatile("" : "+s"(p.partials), "+s"(p.counters), "+s"(p.C), "+s"(p.ldc), "+s"(p.vec_out), "+s"(p.cpk),
                   "+s"(p.cpk_mt), "+s"(p.M), "+s"(p.N), "+s"(p.bias), "+s"(p.act));
  if constexpr (F8) __asm__ volatile("" : "+s"(p.bscale0), "+s"(p.bscale1));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ngroups = (p.nstrips + NS - 1) / NS;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int split = id / ngroups;
  const int group = id - split * ngroups;

  // this wave's ring steps (k-blocks; fp8: k-pairs): its share of the split's range
  const int nks = F8 || ST ? p.nkb / 2 : p.nkb;
  const int s0 = (int)((int64_t)nks * split / p.splitk);
  const int s1 = (int)((int64_t)nks * (split + 1) / p.splitk);
  const int w0 = s0 + (s1 - s0) * wave / KW;
  const int n = s0 + (s1 - s0) * (wave + 1) / KW - w0;

  const u32x4* bp[WF];
#pragma unroll
  for (int j = 0; j < WF; ++j) {
    const int s = j / NB, m = j % NB;
    const int strip = min(group * NS + s, p.nstrips - 1);  // a missing last strip re-reads a real one
    bp[j] = reinterpret_cast<const u32x4*>(m ? p.B1 : p.B0) + (int64_t)strip * 64 + lane;
  }
  const u32x4* ap = reinterpret_cast<const u32x4*>(p.A) + lane;
  // row-major activations (RM): this lane's row and k offset, and which of its rows exist
  const uint16_t* xl = nullptr;
  int64_t lda16 = 0;
  bool row_ok[MT];
  if constexpr (RM) {
    xl = p.xrm + (int64_t)(lane & 15) * p.xlda + (lane >> 4) * 8;
    lda16 = 16 * p.xlda;
#pragma unroll
    for (int i = 0; i < MT; ++i) row_ok[i] = 16 * i + (lane & 15) < p.M;
  }
  // staged row-major activations (ST): this lane's line piece, which of its
  // lines exist, and the wave's staging area (its own reduction slot)
  const uint16_t* xs = nullptr;
  int64_t lda8 = 0;
  bool line_ok[2 * MT];
  char* stg = smem + wave * SLOT;
  if constexpr (ST) {
    xs = p.xrm + (int64_t)(lane >> 3) * p.xlda + (lane & 7) * 8;
    lda8 = 8 * p.xlda;
#pragma unroll
    for (int c = 0; c < 2 * MT; ++c) line_ok[c] = 8 * c + (lane >> 3) < p.M;
  }

  f32x4 acc[MT][WF];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < WF; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  if (ST && n > 0) {
    // The same ring over k-pairs, DEPTH / 2 of them in flight (DEPTH k-blocks).
    constexpr int DP = DEPTH / 2;
    const int64_t kbs = (int64_t)p.nstrips * 64;
    const int q = (n + DP - 1) / DP * DP;
    auto phys = [&](int it) { return w0 + min(it, n - 1); };
    KStep<2 * MT, 2 * WF> ring[DP];
    static_for<0, DP>([&](auto d) { load_pair_x<MT, WF>(ring[d], bp, xs, lda8, line_ok, phys(d), kbs); });
    for (int it = 0; it < q - DP; it += DP) {
      static_for<0, DP>([&](auto d) {
        mma_pair_staged<MT, WF>(ring[d], stg, lane, acc);
        load_pair_x<MT, WF>(ring[d], bp, xs, lda8, line_ok, phys(it + DP + (int)d), kbs);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    static_for<0, DP>([&](auto d) {
      if (q - DP + (int)d < n) mma_pair_staged<MT, WF>(ring[d], stg, lane, acc);
    });
  } else if (!ST && n > 0) {
    // The ring runs over q = n rounded up to whole rings of DEPTH k-blocks:
    // the main loop always loads DEPTH k-blocks ahead and the last ring only
    // drains, so no load is issued past the end (a step past n loads the
    // last k-block again and is not accumulated; that happens only when
    // DEPTH does not divide n).  Loads still in flight when the loop ends
    // would hold up the reduction that follows.
    const int64_t kbs = (int64_t)p.nstrips * 64;  // u32x4 elements from one k-block to the next
    const int q = (n + DEPTH - 1) / DEPTH * DEPTH;
    auto phys = [&](int it) { return w0 + min(it, n - 1); };
    KStep<AT, WF> ring[DEPTH];
    auto mma = [&](const KStep<AT, WF>& r) __attribute__((always_inline)) {
      if constexpr (F8) mma_step_f8<MT, WF>(r, acc);
      else mma_step<MT, WF>(r, acc);
    };
    static_for<0, DEPTH>([&](auto d) {
      if constexpr (RM) load_step_rm<MT, WF, F8>(ring[d], bp, xl, lda16, row_ok, phys(d), kbs);
      else load_step<AT, WF>(ring[d], bp, ap, phys(d), kbs);
    });
    for (int it = 0; it < q - DEPTH; it += DEPTH) {
      static_for<0, DEPTH>([&](auto d) {
        mma(ring[d]);  // it + d < q - DEPTH <= n - 1
        if constexpr (RM) load_step_rm<MT, WF, F8>(ring[d], bp, xl, lda16, row_ok, phys(it + DEPTH + (int)d), kbs);
        else load_step<AT, WF>(ring[d], bp, ap, phys(it + DEPTH + (int)d), kbs);
        // keep the ring order: without this the scheduler hoists all of an
        // iteration's loads above its MFMAs into fresh registers and then
        // waits for the whole previous ring at the top of the next iteration
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    static_for<0, DEPTH>([&](auto d) {
      if (q - DEPTH + (int)d < n) mma(ring[d]);
    });
  }

  // The waves' accumulators meet in LDS, a pass of PF fragments per wave at a
  // time (red[wave][tile][fragment of the pass][lane][4]); wave w owns the
  // output units (16-row tile i, strip s) u = w, w + KW, ... and sums them over
  // the K ranges in order.
  auto red_at = [&](int w, int i, int j) {
    return reinterpret_cast<float*>(smem + w * SLOT) + ((i * PF + j) * 64 + lane) * 4;
  };
  char* patch = smem + KW * SLOT + wave * PATCH;
  constexpr int SPP = PF / NB;                       // strips reduced per pass
  constexpr int UW = (MT * NS + KW - 1) / KW;        // units per wave
  f32x4 v[UW][NB];
#pragma unroll
  for (int k = 0; k < UW; ++k)
#pragma unroll
    for (int m = 0; m < NB; ++m) v[k][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  static_for<0, NPASS>([&](auto pc) {
    constexpr int pass = decltype(pc)::value;
    if (pass > 0) __syncthreads();  // the previous pass's reads are done
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < PF; ++j) *reinterpret_cast<f32x4*>(red_at(wave, i, j)) = acc[i][pass * PF + j];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < UW; ++k) {
      const int u = wave + k * KW;
      const int i = u / NS, s = u % NS;
      if (u >= MT * NS || s / SPP != pass) continue;
#pragma unroll
      for (int m = 0; m < NB; ++m) {
        for (int r = 0; r < KW; ++r)  // the waves' K ranges in order
          v[k][m] += *reinterpret_cast<const f32x4*>(red_at(r, i, (s - pass * SPP) * NB + m));
      }
    }
  });
  if (wave >= MT * NS) return;
  if (p.splitk > 1) {
    f32x4 (&flat)[UW * NB] = reinterpret_cast<f32x4(&)[UW * NB]>(v);
    if (!packed_exchange<UW * NB>(p, group * KW + wave, split, lane, flat)) return;
  }
#pragma unroll
  for (int k = 0; k < UW; ++k) {
    const int u = wave + k * KW;
    const int i = u / NS, s = u % NS;
    const int gs = group * NS + s;
    if (u >= MT * NS || gs >= p.nstrips) continue;
    const int col = gs * 16 + (lane & 15);
    float sc0 = 1.0f, sc1 = 1.0f;  // fp8 column scales (columns past N are not stored)
    if constexpr (F8) {
      if (col < p.N) {
        sc0 = p.bscale0[col];
        if constexpr (DUAL) sc1 = p.bscale1[col];
      }
    }
    float out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = epi_value<EPI>(p, col, v[k][0][j] * sc0, v[k][NB - 1][j] * sc1);
    store_tile<EPI, OutT>(p, i, gs, lane, patch, out);
  }
}

// Activations (M, K) row-major -> packed (nkb k-blocks of mt 16-row tiles).
__global__ __launch_bounds__(256) void pack_act16_kernel(const uint16_t* __restrict__ x, int64_t lda, int M, int K,
                                                         int nkb, int mt, int vec, u32x4* __restrict__ out) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  if (gid >= nkb * mt * 64) return;
  const int lane = gid & 63;
  const int c = gid >> 6;
  const int b = c / mt, i = c - (c / mt) * mt;
  const int m = i * 16 + (lane & 15);
  const int k = b * 32 + (lane >> 4) * 8;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (m < M) {
    const uint16_t* src = x + (int64_t)m * lda + k;
    if (vec && k + 8 <= K) {
      v = *reinterpret_cast<const u32x4*>(src);
    } else {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k + e < K) w[e >> 1] |= (uint32_t)src[e] << (16 * (e & 1));
      v = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
  out[gid] = v;
}

// fp8 codes (K, N) row-major -> packed k-pair chunks.  A workgroup reads a
// 64 x 64 block (one k-pair of four strips) into LDS with 16-byte row
// pieces, then each lane gathers its 16 codes (8 rows of each k-block of the
// pair, one column); codes outside K x N are zero.
__global__ __launch_bounds__(256) void pack_weight8_kernel(const uint8_t* __restrict__ w, int64_t ldw, int K, int N,
                                                           int nstrips, int vec, u32x4* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[64][64 + 16];
  const int kp = blockIdx.x;       // k-pair
  const int sg = blockIdx.y * 4;   // first strip of the four
  const int t = threadIdx.x;
  {
    const int r = t >> 2, c16 = (t & 3) * 16;  // row r, columns c16 .. c16+15 of the block
    const int k = kp * 64 + r, n = sg * 16 + c16;
    u32x4 q = {0u, 0u, 0u, 0u};
    if (k < K && vec && n + 16 <= N) {
      q = *reinterpret_cast<const u32x4*>(w + (int64_t)k * ldw + n);
    } else {
      uint8_t v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = (k < K && n + e < N) ? w[(int64_t)k * ldw + n + e] : (uint8_t)0;
      __builtin_memcpy(&q, v, 16);
    }
    *reinterpret_cast<u32x4*>(&tile[r][c16]) = q;
  }
  __syncthreads();
  const int s = t >> 6, lane = t & 63;
  if (sg + s >= nstrips) return;
  const int col = 16 * s + (lane & 15), r0 = 8 * (lane >> 4);
  uint8_t o[16];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) o[8 * h + j] = tile[32 * h + r0 + j][col];
  u32x4 v;
  __builtin_memcpy(&v, o, 16);
  out[((int64_t)kp * nstrips + sg + s) * 64 + lane] = v;
}

// Weights (K, N) row-major -> packed chunks.  A workgroup rearranges a 32 x 64
// block (one k-block of four strips) through LDS: coalesced 16-byte reads of
// row pieces in, 16-byte column pieces out (four neighbouring chunks).
__global__ __launch_bounds__(256) void pack_weight16_kernel(const uint16_t* __restrict__ w, int64_t ldw, int K,
                                                            int N, int nkb, int nstrips, int vec,
                                                            u32x4* __restrict__ out) {
  __shared__ uint16_t tile[32][64 + 8];
  const int b = blockIdx.x;        // k-block
  const int sg = blockIdx.y * 4;   // first strip of the four
  const int t = threadIdx.x;
  {
    const int r = t >> 3, c8 = (t & 7) * 8;  // row r, columns c8 .. c8+7 of the block
    const int k = b * 32 + r, n = sg * 16 + c8;
    uint16_t v[8];
    if (k < K && vec && n + 8 <= N) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(w + (int64_t)k * ldw + n);
      __builtin_memcpy(v, &q, 16);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (k < K && n + e < N) ? w[(int64_t)k * ldw + n + e] : (uint16_t)0;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[r][c8 + e] = v[e];
  }
  __syncthreads();
  const int s = t >> 6, lane = t & 63;  // strip sg + s, lane of its chunk
  if (sg + s >= nstrips) return;
  const int col = s * 16 + (lane & 15), r0 = (lane >> 4) * 8;
  uint32_t q[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) q[e] = (uint32_t)tile[r0 + 2 * e][col] | ((uint32_t)tile[r0 + 2 * e + 1][col] << 16);
  out[((int64_t)b * nstrips + sg + s) * 64 + lane] = u32x4{q[0], q[1], q[2], q[3]};
}

template <int MT, int NS, bool DUAL, int EPI, typename OutT, bool F8, int KW>
hipError_t launch_ns(const PackedParams& p, hipStream_t s) {
  const int ngroups = (p.nstrips + NS - 1) / NS;
  if constexpr (!F8) {
    if (p.xrm && p.xstage) {
      hipLaunchKernelGGL((packed_gemm_kernel<MT, NS, DUAL, EPI, OutT, F8, 2, KW>), dim3(ngroups * p.splitk),
                         dim3(KW * 64), 0, s, p);
      return hipGetLastError();
    }
  }
  if (p.xstage) return hipErrorInvalidValue;
  if (p.xrm) {
    hipLaunchKernelGGL((packed_gemm_kernel<MT, NS, DUAL, EPI, OutT, F8, 1, KW>), dim3(ngroups * p.splitk),
                       dim3(KW * 64), 0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((packed_gemm_kernel<MT, NS, DUAL, EPI, OutT, F8, 0, KW>), dim3(ngroups * p.splitk),
                     dim3(KW * 64), 0, s, p);
  return hipGetLastError();
}

template <bool DUAL, int EPI, typename OutT, bool F8, int KW>
hipError_t launch_packed_kw(const PackedParams& p, int ns, hipStream_t s) {
  const int mt = p.mt;
  if (ns == 1) {
    if (mt == 1) return launch_ns<1, 1, DUAL, EPI, OutT, F8, KW>(p, s);
    if (mt == 2) return launch_ns<2, 1, DUAL, EPI, OutT, F8, KW>(p, s);
    if (mt == 4) return launch_ns<4, 1, DUAL, EPI, OutT, F8, KW>(p, s);
  } else if (ns == 2) {
    if (mt == 1) return launch_ns<1, 2, DUAL, EPI, OutT, F8, KW>(p, s);
    if (mt == 2) return launch_ns<2, 2, DUAL, EPI, OutT, F8, KW>(p, s);
    if (mt == 4) return launch_ns<4, 2, DUAL, EPI, OutT, F8, KW>(p, s);
  } else if (ns == 4) {
    if (mt == 1) return launch_ns<1, 4, DUAL, EPI, OutT, F8, KW>(p, s);
    if (mt == 2) return launch_ns<2, 4, DUAL, EPI, OutT, F8, KW>(p, s);
    if (mt == 4) return launch_ns<4, 4, DUAL, EPI, OutT, F8, KW>(p, s);
  }
  return hipErrorInvalidValue;
}

// The plan's waves per workgroup: PACKED_KW_DUAL for the bf16 dual
// (gate/up) launches, PACKED_KW for every other.
template <bool DUAL, int EPI, typename OutT, bool F8>
hipError_t launch_packed(const PackedParams& p, int ns, int kw, hipStream_t s) {
  if constexpr (DUAL && !F8) {
    if (kw == PACKED_KW_DUAL) return launch_packed_kw<DUAL, EPI, OutT, F8, PACKED_KW_DUAL>(p, ns, s);
  }
  if (kw != PACKED_KW) return hipErrorInvalidValue;
  return launch_packed_kw<DUAL, EPI, OutT, F8, PACKED_KW>(p, ns, s);
}

}  // namespace

int packed_mt(int M) { return M <= 16 ? 1 : (M <= 32 ? 2 : 4); }

PackedPlan plan_packed(int M, int N, int K, bool split_ok, bool f8, bool dual, bool staged) {
  PackedPlan pl;
  pl.kw = dual && !f8 ? PACKED_KW_DUAL : PACKED_KW;
  const int nstrips = (N + 15) / 16;
  const int nkb = f8 ? (K + 63) / 64 : (K + 31) / 32;  // ring steps along K
  // two strips per workgroup once there are enough strips for 64 groups
  // (fewer activation bytes per weight byte), then K split across
  // workgroups until the grid fills the CUs.  (Four strips with twice the
  // K splits measured slower for bf16 and for fp8 codes alike: the larger
  // split-K exchange costs more than the activation loads it saves.)
  // (A launch staging row-major x takes two strips from 64 strips on: QKV at
  // T=64, 80 strips, 40 groups x 6 K splits, 14.3 against 15.25 us with one
  // strip per workgroup and its packing launch.)
  pl.ns = nstrips >= 128 || (staged && nstrips >= 64) ? 2 : 1;
  const int ngroups = (nstrips + pl.ns - 1) / pl.ns;
  pl.splitk = 1;
  if (split_ok) {
    // split K while the grid stays within one workgroup per CU and every
    // wave keeps at least two k-blocks
    while (ngroups * (pl.splitk + 1) <= 256 && nkb / (pl.splitk + 1) >= 2 * pl.kw) ++pl.splitk;
  }
  (void)M;
  return pl;
}

size_t packed_act_bytes(int M, int K) { return (size_t)((K + 31) / 32) * packed_mt(M) * 1024; }

// Split-K arrival tickets of a launch: one per workgroup group and wave.
size_t packed_units(int M, int N, const PackedPlan& pl) {
  const int nstrips = (N + 15) / 16;
  const int ngroups = (nstrips + pl.ns - 1) / pl.ns;
  (void)M;
  return (size_t)ngroups * pl.kw;
}

size_t packed_partial_bytes(int M, int N, bool dual, const PackedPlan& pl) {
  if (pl.splitk <= 1) return 0;
  const int uw = (packed_mt(M) * pl.ns + pl.kw - 1) / pl.kw;  // output units per wave
  return packed_units(M, N, pl) * pl.splitk * uw * (dual ? 2 : 1) * 1024;
}

hipError_t pack_weight8(const void* w, int64_t ldw, int K, int N, bool vec, void* out, hipStream_t s) {
  const int nkp = (K + 63) / 64, nstrips = (N + 15) / 16;
  if (nkp == 0 || nstrips == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_weight8_kernel, dim3(nkp, (nstrips + 3) / 4), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(w), ldw, K, N, nstrips, vec ? 1 : 0, reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

hipError_t pack_act16(const void* x, int64_t lda, int M, int K, bool vec, void* out, hipStream_t s, int nkb_out) {
  const int nkb = nkb_out > (K + 31) / 32 ? nkb_out : (K + 31) / 32, mt = packed_mt(M);
  const int n = nkb * mt * 64;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_act16_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(x), lda, M, K, nkb, mt, vec ? 1 : 0,
                     reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

hipError_t pack_weight16(const void* w, int64_t ldw, int K, int N, bool vec, void* out, hipStream_t s) {
  const int nkb = (K + 31) / 32, nstrips = (N + 15) / 16;
  if (nkb == 0 || nstrips == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_weight16_kernel, dim3(nkb, (nstrips + 3) / 4), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t*>(w), ldw, K, N, nkb, nstrips, vec ? 1 : 0,
                     reinterpret_cast<u32x4*>(out));
  return hipGetLastError();
}

template <bool F8>
hipError_t gemm_packed_kind(const PackedParams& p, const PackedPlan& pl, GemmKind kind, bool out_f32, hipStream_t s) {
  switch (kind) {
    case GK_FWD_STORE:
      return out_f32 ? launch_packed<false, EPI_STORE, float, F8>(p, pl.ns, pl.kw, s)
                     : launch_packed<false, EPI_STORE, uint16_t, F8>(p, pl.ns, pl.kw, s);
    case GK_FWD_ACT: return launch_packed<false, EPI_ACT, uint16_t, F8>(p, pl.ns, pl.kw, s);
    case GK_FWD_SWIGLU: return launch_packed<true, EPI_SWIGLU, uint16_t, F8>(p, pl.ns, pl.kw, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_packed(const PackedParams& p, const PackedPlan& pl, GemmKind kind, bool out_f32, hipStream_t s,
                       bool f8) {
  if (f8) {
    if (p.nkb % 2 != 0 || !p.bscale0 || (kind == GK_FWD_SWIGLU && !p.bscale1)) return hipErrorInvalidValue;
    return gemm_packed_kind<true>(p, pl, kind, out_f32, s);
  }
  return gemm_packed_kind<false>(p, pl, kind, out_f32, s);
}

}  // namespace tpk
