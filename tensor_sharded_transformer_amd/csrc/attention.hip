// Local grouped-query attention over one tensor-parallel rank's heads, for
// gfx950 (CDNA4): the step between the fused QKV projection and o_proj.
//
// What is computed ("Tensor Parallelism" notes, second paragraph: each rank
// owns whole query and KV heads and runs attention locally over them; "How
// does tensor parallelism split a transformer feed-forward block's two
// matmuls across devices?", attention paragraph: heads are independent, so
// no communication is needed):
//   for query head j, served by KV head g = j / (n_q / n_kv),
//     S = scale * Q_j K_g^T   (entries with key > query dropped when causal)
//     O_j = softmax_rows(S) V_g
// The same notes' FlashAttention paragraph gives the method: tile Q K^T,
// softmax and V so the T x T scores never reach HBM.
//
// Design (one workgroup = 8 waves on NQG x 32 queries of one query head):
//  * Input is the rank's fused projection output, row t = [Q heads | K heads
//    | V heads] (head_dim 128), read in place; the output row t is the
//    heads side by side, the layout o_proj consumes.
//  * The 8 waves form NSPLIT groups of NQG waves; the groups split the
//    workgroup's key tiles into contiguous ranges (each group has its own
//    LDS ring) and wave w of a group owns queries 32 w .. + 32.  At the end
//    groups 1.. hand their running max, row sum and unnormalised output to
//    group 0 through LDS, which merges them in group order.  Two waves per
//    SIMD let one wave's softmax overlap the other's matrix work.  Causal
//    attention uses 64 queries x 4 key ranges of 32-key tiles, so the long
//    rows near the end of the sequence are cut into short pieces and the
//    workgroups, dispatched longest first, finish together; non-causal
//    attention uses 128 queries x 2 ranges of 64-key tiles.
//  * A wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K is the A
//    operand (keys are rows, head dim is k) and Q^T the B operand, whose
//    fragments stay in registers for the whole key loop.  In the S^T
//    accumulator layout a lane holds 16 scores of ONE query, so the row max
//    and row sum are lane-local plus one exchange with the lane 32 apart.
//  * O^T = V^T P^T: V^T is the A operand read from LDS with
//    ds_read_b64_tr_b16 (V keeps its key-major layout), P^T the B operand
//    built from the exponentiated S^T accumulators (hardware bf16
//    conversion); the two lanes of a query swap one 4-key group with
//    v_permlane32_swap (no LDS traffic) so the fragment's k order is the
//    standard one.  The row max and the final row sum combine the two lanes
//    the same way.
//  * Keys advance in tiles of BKEY through a two-stage ring per group (K and
//    V, 256 bytes per key each), filled by buffer loads that write LDS directly;
//    the next tile's loads are in flight while the current tile feeds the
//    MFMAs.  One barrier per tile.
//  * Online softmax in fp32 with base-2 exponentials (scale * log2 e folded
//    into the scores); the output is rescaled only when some query's running
//    max grew, and divided by the row sum once at the end.
//  * Causal: the workgroup stops at its last visible key tile, a wave skips
//    the tiles that lie entirely above its diagonal, and only tiles that
//    cross it (or the ragged end of the sequence) are masked.  Workgroups
//    with the most key tiles are dispatched first.
#include "tp_kernels.h"
#include "tp_device.h"

namespace tpk {
namespace {

constexpr int HD = 128;                   // head dim
constexpr int NT = 512;                   // threads per workgroup (8 waves)
constexpr uint32_t OOB = 0x80000000u;     // buffer offset past the record bound: reads as zero
constexpr int MERGE_FLOATS = (HD / 32 * 16 + 2) * 64;  // one wave's O, m, l in the merge area

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// K half-tile [BKEY keys][64 d] (128-byte rows): 16-byte chunk c of key row
// r sits at chunk c ^ kswz(r), conflict-free for ds_read_b128 of 32 rows.
__device__ __forceinline__ int kswz(int r) { return (r ^ (r >> 3)) & 7; }
// V tile [BKEY keys][128 d] (256-byte rows): chunk c of key row r sits at
// c ^ vswz(r), conflict-free for ds_read_b64_tr_b16 of four key rows.
__device__ __forceinline__ int vswz(int r) { return ((r & 1) * 10) ^ ((r & 2) * 2); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// The two lanes of a query (l and l + 32) exchange halves with
// v_permlane32_swap (VALU, no LDS traffic): it returns {x with the upper
// half replaced by y's lower half, y with the lower half replaced by x's
// upper half}.  half_max / half_sum combine a value over the lane pair
// (both lanes get the same result, low lane's value first).
__device__ __forceinline__ float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// s_waitcnt vmcnt(0) lgkmcnt(0), then s_barrier, as one statement with a
// memory clobber: this wave's LDS-bound loads have landed, then everyone's.
__device__ __forceinline__ void wait_all_barrier() {
  __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Stage 0 and stage 1 of every group's ring are two separate LDS objects,
// so the compiler orders a fragment read only after the loads into its stage.
constexpr int RING_BYTES = 64 * 1024;
__shared__ __attribute__((aligned(16))) char ring0[RING_BYTES];
__shared__ __attribute__((aligned(16))) char ring1[RING_BYTES];

template <int NQG, int NSPLIT, int BKEY>
struct AttnCfg {
  static_assert(NQG * NSPLIT * 64 == NT, "8 waves");
  static_assert(BKEY == 32 || BKEY == 64, "key tile");
  static constexpr int BQ = 32 * NQG;                      // queries per workgroup
  static constexpr int GT = 64 * NQG;                      // threads per group
  static constexpr int K_BYTES = BKEY * HD * 2;            // K tile: two [BKEY][64 d] halves
  static constexpr int STAGE = 2 * K_BYTES;                // K then V
  static constexpr int CHUNKS = BKEY * HD / 8 / GT;        // 16-byte loads per thread per operand tile
  static constexpr int NKT = BKEY / 32;                    // 32-key MFMA tiles per key tile
  static constexpr int AREAS_R0 = RING_BYTES / (MERGE_FLOATS * 4);     // merge areas per ring
  static_assert(CHUNKS * GT * 8 == BKEY * HD, "whole chunks");
  static_assert(2 * AREAS_R0 >= (NSPLIT - 1) * NQG, "merge areas fit the rings");
  static_assert(NSPLIT * STAGE <= RING_BYTES, "each ring holds one stage of every group");
};

template <bool CAUSAL, int NQG, int NSPLIT, int BKEY>
__global__ __launch_bounds__(NT) void attn_fwd_kernel(const uint16_t* __restrict__ qkv, int ld, uint16_t* __restrict__ out,
                                                      int ldo, int T, int n_q, int group, int nqb, float c2) {
  using C = AttnCfg<NQG, NSPLIT, BKEY>;

  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
  const int wave = wv % NQG;                // query group inside the split group
  const int split = wv / NQG;               // which key range
  const int gtid = tid % C::GT;
  const int bid = blockIdx.x;
  const int qb = nqb - 1 - bid / n_q;       // most key tiles first
  const int head = bid % n_q;
  const int kv = head / group;
  const int q0 = qb * C::BQ;
  const int qw = q0 + wave * 32;            // this wave's first query
  const int myq = qw + (lane & 31);         // the query this lane's columns belong to
  const int qcol = head * HD;
  const int kcol = n_q * HD + kv * HD;
  const int vcol = kcol + (n_q / group) * HD;

  // key tiles of the workgroup, cut into NSPLIT contiguous ranges
  const int last_key = CAUSAL ? min(q0 + C::BQ - 1, T - 1) : T - 1;
  const int nkb = last_key / BKEY + 1;
  const int base = nkb / NSPLIT, rem = nkb % NSPLIT;
  const int kb_first = split * base + min(split, rem);
  const int my_n = base + (split < rem ? 1 : 0);
  const int iters = base + (rem > 0 ? 1 : 0);

  // Q^T fragments (B operand): query myq, head dims 16 s + 8 h .. + 8
  bf16x8 qf[HD / 16];
#pragma unroll
  for (int s = 0; s < HD / 16; ++s) {
    if (myq < T)
      qf[s] = *reinterpret_cast<const bf16x8*>(qkv + (size_t)myq * ld + qcol + 16 * s + 8 * h);
    else
      qf[s] = bf16x8{};
  }

  // LDS-bound loads: slot c * GT + gtid of each operand tile (16 bytes);
  // K slot -> (d half, key row, chunk position), V slot -> (key row, chunk position)
  // (arrays the lambdas capture have sizes that do not depend on the
  // template arguments: the host pass drops the kernel otherwise)
  static_assert(C::CHUNKS == 4 && C::NKT <= 2, "fixed array sizes below");
  uint32_t koff_g[4], voff_g[4];
  int krow[4], vrow[4];
#pragma unroll
  for (int c = 0; c < C::CHUNKS; ++c) {
    const int slot = c * C::GT + gtid;
    const int kh = slot / (BKEY * 8), kr = (slot >> 3) % BKEY, kp = slot & 7;
    koff_g[c] = (uint32_t)(kr * ld * 2 + (kh * 64 + ((kp ^ kswz(kr)) << 3)) * 2);
    krow[c] = kr;
    const int vr = slot >> 4, vp = slot & 15;
    voff_g[c] = (uint32_t)(vr * ld * 2 + ((vp ^ vswz(vr)) << 3) * 2);
    vrow[c] = vr;
  }
  auto issue = [&](int kb, char* stage) __attribute__((always_inline)) {
    const int row0 = kb * BKEY;
    const __amdgpu_buffer_rsrc_t rk = rsrc_at(qkv + (size_t)row0 * ld + kcol);
    const __amdgpu_buffer_rsrc_t rv = rsrc_at(qkv + (size_t)row0 * ld + vcol);
#pragma unroll
    for (int c = 0; c < C::CHUNKS; ++c) {
      const int slot0 = c * C::GT + wave * 64;   // this wave's first slot
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(stage + slot0 * 16), 16,
                                               row0 + krow[c] < T ? koff_g[c] : OOB, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(stage + C::K_BYTES + slot0 * 16), 16,
                                               row0 + vrow[c] < T ? voff_g[c] : OOB, 0, 0, 0);
    }
  };

  // lane-constant LDS offsets of the fragments
  int koff[2], ksw[2];  // K (A operand, k-contiguous): key row 32 kt + lane % 32
#pragma unroll
  for (int kt = 0; kt < C::NKT; ++kt) {
    koff[kt] = (32 * kt + (lane & 31)) * 128;
    ksw[kt] = kswz(32 * kt + (lane & 31));
  }
  int voff[HD / 32];  // V^T (A operand, m-contiguous): 32 head-dim columns per tile
  {
    const int g = lane >> 4, i = lane & 15;
    const int kr = (g >> 1) * 8 + (i >> 2);
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) {
      const int col = 32 * dt + (g & 1) * 16 + 4 * (i & 3);
      voff[dt] = kr * 256 + (((col >> 3) ^ vswz(kr)) << 4) + (col & 7) * 2;
    }
  }

  f32x16 oacc[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  auto tile = [&](const char* kt_lds, int kb) __attribute__((always_inline)) {
    const char* vt_lds = kt_lds + C::K_BYTES;
    const int key0 = kb * BKEY;
    // S^T = K Q^T for the tile's 32-key pieces; with a single piece the two
    // head-dim halves accumulate in separate chains (two MFMAs in flight)
    constexpr int NCH = C::NKT == 1 ? 2 : 1;
    f32x16 sacc[C::NKT * NCH];
#pragma unroll
    for (int kt = 0; kt < C::NKT * NCH; ++kt) sacc[kt] = f32x16{};
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) {
      const int dh = s >> 2, ss = s & 3;
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt_lds + dh * (C::K_BYTES / 2) + koff[kt] +
                                                          (((2 * ss + h) ^ ksw[kt]) << 4));
        const int a = NCH == 2 ? dh : kt;
        sacc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[a], 0, 0, 0);
      }
    }
    if constexpr (NCH == 2) sacc[0] += sacc[1];
    // mask keys past the diagonal or the end of the sequence (raw scores)
    if (__builtin_expect((CAUSAL && key0 + BKEY - 1 > qw) || key0 + BKEY > T, 0)) {
#pragma unroll
      for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= T || (CAUSAL && key > myq)) sacc[kt][r] = -INFINITY;
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[kt][r]);
    mloc = half_max(mloc);
    // running max in base-2 units (c2 = scale * log2 e > 0 keeps the order)
    const float m_new = fmaxf(m_run, mloc * c2);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // four short add chains instead of one long one
#pragma unroll
    for (int kt = 0; kt < C::NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], c2, -m_use));
        sacc[kt][r] = p;
        ls[r & 3] += p;
      }
    const float lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    if (__any(m_new > m_run)) {  // some running max grew: rescale
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt) oacc[dt] *= alpha;
    }
    l_run += lsum;
    m_run = m_new;
    // O^T += V^T P^T over the tile's 16-key substeps
#pragma unroll
    for (int s = 0; s < BKEY / 16; ++s) {
      const int kt = s >> 1, r0 = (s & 1) * 8;
      // this lane: keys 4h..4h+3 (a) and 8+4h..8+4h+3 (b) of the substep
      const u32x2 a = {pack2(sacc[kt][r0 + 0], sacc[kt][r0 + 1]), pack2(sacc[kt][r0 + 2], sacc[kt][r0 + 3])};
      const u32x2 b = {pack2(sacc[kt][r0 + 4], sacc[kt][r0 + 5]), pack2(sacc[kt][r0 + 6], sacc[kt][r0 + 7])};
      // low lane: {a, partner's a} = keys 0..7; high lane: {partner's b, b} = keys 8..15
      const auto s0 = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
      const auto s1 = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
      const u32x4 pf = {s0[0], s1[0], s0[1], s1[1]};
      const bf16x8 pfrag = __builtin_bit_cast(bf16x8, pf);
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt) {
        const char* p = vt_lds + voff[dt] + s * 16 * 256;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * 256));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfrag, oacc[dt], 0, 0, 0);
      }
    }
  };

  char* const s0 = ring0 + split * C::STAGE;
  char* const s1 = ring1 + split * C::STAGE;
  if (my_n > 0) issue(kb_first, s0);
  wait_all_barrier();
  for (int it = 0; it < iters; it += 2) {
    // stage 0 holds tile it of this group's range, stage 1 gets tile it + 1
    if (it + 1 < my_n) issue(kb_first + it + 1, s1);
    if (it < my_n) {
      const int kb = kb_first + it;
      if (qw < T && (!CAUSAL || kb * BKEY <= qw + 31)) tile(s0, kb);
    }
    wait_all_barrier();
    if (it + 1 >= iters) break;
    if (it + 2 < my_n) issue(kb_first + it + 2, s0);
    if (it + 1 < my_n) {
      const int kb = kb_first + it + 1;
      if (qw < T && (!CAUSAL || kb * BKEY <= qw + 31)) tile(s1, kb);
    }
    wait_all_barrier();
  }

  // groups 1.. hand their state to group 0 through LDS (the rings are free now)
  auto area = [&](int i) __attribute__((always_inline)) {
    return i < C::AREAS_R0 ? reinterpret_cast<float*>(ring0) + i * MERGE_FLOATS
                           : reinterpret_cast<float*>(ring1) + (i - C::AREAS_R0) * MERGE_FLOATS;
  };
  if (split > 0) {
    float* xo = area((split - 1) * NQG + wave);
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(dt * 16 + r) * 64 + lane] = oacc[dt][r];
    xo[(HD / 32 * 16) * 64 + lane] = m_run;
    xo[(HD / 32 * 16 + 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (split > 0 || myq >= T) return;
  float m = m_run;
#pragma unroll
  for (int g = 1; g < NSPLIT; ++g) m = fmaxf(m, area((g - 1) * NQG + wave)[(HD / 32 * 16) * 64 + lane]);
  const float mu = m == -INFINITY ? 0.0f : m;
  const float a0 = __builtin_amdgcn_exp2f(m_run - mu);
  float l_lane = l_run * a0;
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) oacc[dt] *= a0;
#pragma unroll
  for (int g = 1; g < NSPLIT; ++g) {
    const float* xo = area((g - 1) * NQG + wave);
    const float ag = __builtin_amdgcn_exp2f(xo[(HD / 32 * 16) * 64 + lane] - mu);
    l_lane += xo[(HD / 32 * 16 + 1) * 64 + lane] * ag;
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] += xo[(dt * 16 + r) * 64 + lane] * ag;
  }
  const float inv = 1.0f / half_sum(l_lane);
  uint16_t* orow = out + (size_t)myq * ldo + head * HD;
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * h;
      *reinterpret_cast<u32x2*>(orow + d) =
          u32x2{pack2(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv),
                pack2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv)};
    }
}

using AttnKernel = void (*)(const uint16_t*, int, uint16_t*, int, int, int, int, int, float);

hipError_t launch_attn(AttnKernel k, int bq, const uint16_t* q, uint16_t* o, int T, int n_q, int n_kv, float c2,
                       hipStream_t s) {
  const int ld = (n_q + 2 * n_kv) * HD;
  const int ldo = n_q * HD;
  const int nqb = (T + bq - 1) / bq;
  hipLaunchKernelGGL(k, dim3(nqb * n_q), dim3(NT), 0, s, q, ld, o, ldo, T, n_q, n_q / n_kv, nqb, c2);
  return hipGetLastError();
}

}  // namespace

int attention_head_dim() { return HD; }

hipError_t gqa_attention_fwd(const void* qkv, void* out, int T, int n_q, int n_kv, bool causal, float scale,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  const float c2 = scale * 1.4426950408889634f;  // scores in base-2 units
  const auto* q = reinterpret_cast<const uint16_t*>(qkv);
  auto* o = reinterpret_cast<uint16_t*>(out);
  if (causal) return launch_attn(attn_fwd_kernel<true, 2, 4, 32>, AttnCfg<2, 4, 32>::BQ, q, o, T, n_q, n_kv, c2, s);
  return launch_attn(attn_fwd_kernel<false, 4, 2, 64>, AttnCfg<4, 2, 64>::BQ, q, o, T, n_q, n_kv, c2, s);
}

}  // namespace tpk
