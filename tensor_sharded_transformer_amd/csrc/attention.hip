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
// Design (one workgroup = 8 waves = 128 queries of one query head):
//  * Input is the rank's fused projection output, row t = [Q heads | K heads
//    | V heads] (head_dim 128), read in place; the output row t is the
//    heads side by side, the layout o_proj consumes.
//  * Waves 0-3 and 4-7 are two halves that split the workgroup's key tiles
//    between them (each half has its own LDS ring); wave w of a half owns
//    queries 32 (w mod 4) .. + 32.  At the end the second half hands its
//    running max, row sum and unnormalised output to the first through LDS
//    and the first merges them.  Two waves per SIMD let one wave's softmax
//    overlap the other's matrix work.
//  * A wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K is the A
//    operand (keys are rows, head dim is k) and Q^T the B operand, whose
//    fragments stay in registers for the whole key loop.  In the S^T
//    accumulator layout a lane holds 16 scores of ONE query, so the row max
//    and row sum are lane-local plus one exchange with the lane 32 apart.
//  * O^T = V^T P^T: V^T is the A operand read from LDS with
//    ds_read_b64_tr_b16 (V keeps its key-major layout), P^T the B operand
//    built from the exponentiated S^T accumulators (hardware bf16
//    conversion); the two lanes of a query swap one 4-key group so the
//    fragment's k order is the standard one.
//  * Keys advance in tiles of 64 through a two-stage ring per half (K 16 KB
//    + V 16 KB per stage), filled by buffer loads that write LDS directly;
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
constexpr int BQ = 128;                   // queries per workgroup
constexpr int BKEY = 64;                  // keys per tile
constexpr int NT = 512;                   // threads per workgroup (two halves of 4 waves)
constexpr int HT = NT / 2;                // threads per half
constexpr int K_BYTES = BKEY * HD * 2;    // K tile: two [64 keys][64 d] halves
constexpr int STAGE_BYTES = 2 * K_BYTES;  // K then V
constexpr int CHUNKS = BKEY * HD / 8 / HT;  // 16-byte loads per thread per operand tile
constexpr uint32_t OOB = 0x80000000u;     // buffer offset past the record bound: reads as zero

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// The four stages (two per half) are separate LDS objects, so the compiler
// orders a fragment read only after the loads into its own stage.
__shared__ __attribute__((aligned(16))) char st00[STAGE_BYTES];
__shared__ __attribute__((aligned(16))) char st01[STAGE_BYTES];
__shared__ __attribute__((aligned(16))) char st10[STAGE_BYTES];
__shared__ __attribute__((aligned(16))) char st11[STAGE_BYTES];

// K half-tile [64 keys][64 d] (128-byte rows): 16-byte chunk c of key row r
// sits at chunk c ^ kswz(r), conflict-free for ds_read_b128 of 32 rows.
__device__ __forceinline__ int kswz(int r) { return (r ^ (r >> 3)) & 7; }
// V tile [64 keys][128 d] (256-byte rows): chunk c of key row r sits at
// c ^ vswz(r), conflict-free for ds_read_b64_tr_b16 of four key rows.
__device__ __forceinline__ int vswz(int r) { return ((r & 1) * 10) ^ ((r & 2) * 2); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, 0x00020000);
}

// s_waitcnt vmcnt(0) lgkmcnt(0), then s_barrier, as one statement with a
// memory clobber: this wave's LDS-bound loads have landed, then everyone's.
__device__ __forceinline__ void wait_all_barrier() {
  __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool CAUSAL>
__global__ __launch_bounds__(NT) void attn_fwd_kernel(const uint16_t* __restrict__ qkv, int ld, uint16_t* __restrict__ out,
                                                      int ldo, int T, int n_q, int group, int nqb, float c2) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
  const int wave = wv & 3;                  // query group inside the half
  const int half = wv >> 2;                 // which half of the key tiles
  const int htid = tid & (HT - 1);
  const int bid = blockIdx.x;
  const int qb = nqb - 1 - bid / n_q;       // most key tiles first
  const int head = bid % n_q;
  const int kv = head / group;
  const int q0 = qb * BQ;
  const int qw = q0 + wave * 32;            // this wave's first query
  const int myq = qw + (lane & 31);         // the query this lane's columns belong to
  const int qcol = head * HD;
  const int kcol = n_q * HD + kv * HD;
  const int vcol = kcol + (n_q / group) * HD;

  // key tiles of the workgroup, split between the halves
  const int last_key = CAUSAL ? min(q0 + BQ - 1, T - 1) : T - 1;
  const int nkb = last_key / BKEY + 1;
  const int n0 = (nkb + 1) >> 1;
  const int kb_first = half ? n0 : 0;
  const int my_n = half ? nkb - n0 : n0;
  const int iters = n0;                     // >= my_n for both halves

  // Q^T fragments (B operand): query myq, head dims 16 s + 8 h .. + 8
  bf16x8 qf[HD / 16];
#pragma unroll
  for (int s = 0; s < HD / 16; ++s) {
    if (myq < T)
      qf[s] = *reinterpret_cast<const bf16x8*>(qkv + (size_t)myq * ld + qcol + 16 * s + 8 * h);
    else
      qf[s] = bf16x8{};
  }

  // LDS-bound loads: slot c * HT + htid of each operand tile (16 bytes);
  // K slot -> (d half, key row, chunk position), V slot -> (key row, chunk position)
  uint32_t koff_g[CHUNKS], voff_g[CHUNKS];
  int krow_of[CHUNKS];
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const int slot = c * HT + htid;
    const int kh = slot >> 9, kr = (slot >> 3) & 63, kp = slot & 7;
    koff_g[c] = (uint32_t)(kr * ld * 2 + (kh * 64 + ((kp ^ kswz(kr)) << 3)) * 2);
    const int vr = slot >> 4, vp = slot & 15;
    voff_g[c] = (uint32_t)(vr * ld * 2 + ((vp ^ vswz(vr)) << 3) * 2);
    krow_of[c] = kr;
  }
  auto issue = [&](int kb, char* stage) __attribute__((always_inline)) {
    const int row0 = kb * BKEY;
    const __amdgpu_buffer_rsrc_t rk = rsrc_at(qkv + (size_t)row0 * ld + kcol);
    const __amdgpu_buffer_rsrc_t rv = rsrc_at(qkv + (size_t)row0 * ld + vcol);
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      const int slot0 = c * HT + wave * 64;   // this wave's first slot
      const bool krow_ok = row0 + krow_of[c] < T;
      const int vr = (c * HT + htid) >> 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(stage + slot0 * 16), 16, krow_ok ? koff_g[c] : OOB, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(stage + K_BYTES + slot0 * 16), 16,
                                               row0 + vr < T ? voff_g[c] : OOB, 0, 0, 0);
    }
  };

  // lane-constant LDS offsets of the fragments
  int koff[2], ksw[2];  // K (A operand, k-contiguous): key row 32 kt + lane % 32
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    koff[kt] = (32 * kt + (lane & 31)) * 128;
    ksw[kt] = kswz(32 * kt + (lane & 31));
  }
  int voff[HD / 32];  // V^T (A operand, m-contiguous): 32 head-dim columns per tile
  {
    const int g = lane >> 4, i = lane & 15;
    const int krow = (g >> 1) * 8 + (i >> 2);
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) {
      const int col = 32 * dt + (g & 1) * 16 + 4 * (i & 3);
      voff[dt] = krow * 256 + (((col >> 3) ^ vswz(krow)) << 4) + (col & 7) * 2;
    }
  }

  f32x16 oacc[HD / 32];
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  auto tile = [&](const char* kt_lds, int kb) __attribute__((always_inline)) {
    const char* vt_lds = kt_lds + K_BYTES;
    const int key0 = kb * BKEY;
    // S^T = K Q^T for the tile's two 32-key halves
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < HD / 16; ++s) {
      const int dh = s >> 2, ss = s & 3;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt_lds + dh * (K_BYTES / 2) + koff[kt] +
                                                          (((2 * ss + h) ^ ksw[kt]) << 4));
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kt], 0, 0, 0);
      }
    }
    // mask keys past the diagonal or the end of the sequence (raw scores)
    if (__builtin_expect((CAUSAL && key0 + BKEY - 1 > qw) || key0 + BKEY > T, 0)) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= T || (CAUSAL && key > myq)) sacc[kt][r] = -INFINITY;
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[kt][r]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    // running max in base-2 units (c2 = scale * log2 e > 0 keeps the order)
    const float m_new = fmaxf(m_run, mloc * c2);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], c2, -m_use));
        sacc[kt][r] = p;
        lsum += p;
      }
    if (__any(m_new > m_run)) {  // some running max grew: rescale
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt) oacc[dt] *= alpha;
    }
    l_run += lsum;
    m_run = m_new;
    // O^T += V^T P^T over four 16-key substeps
#pragma unroll
    for (int s = 0; s < BKEY / 16; ++s) {
      const int kt = s >> 1, r0 = (s & 1) * 8;
      // this lane: keys 4h..4h+3 (a) and 8+4h..8+4h+3 (b) of the substep
      const u32x2 a = {pack2(sacc[kt][r0 + 0], sacc[kt][r0 + 1]), pack2(sacc[kt][r0 + 2], sacc[kt][r0 + 3])};
      const u32x2 b = {pack2(sacc[kt][r0 + 4], sacc[kt][r0 + 5]), pack2(sacc[kt][r0 + 6], sacc[kt][r0 + 7])};
      const u32x2 send = h ? a : b;
      const u32x2 recv = {(unsigned)__shfl_xor((int)send[0], 32), (unsigned)__shfl_xor((int)send[1], 32)};
      const u32x4 pf = h ? u32x4{recv[0], recv[1], b[0], b[1]} : u32x4{a[0], a[1], recv[0], recv[1]};
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

  char* const s0 = half ? st10 : st00;
  char* const s1 = half ? st11 : st01;
  if (my_n > 0) issue(kb_first, s0);
  wait_all_barrier();
  for (int it = 0; it < iters; it += 2) {
    // stage 0 holds tile it, stage 1 gets tile it + 1
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

  // merge the second half into the first through LDS (the rings are free now)
  static_assert((HD / 32 * 16 + 2) * 64 * 4 <= STAGE_BYTES, "merge area fits one stage");
  float* xo = reinterpret_cast<float*>(wave == 0 ? st00 : wave == 1 ? st01 : wave == 2 ? st10 : st11);
  if (half) {
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(dt * 16 + r) * 64 + lane] = oacc[dt][r];
    xo[(HD / 32 * 16) * 64 + lane] = m_run;
    xo[(HD / 32 * 16 + 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (half || myq >= T) return;
  const float m1 = xo[(HD / 32 * 16) * 64 + lane];
  const float l1 = xo[(HD / 32 * 16 + 1) * 64 + lane];
  const float m = fmaxf(m_run, m1);
  const float mu = m == -INFINITY ? 0.0f : m;
  const float a0 = __builtin_amdgcn_exp2f(m_run - mu), a1 = __builtin_amdgcn_exp2f(m1 - mu);
  const float l_lane = l_run * a0 + l1 * a1;
  const float inv = 1.0f / (l_lane + __shfl_xor(l_lane, 32));
  uint16_t* orow = out + (size_t)myq * ldo + head * HD;
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        o[e] = (oacc[dt][r] * a0 + xo[(dt * 16 + r) * 64 + lane] * a1) * inv;
      }
      const int d = 32 * dt + 8 * g + 4 * h;
      *reinterpret_cast<u32x2*>(orow + d) = u32x2{pack2(o[0], o[1]), pack2(o[2], o[3])};
    }
}

}  // namespace

int attention_head_dim() { return HD; }

hipError_t gqa_attention_fwd(const void* qkv, void* out, int T, int n_q, int n_kv, bool causal, float scale,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int ld = (n_q + 2 * n_kv) * HD;
  const int ldo = n_q * HD;
  const int nqb = (T + BQ - 1) / BQ;
  const float c2 = scale * 1.4426950408889634f;  // scores in base-2 units
  const dim3 grid(nqb * n_q), block(NT);
  const auto* q = reinterpret_cast<const uint16_t*>(qkv);
  auto* o = reinterpret_cast<uint16_t*>(out);
  if (causal)
    hipLaunchKernelGGL(attn_fwd_kernel<true>, grid, block, 0, s, q, ld, o, ldo, T, n_q, n_q / n_kv, nqb, c2);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<false>, grid, block, 0, s, q, ld, o, ldo, T, n_q, n_q / n_kv, nqb, c2);
  return hipGetLastError();
}

}  // namespace tpk
