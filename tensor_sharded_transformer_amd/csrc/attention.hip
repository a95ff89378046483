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
// Design (one workgroup = 4 waves = 128 queries of one query head):
//  * Input is the rank's fused projection output, row t = [Q heads | K heads
//    | V heads] (head_dim 128), read in place; the output row t is the
//    heads side by side, the layout o_proj consumes.
//  * Each wave owns 32 queries and computes S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16: K is the A operand (keys are rows, head dim
//    is k) and Q^T the B operand, whose fragments stay in registers for the
//    whole key loop.  In the S^T accumulator layout a lane holds 16 scores
//    of ONE query, so the row max and row sum are lane-local plus one
//    exchange with the lane 32 apart.
//  * O^T = V^T P^T: V^T is the A operand read from LDS with
//    ds_read_b64_tr_b16 (V keeps its key-major layout), P^T the B operand
//    built from the exponentiated S^T accumulators; the two lanes of a query
//    swap one 4-key group so the fragment's k order is the standard one.
//  * Keys advance in tiles of 64 through a two-stage LDS ring (K 16 KB +
//    V 16 KB per stage); the next tile's global loads are in flight while
//    the current tile feeds the MFMAs.  One barrier per tile.
//  * Online softmax in fp32 with base-2 exponentials (scale * log2 e folded
//    into the scores); the final division by the row sum happens once.
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
constexpr int NT = 256;                   // threads per workgroup
constexpr int K_BYTES = BKEY * HD * 2;    // K tile: two [64 keys][64 d] halves
constexpr int STAGE_BYTES = 2 * K_BYTES;  // K then V
constexpr int LDS_BYTES = 2 * STAGE_BYTES;
constexpr int CHUNKS = BKEY * HD / 8 / NT;  // 16-byte chunks per thread per operand tile

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// K half-tile [64 keys][64 d] (128-byte rows): 16-byte chunk c of key row r
// sits at chunk c ^ kswz(r), conflict-free for ds_read_b128 of 32 rows.
__device__ __forceinline__ int kswz(int r) { return (r ^ (r >> 3)) & 7; }
// V tile [64 keys][128 d] (256-byte rows): chunk c of key row r sits at
// c ^ vswz(r), conflict-free for ds_read_b64_tr_b16 of four key rows.
__device__ __forceinline__ int vswz(int r) { return ((r & 1) * 10) ^ ((r & 2) * 2); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

template <bool CAUSAL>
__global__ __launch_bounds__(NT) void attn_fwd_kernel(const uint16_t* __restrict__ qkv, int ld, uint16_t* __restrict__ out,
                                                      int ldo, int T, int n_q, int group, int nqb, float c2) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, h = lane >> 5;
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

  // key tiles this workgroup visits
  const int last_key = CAUSAL ? min(q0 + BQ - 1, T - 1) : T - 1;
  const int nkb = last_key / BKEY + 1;

  // Q^T fragments (B operand): query myq, head dims 16 s + 8 h .. + 8
  bf16x8 qf[HD / 16];
#pragma unroll
  for (int s = 0; s < HD / 16; ++s) {
    if (myq < T)
      qf[s] = *reinterpret_cast<const bf16x8*>(qkv + (size_t)myq * ld + qcol + 16 * s + 8 * h);
    else
      qf[s] = bf16x8{};
  }

  // tile loads: chunk c = tid + NT * i of each operand is key c / 16, 16-byte column chunk c % 16
  u32x4 pk[CHUNKS], pv[CHUNKS];
  auto load_tile = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + NT * i;
      const int row = kb * BKEY + (c >> 4);
      if (row < T) {
        const uint16_t* src = qkv + (size_t)row * ld + (c & 15) * 8;
        pk[i] = *reinterpret_cast<const u32x4*>(src + kcol);
        pv[i] = *reinterpret_cast<const u32x4*>(src + vcol);
      } else {
        pk[i] = u32x4{0, 0, 0, 0};
        pv[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int stage) __attribute__((always_inline)) {
    char* kt = lds + stage * STAGE_BYTES;
    char* vt = kt + K_BYTES;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = tid + NT * i;
      const int r = c >> 4, cc = c & 15;
      *reinterpret_cast<u32x4*>(kt + (cc >> 3) * (K_BYTES / 2) + r * 128 + (((cc & 7) ^ kswz(r)) << 4)) = pk[i];
      *reinterpret_cast<u32x4*>(vt + r * 256 + ((cc ^ vswz(r)) << 4)) = pv[i];
    }
  };

  // lane-constant LDS offsets of the fragments
  int koff[2];  // K (A operand, k-contiguous): key row 32 kt + lane % 32
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) koff[kt] = (32 * kt + (lane & 31)) * 128;
  int ksw[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) ksw[kt] = kswz(32 * kt + (lane & 31));
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

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const bool more = kb + 1 < nkb;
    if (more) load_tile(kb + 1);
    const char* kt_lds = lds + (kb & 1) * STAGE_BYTES;
    const char* vt_lds = kt_lds + K_BYTES;
    const int key0 = kb * BKEY;
    // wave-uniform: does any of this wave's queries see a key of this tile?
    const bool active = qw < T && (!CAUSAL || key0 <= qw + 31);
    if (active) {
      // S^T = K Q^T for the tile's two 32-key halves
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < HD / 16; ++s) {
        const int half = s >> 2, ss = s & 3;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt_lds + half * (K_BYTES / 2) + koff[kt] +
                                                            (((2 * ss + h) ^ ksw[kt]) << 4));
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kt], 0, 0, 0);
        }
      }
      // scores in base-2 units; mask keys past the diagonal or the sequence
      const bool need_mask = (CAUSAL && key0 + BKEY - 1 > qw) || key0 + BKEY > T;
      float mloc = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = sacc[kt][r] * c2;
          if (need_mask) {
            const int key = key0 + 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key >= T || (CAUSAL && key > myq)) v = -INFINITY;
          }
          sacc[kt][r] = v;
          mloc = fmaxf(mloc, v);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float lsum = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(sacc[kt][r] - m_use);
          sacc[kt][r] = p;
          lsum += p;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < HD / 32; ++dt) oacc[dt] *= alpha;
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
    }
    if (more) store_tile((kb + 1) & 1);
    __syncthreads();
  }

  if (myq >= T) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  uint16_t* orow = out + (size_t)myq * ldo + head * HD;
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = 32 * dt + 8 * g + 4 * h;
      const u32x2 v = {pack2(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv),
                       pack2(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + d) = v;
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
  if (causal) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_fwd_kernel<true>, grid, block, LDS_BYTES, s, q, ld, o, ldo, T, n_q, n_q / n_kv, nqb, c2);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel<false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_fwd_kernel<false>, grid, block, LDS_BYTES, s, q, ld, o, ldo, T, n_q, n_q / n_kv, nqb, c2);
  }
  return hipGetLastError();
}

}  // namespace tpk
