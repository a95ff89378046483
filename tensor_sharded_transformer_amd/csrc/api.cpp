// C ABI of the tpshard library: argument checks on the host, workspace
// layout, and dispatch to the HIP kernels.  Every check happens before the
// first launch, so a rejected call has no side effect.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/tpshard.h"
#include "tp_kernels.h"

using tpk::GemmKind;
using tpk::GemmParams;
using tpk::GemmPlan;

namespace {

thread_local std::string g_last_error;

tp_status fail(tp_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tp_status fail(tp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

tp_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return TP_OK;
  return fail(TP_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kMaxDim = 0x7fffffff;  // kernels index rows/cols with int

bool dim_ok(int64_t v) { return v >= 0 && v <= kMaxDim; }

bool valid_dtype(int d) { return d == TP_BF16 || d == TP_F32; }
bool valid_act(int a) { return a >= TP_ACT_NONE && a <= TP_ACT_SWIGLU; }
size_t esize(int d) { return d == TP_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// product of element counts must stay addressable
bool prod_ok(int64_t a, int64_t b) { return a == 0 || b <= INT64_MAX / 8 / a; }

GemmParams base_params() {
  GemmParams p;
  std::memset(&p, 0, sizeof p);
  p.splitk = 1;
  return p;
}

// Workspace layout shared by the entry points:
//   [ split-K counters (zero between calls) ][ buffers ... ][ split-K partials ]
//   [ packed activations of the decode kernel ]
// The counter region always starts at offset 0 and spans at least
// CNT_RESERVE bytes, and no entry point writes anything else there, so one
// workspace can serve any sequence of calls (of any entry point and shape)
// as long as no call needs more than CNT_RESERVE / 4 arrival counters.
constexpr size_t CNT_RESERVE = 64 * 1024;
struct SplitNeeds {
  size_t part_bytes = 0;
  size_t n_tiles = 0;
  size_t pack_bytes = 0;
  void add(const GemmPlan& plan, int M, int N, int K, bool dual) {
    size_t pb, nt, pk;
    tpk::gemm_split_sizes(plan, M, N, K, dual, &pb, &nt, &pk);
    if (pb > part_bytes) part_bytes = pb;
    if (nt > n_tiles) n_tiles = nt;
    if (pk > pack_bytes) pack_bytes = pk;
  }
  size_t counter_bytes() const {
    const size_t b = tpk::align_up(n_tiles * sizeof(int), 256);
    return b > CNT_RESERVE ? b : CNT_RESERVE;
  }
  size_t partial_bytes() const { return tpk::align_up(part_bytes, 256); }
  size_t packed_bytes() const { return tpk::align_up(pack_bytes, 256); }
};

// Does this plan use workspace (split-K scratch or packed activations)?
bool needs_ws(const GemmPlan& plan) { return plan.splitk > 1 || plan.kernel == tpk::KERNEL_DECODE; }

void attach_split(GemmParams& p, const GemmPlan& plan, char* counters, char* partials, char* pack) {
  p.splitk = plan.splitk;
  p.counters = plan.splitk > 1 ? reinterpret_cast<int*>(counters) : nullptr;
  p.partials = plan.splitk > 1 ? reinterpret_cast<float*>(partials) : nullptr;
  p.apk = plan.kernel == tpk::KERNEL_DECODE ? pack : nullptr;
}

GemmPlan plan_for(int dtype, int M, int N, int K, bool dual, bool allow_split, bool fwd_layout, bool vec_ok) {
  return tpk::plan_gemm(M, N, K, dual, fwd_layout, vec_ok, allow_split && dtype == TP_BF16);
}

hipError_t run_gemm(int dtype, const GemmParams& p, const GemmPlan& plan, GemmKind kind, bool out_f32,
                    hipStream_t s) {
  if (dtype == TP_F32) return tpk::gemm_f32(p, kind, s);
  return tpk::gemm_bf16(p, plan, kind, out_f32, s);
}

// ---- forward shard layout ----------------------------------------------------
struct FwdLayout {
  GemmPlan p1, p2;
  size_t h_bytes = 0, h_off = 0, cnt_off = 0, part_off = 0, pack_off = 0, pack2_off = 0, total = 0;
  bool fuse_pack = false;  // the column GEMM writes h straight into the row GEMM's packed A
};

// vec: every operand allows 16-byte vector loads (aligned, rows multiple of 8).
FwdLayout fwd_layout(int64_t T, int64_t d, int64_t ff_i, int dtype, int act, bool vec) {
  FwdLayout L;
  const bool dual = act == TP_ACT_SWIGLU;
  L.p1 = plan_for(dtype, (int)T, (int)ff_i, (int)d, dual, true, true, vec);
  L.p2 = plan_for(dtype, (int)T, (int)d, (int)ff_i, false, true, true, vec);
  SplitNeeds s1, s2, sn;
  s1.add(L.p1, (int)T, (int)ff_i, (int)d, dual);
  s2.add(L.p2, (int)T, (int)d, (int)ff_i, false);
  sn.add(L.p1, (int)T, (int)ff_i, (int)d, dual);
  sn.add(L.p2, (int)T, (int)d, (int)ff_i, false);
  L.h_bytes = tpk::align_up((size_t)T * ff_i * esize(dtype), 256);
  L.cnt_off = 0;
  L.h_off = sn.counter_bytes();
  L.part_off = L.h_off + L.h_bytes;
  L.pack_off = L.part_off + sn.partial_bytes();
  L.pack2_off = L.pack_off + s1.packed_bytes();
  L.total = L.pack2_off + s2.packed_bytes();
  // h goes straight into the packed A of the row GEMM when both GEMMs use
  // the decode kernel and h has no partial 16-wide k step (whose pad must be 0).
  L.fuse_pack = L.p1.kernel == tpk::KERNEL_DECODE && L.p2.kernel == tpk::KERNEL_DECODE && ff_i % 16 == 0;
  return L;
}

struct BwdLayout {
  GemmPlan pa, pb, pc, pd;
  size_t dgu_bytes = 0, dgu_off = 0, h_off = 0, cnt_off = 0, part_off = 0, pack_off = 0, total = 0;
};

BwdLayout bwd_layout(int64_t T, int64_t d, int64_t ff_i, int dtype, int act) {
  BwdLayout L;
  const bool sw = act == TP_ACT_SWIGLU;
  L.pa = plan_for(dtype, (int)T, (int)ff_i, (int)d, false, true, false, false);   // dh
  L.pb = plan_for(dtype, (int)ff_i, (int)d, (int)T, false, true, false, false);   // dW2
  L.pc = plan_for(dtype, (int)d, (int)ff_i, (int)T, sw, true, false, false);      // dW1 (+dWup)
  L.pd = plan_for(dtype, (int)T, (int)d, (int)((sw ? 2 : 1) * ff_i), false, true, false, false);  // dx
  SplitNeeds sn;
  sn.add(L.pa, (int)T, (int)ff_i, (int)d, false);
  sn.add(L.pb, (int)ff_i, (int)d, (int)T, false);
  sn.add(L.pc, (int)d, (int)ff_i, (int)T, sw);
  sn.add(L.pd, (int)T, (int)d, (int)((sw ? 2 : 1) * ff_i), false);
  L.dgu_bytes = tpk::align_up((size_t)T * ff_i * (sw ? 2 : 1) * esize(dtype), 256);
  L.cnt_off = 0;
  L.dgu_off = sn.counter_bytes();
  L.h_off = L.dgu_off + L.dgu_bytes;
  L.part_off = L.h_off + tpk::align_up((size_t)T * ff_i * esize(dtype), 256);
  L.pack_off = L.part_off + sn.partial_bytes();
  L.total = L.pack_off + sn.packed_bytes();
  return L;
}

// ---- backward of one linear shard ---------------------------------------------
struct LinBwdLayout {
  GemmPlan pw, px;
  size_t cnt_off = 0, part_off = 0, pack_off = 0, total = 0;
};

LinBwdLayout lin_bwd_layout(int64_t T, int64_t K, int64_t N, int dtype) {
  LinBwdLayout L;
  L.pw = plan_for(dtype, (int)K, (int)N, (int)T, false, true, false, false);  // dW = x^T dy
  L.px = plan_for(dtype, (int)T, (int)K, (int)N, false, true, false, false);  // dx = dy W^T
  SplitNeeds sn;
  sn.add(L.pw, (int)K, (int)N, (int)T, false);
  sn.add(L.px, (int)T, (int)K, (int)N, false);
  if (!needs_ws(L.pw) && !needs_ws(L.px)) return L;
  L.cnt_off = 0;
  L.part_off = sn.counter_bytes();
  L.pack_off = L.part_off + sn.partial_bytes();
  L.total = L.pack_off + sn.packed_bytes();
  return L;
}

// Optional workspace of a single GEMM entry point: [counters][partials][packed A].
struct SingleWs {
  GemmPlan plan;
  bool dual = false;
  size_t cnt_bytes = 0, part_bytes = 0, total = 0;
  // With no workspace the call runs unsplit without packed activations
  // (re-planned for that); a too-small workspace is an error.
  tp_status bind(GemmParams& p, void* ws, size_t ws_bytes, const char* who) {
    if (!ws || !needs_ws(plan)) {
      if (needs_ws(plan)) plan = tpk::plan_gemm(p.M, p.N, p.K0, dual, true, p.vecA && p.vecB, false);
      attach_split(p, plan, nullptr, nullptr, nullptr);
      return TP_OK;
    }
    if (ws_bytes < total) return fail(TP_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu needed", who, ws_bytes, total);
    char* base = reinterpret_cast<char*>(ws);
    attach_split(p, plan, base, base + cnt_bytes, base + cnt_bytes + part_bytes);
    return TP_OK;
  }
};

SingleWs single_ws(int dtype, int M, int N, int K, bool dual, bool vec) {
  SingleWs W;
  W.dual = dual;
  W.plan = plan_for(dtype, M, N, K, dual, true, true, vec);
  SplitNeeds sn;
  sn.add(W.plan, M, N, K, dual);
  if (needs_ws(W.plan)) {
    W.cnt_bytes = sn.counter_bytes();
    W.part_bytes = sn.partial_bytes();
    W.total = W.cnt_bytes + W.part_bytes + sn.packed_bytes();
  }
  return W;
}

tp_status check_common(int dtype, int act) {
  if (!valid_dtype(dtype)) return fail(TP_ERR_DTYPE, "unknown dtype %d", dtype);
  if (!valid_act(act)) return fail(TP_ERR_ACT, "unknown act %d", act);
  return TP_OK;
}

// Shared checks and launch of the fp8-weight decode GEMM.
tp_status linear_fp8(const char* who, const void* x, const void* wq, const float* scale, const void* wq_up,
                     const float* scale_up, const void* bias, void* y, void* ws, size_t ws_bytes, int64_t T, int64_t K,
                     int64_t N, int act, bool out_f32, GemmKind kind, hipStream_t s) {
  if (!dim_ok(T) || !dim_ok(K) || !dim_ok(N) || !prod_ok(K, N))
    return fail(TP_ERR_SHAPE, "%s: sizes out of range", who);
  if (T > tpk::STREAM_MAX_M)
    return fail(TP_ERR_UNSUPPORTED, "%s: T=%lld (fp8 weights are built for decode sizes, T <= %d)", who,
                (long long)T, tpk::STREAM_MAX_M);
  if (T == 0 || N == 0) return TP_OK;
  if ((!x && K > 0) || (!wq && K > 0) || !scale || !y ||
      (kind == tpk::GK_FWD_SWIGLU && ((!wq_up && K > 0) || !scale_up)))
    return fail(TP_ERR_NULL, "%s: null input or output pointer", who);
  if (N % 64 || K % 8 || !aligned16(x) || !aligned16(wq) || (wq_up && !aligned16(wq_up)))
    return fail(TP_ERR_UNSUPPORTED, "%s: needs N %% 64 == 0, K %% 8 == 0 and 16-byte aligned x and weights", who);
  GemmParams p = base_params();
  p.A0 = x;
  p.lda = K;
  p.B0 = wq;
  p.B1 = kind == tpk::GK_FWD_SWIGLU ? wq_up : nullptr;
  p.ldb = N;
  p.K0 = (int)K;
  p.M = (int)T;
  p.N = (int)N;
  p.C = y;
  p.ldc = N;
  p.bias = bias;
  p.act = act;
  p.vecA = p.vecB = 1;
  p.b_fp8 = 1;
  p.bscale0 = scale;
  p.bscale1 = kind == tpk::GK_FWD_SWIGLU ? scale_up : nullptr;
  SingleWs W = single_ws(TP_BF16, (int)T, (int)N, (int)K, kind == tpk::GK_FWD_SWIGLU, true);
  if (W.plan.kernel != tpk::KERNEL_DECODE) return fail(TP_ERR_UNSUPPORTED, "%s: no fp8 kernel for this shape", who);
  if (!ws) return fail(TP_ERR_WORKSPACE, "%s: workspace required (%zu bytes)", who, W.total);
  tp_status ws_st = W.bind(p, ws, ws_bytes, who);
  if (ws_st != TP_OK) return ws_st;
  return hip_status(tpk::gemm_bf16(p, W.plan, kind, out_f32, s), who);
}

struct MoeLayout {
  int64_t rows = 0, n_tiles = 0;
  bool gather = false;  // x too large for the GEMM's 32-bit row offsets: copy the routed rows first
  size_t offsets = 0, cursors = 0, tiles = 0, src = 0, dst = 0, pos = 0, xs = 0, hs = 0, zs = 0, total = 0;
};
MoeLayout moe_layout(int64_t T, int64_t d, int64_t ff_i, int E, int k) {
  MoeLayout L;
  const int64_t tile = tpk::MOE_TILE;
  L.rows = ((T * k + tile - 1) / tile + E) * tile;  // every expert's group padded to whole tiles
  L.n_tiles = L.rows / tile;
  size_t o = CNT_RESERVE;                           // (the shared counter region stays untouched)
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += tpk::align_up(bytes, 256);
    return at;
  };
  L.offsets = take((size_t)(E + 1) * 4);
  L.cursors = take((size_t)E * 4);
  L.tiles = take((size_t)L.n_tiles * 4);
  L.src = take((size_t)L.rows * 4);
  L.dst = take((size_t)L.rows * 4);
  L.pos = take((size_t)T * k * 4);
  L.gather = T * d * 2 > INT32_MAX - 64;
  L.xs = take(L.gather ? (size_t)L.rows * d * 2 : 0);
  L.hs = take((size_t)L.rows * ff_i * 2);
  L.zs = take((size_t)T * k * d * 4);  // down-projection rows in (token, slot) order (fp32 or bf16)
  L.total = o;
  return L;
}

}  // namespace

extern "C" {

const char* tp_status_string(tp_status s) {
  switch (s) {
    case TP_OK: return "ok";
    case TP_ERR_NULL: return "null pointer";
    case TP_ERR_SHAPE: return "invalid shape";
    case TP_ERR_DTYPE: return "invalid dtype";
    case TP_ERR_ACT: return "invalid activation arguments";
    case TP_ERR_WORKSPACE: return "workspace too small";
    case TP_ERR_UNSUPPORTED: return "unsupported";
    case TP_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* tp_last_error(void) { return g_last_error.c_str(); }

int tp_abi_version(void) { return TPSHARD_ABI_VERSION; }

tp_status tp_shard_range(int64_t n_total, int p, int i, int64_t* begin, int64_t* len) {
  if (!begin || !len) return fail(TP_ERR_NULL, "tp_shard_range: null output pointer");
  if (p <= 0 || i < 0 || i >= p || n_total < 0)
    return fail(TP_ERR_SHAPE, "tp_shard_range: need p > 0, 0 <= i < p, n_total >= 0 (got n=%lld p=%d i=%d)",
                (long long)n_total, p, i);
  if (n_total % p != 0)
    return fail(TP_ERR_SHAPE, "tp_shard_range: %lld is not divisible into %d equal shards", (long long)n_total, p);
  *len = n_total / p;
  *begin = (int64_t)i * (*len);
  return TP_OK;
}

tp_status tp_gqa_shard(int n_q_heads, int n_kv_heads, int head_dim, int p, int i, int64_t* q_begin, int64_t* q_len,
                       int64_t* kv_begin, int64_t* kv_len) {
  if (!q_begin || !q_len || !kv_begin || !kv_len) return fail(TP_ERR_NULL, "tp_gqa_shard: null output pointer");
  if (n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 || p <= 0 || i < 0 || i >= p)
    return fail(TP_ERR_SHAPE, "tp_gqa_shard: sizes must be positive and 0 <= i < p");
  if (n_q_heads % n_kv_heads != 0)
    return fail(TP_ERR_SHAPE, "tp_gqa_shard: %d query heads do not group evenly over %d KV heads", n_q_heads,
                n_kv_heads);
  if (n_q_heads % p != 0 || n_kv_heads % p != 0)
    return fail(TP_ERR_SHAPE, "tp_gqa_shard: head counts (%d Q, %d KV) must divide by p=%d (a head is never split)",
                n_q_heads, n_kv_heads, p);
  const int64_t qh = n_q_heads / p, kh = n_kv_heads / p;
  *q_begin = (int64_t)i * qh * head_dim;
  *q_len = qh * head_dim;
  *kv_begin = (int64_t)i * kh * head_dim;
  *kv_len = kh * head_dim;
  return TP_OK;
}

tp_status tp_workspace_init(void* ws, size_t bytes, tp_stream stream) {
  if (bytes == 0) return TP_OK;
  if (!ws) return fail(TP_ERR_NULL, "tp_workspace_init: null workspace");
  return hip_status(tpk::zero_fill(ws, bytes, reinterpret_cast<hipStream_t>(stream)), "tp_workspace_init");
}

// ---- column-parallel linear ---------------------------------------------------
size_t tp_col_linear_workspace(int64_t T, int64_t K, int64_t N_i, tp_dtype dtype, tp_act act) {
  if (!valid_dtype(dtype) || !valid_act(act) || !dim_ok(T) || !dim_ok(K) || !dim_ok(N_i) || T == 0) return 0;
  // the kernel choice depends on operand alignment: report the larger need
  const bool sw = act == TP_ACT_SWIGLU;
  const size_t a = single_ws(dtype, (int)T, (int)N_i, (int)K, sw, true).total;
  const size_t b = single_ws(dtype, (int)T, (int)N_i, (int)K, sw, false).total;
  return a > b ? a : b;
}

tp_status tp_col_linear(const void* x, const void* w, const void* w_up, const void* bias, void* y, void* ws,
                        size_t ws_bytes, int64_t T, int64_t K, int64_t N_i, tp_dtype dtype, tp_act act,
                        tp_stream stream) {
  tp_status st = check_common(dtype, act);
  if (st != TP_OK) return st;
  if (!dim_ok(T) || !dim_ok(K) || !dim_ok(N_i) || !prod_ok(T, K) || !prod_ok(K, N_i) || !prod_ok(T, N_i))
    return fail(TP_ERR_SHAPE, "tp_col_linear: sizes out of range (T=%lld K=%lld N_i=%lld)", (long long)T,
                (long long)K, (long long)N_i);
  const bool sw = act == TP_ACT_SWIGLU;
  if (sw && !w_up) return fail(TP_ERR_ACT, "tp_col_linear: SWIGLU needs w_up");
  if (!sw && w_up) return fail(TP_ERR_ACT, "tp_col_linear: w_up is only used by SWIGLU");
  if (sw && bias) return fail(TP_ERR_ACT, "tp_col_linear: a bias is not defined for SWIGLU");
  if (T == 0 || N_i == 0) return TP_OK;
  // (an empty x or w, K == 0, may be NULL: the output is then act(bias))
  if ((!x && K > 0) || (!w && K > 0) || !y)
    return fail(TP_ERR_NULL, "tp_col_linear: null x, w or y");
  GemmParams p = base_params();
  p.A0 = x;
  p.lda = K;
  p.B0 = w;
  p.B1 = sw ? w_up : nullptr;
  p.ldb = N_i;
  p.K0 = (int)K;
  p.M = (int)T;
  p.N = (int)N_i;
  p.C = y;
  p.ldc = N_i;
  p.bias = bias;
  p.act = act;
  p.vecA = aligned16(x) && K % 8 == 0;
  p.vecB = aligned16(w) && (!sw || aligned16(w_up)) && N_i % 8 == 0;
  SingleWs W = single_ws(dtype, (int)T, (int)N_i, (int)K, sw, p.vecA && p.vecB);
  tp_status ws_st = W.bind(p, ws, ws_bytes, "tp_col_linear");
  if (ws_st != TP_OK) return ws_st;
  return hip_status(run_gemm(dtype, p, W.plan, sw ? tpk::GK_FWD_SWIGLU : tpk::GK_FWD_ACT, false,
                             reinterpret_cast<hipStream_t>(stream)),
                    "tp_col_linear");
}

tp_status tp_act_inplace(void* h, const void* up, int64_t T, int64_t N_i, tp_dtype dtype, tp_act act,
                         tp_stream stream) {
  tp_status st = check_common(dtype, act);
  if (st != TP_OK) return st;
  if (!dim_ok(T) || !dim_ok(N_i) || !prod_ok(T, N_i))
    return fail(TP_ERR_SHAPE, "tp_act_inplace: sizes out of range");
  const bool sw = act == TP_ACT_SWIGLU;
  if (sw && !up) return fail(TP_ERR_ACT, "tp_act_inplace: SWIGLU needs up");
  if (!sw && up) return fail(TP_ERR_ACT, "tp_act_inplace: up is only used by SWIGLU");
  if (T == 0 || N_i == 0 || act == TP_ACT_NONE) return TP_OK;
  if (!h) return fail(TP_ERR_NULL, "tp_act_inplace: null h");
  return hip_status(tpk::act_inplace(h, up, T * N_i, dtype == TP_BF16, act, reinterpret_cast<hipStream_t>(stream)),
                    "tp_act_inplace");
}

// ---- row-parallel partial ------------------------------------------------------
size_t tp_row_linear_partial_workspace(int64_t T, int64_t K_i, int64_t N, tp_dtype in_dtype) {
  if (!valid_dtype(in_dtype) || !dim_ok(T) || !dim_ok(K_i) || !dim_ok(N) || T == 0) return 0;
  const size_t a = single_ws(in_dtype, (int)T, (int)N, (int)K_i, false, true).total;
  const size_t b = single_ws(in_dtype, (int)T, (int)N, (int)K_i, false, false).total;
  return a > b ? a : b;
}

tp_status tp_row_linear_partial(const void* x_i, const void* w_i, void* z_i, void* ws, size_t ws_bytes, int64_t T,
                                int64_t K_i, int64_t N, tp_dtype in_dtype, tp_dtype out_dtype, tp_stream stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(TP_ERR_DTYPE, "tp_row_linear_partial: unknown dtype");
  if (in_dtype == TP_F32 && out_dtype != TP_F32)
    return fail(TP_ERR_DTYPE, "tp_row_linear_partial: f32 inputs need an f32 output");
  if (!dim_ok(T) || !dim_ok(K_i) || !dim_ok(N) || !prod_ok(T, K_i) || !prod_ok(K_i, N) || !prod_ok(T, N))
    return fail(TP_ERR_SHAPE, "tp_row_linear_partial: sizes out of range");
  if (T == 0 || N == 0) return TP_OK;
  if ((!x_i && K_i > 0) || (!w_i && K_i > 0) || !z_i)
    return fail(TP_ERR_NULL, "tp_row_linear_partial: null x_i, w_i or z_i");
  GemmParams p = base_params();
  p.A0 = x_i;
  p.lda = K_i;
  p.B0 = w_i;
  p.ldb = N;
  p.K0 = (int)K_i;
  p.M = (int)T;
  p.N = (int)N;
  p.C = z_i;
  p.ldc = N;
  p.vecA = aligned16(x_i) && K_i % 8 == 0;
  p.vecB = aligned16(w_i) && N % 8 == 0;
  SingleWs W = single_ws(in_dtype, (int)T, (int)N, (int)K_i, false, p.vecA && p.vecB);
  tp_status ws_st = W.bind(p, ws, ws_bytes, "tp_row_linear_partial");
  if (ws_st != TP_OK) return ws_st;
  return hip_status(run_gemm(in_dtype, p, W.plan, tpk::GK_FWD_STORE, out_dtype == TP_F32,
                             reinterpret_cast<hipStream_t>(stream)),
                    "tp_row_linear_partial");
}

// ---- fp8-weight linears (decode sizes) --------------------------------------------
size_t tp_linear_fp8_workspace(int64_t T, int64_t K, int64_t N, tp_act act) {
  if (!valid_act(act) || T < 1 || T > tpk::STREAM_MAX_M || !dim_ok(K) || !dim_ok(N)) return 0;
  return single_ws(TP_BF16, (int)T, (int)N, (int)K, act == TP_ACT_SWIGLU, true).total;
}


tp_status tp_col_linear_fp8(const void* x, const void* wq, const float* scale, const void* wq_up,
                            const float* scale_up, const void* bias, void* y, void* ws, size_t ws_bytes, int64_t T,
                            int64_t K, int64_t N_i, tp_act act, tp_stream stream) {
  if (!valid_act(act)) return fail(TP_ERR_ACT, "tp_col_linear_fp8: unknown act %d", act);
  const bool sw = act == TP_ACT_SWIGLU;
  if (sw != (wq_up != nullptr) || sw != (scale_up != nullptr))
    return fail(TP_ERR_ACT, "tp_col_linear_fp8: wq_up and scale_up must be given iff SWIGLU");
  if (sw && bias) return fail(TP_ERR_ACT, "tp_col_linear_fp8: a bias is not defined for SWIGLU");
  return linear_fp8("tp_col_linear_fp8", x, wq, scale, wq_up, scale_up, bias, y, ws, ws_bytes, T, K, N_i, act, false,
                    sw ? tpk::GK_FWD_SWIGLU : tpk::GK_FWD_ACT, reinterpret_cast<hipStream_t>(stream));
}

tp_status tp_row_linear_partial_fp8(const void* x_i, const void* wq_i, const float* scale_i, void* z_i, void* ws,
                                    size_t ws_bytes, int64_t T, int64_t K_i, int64_t N, tp_dtype out_dtype,
                                    tp_stream stream) {
  if (!valid_dtype(out_dtype)) return fail(TP_ERR_DTYPE, "tp_row_linear_partial_fp8: unknown dtype");
  return linear_fp8("tp_row_linear_partial_fp8", x_i, wq_i, scale_i, nullptr, nullptr, nullptr, z_i, ws, ws_bytes, T,
                    K_i, N, TP_ACT_NONE, out_dtype == TP_F32, tpk::GK_FWD_STORE, reinterpret_cast<hipStream_t>(stream));
}

size_t tp_mlp_shard_fwd_fp8_workspace(int64_t T, int64_t d, int64_t ff_i, tp_act act) {
  if (!valid_act(act) || T < 1 || T > tpk::STREAM_MAX_M || !dim_ok(d) || !dim_ok(ff_i)) return 0;
  return fwd_layout(T, d, ff_i, TP_BF16, act, true).total;
}

tp_status tp_mlp_shard_fwd_fp8(const void* x, const void* wq1_i, const float* s1_i, const void* wq_up_i,
                               const float* s_up_i, const void* wq2_i, const float* s2_i, void* y_i, void* ws,
                               size_t ws_bytes, int64_t T, int64_t d, int64_t ff_i, tp_dtype out_dtype, tp_act act,
                               tp_stream stream) {
  if (!valid_act(act)) return fail(TP_ERR_ACT, "tp_mlp_shard_fwd_fp8: unknown act %d", act);
  if (!valid_dtype(out_dtype)) return fail(TP_ERR_DTYPE, "tp_mlp_shard_fwd_fp8: unknown out_dtype");
  if (!dim_ok(T) || !dim_ok(d) || !dim_ok(ff_i) || !prod_ok(d, ff_i))
    return fail(TP_ERR_SHAPE, "tp_mlp_shard_fwd_fp8: sizes out of range");
  const bool sw = act == TP_ACT_SWIGLU;
  if (sw != (wq_up_i != nullptr) || sw != (s_up_i != nullptr))
    return fail(TP_ERR_ACT, "tp_mlp_shard_fwd_fp8: wq_up_i and s_up_i must be given iff SWIGLU");
  if (T > tpk::STREAM_MAX_M)
    return fail(TP_ERR_UNSUPPORTED, "tp_mlp_shard_fwd_fp8: T=%lld (decode sizes, T <= %d)", (long long)T,
                tpk::STREAM_MAX_M);
  if (T == 0 || d == 0) return TP_OK;
  if (ff_i == 0) {  // empty intermediate: the partial is zero
    if (!y_i) return fail(TP_ERR_NULL, "tp_mlp_shard_fwd_fp8: null y_i");
    const size_t yb = (size_t)T * d * (out_dtype == TP_F32 ? 4 : 2);
    return hip_status(tpk::zero_fill(y_i, yb, reinterpret_cast<hipStream_t>(stream)), "tp_mlp_shard_fwd_fp8 (ff_i=0)");
  }
  if (!x || !wq1_i || !s1_i || !wq2_i || !s2_i || !y_i) return fail(TP_ERR_NULL, "tp_mlp_shard_fwd_fp8: null pointer");
  if (d % 64 || ff_i % 64 || !aligned16(x) || !aligned16(wq1_i) || (sw && !aligned16(wq_up_i)) || !aligned16(wq2_i))
    return fail(TP_ERR_UNSUPPORTED, "tp_mlp_shard_fwd_fp8: needs d, ff_i multiples of 64 and 16-byte aligned x, weights");
  const FwdLayout L = fwd_layout(T, d, ff_i, TP_BF16, act, true);
  if (L.p1.kernel != tpk::KERNEL_DECODE || L.p2.kernel != tpk::KERNEL_DECODE)
    return fail(TP_ERR_UNSUPPORTED, "tp_mlp_shard_fwd_fp8: no fp8 kernel for this shape");
  if (!ws) return fail(TP_ERR_WORKSPACE, "tp_mlp_shard_fwd_fp8: workspace required (%zu bytes)", L.total);
  if (ws_bytes < L.total)
    return fail(TP_ERR_WORKSPACE, "tp_mlp_shard_fwd_fp8: workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(ws);

  // column GEMM: h = act(x W1) (or SwiGLU) written straight into the row
  // GEMM's packed activation layout (ff_i is a multiple of 16 here)
  GemmParams p1 = base_params();
  p1.A0 = x;
  p1.lda = d;
  p1.B0 = wq1_i;
  p1.B1 = wq_up_i;
  p1.ldb = ff_i;
  p1.K0 = (int)d;
  p1.M = (int)T;
  p1.N = (int)ff_i;
  p1.C = base + L.h_off;
  p1.ldc = ff_i;
  p1.act = act;
  p1.vecA = p1.vecB = 1;
  p1.b_fp8 = 1;
  p1.bscale0 = s1_i;
  p1.bscale1 = s_up_i;
  attach_split(p1, L.p1, base + L.cnt_off, base + L.part_off, base + L.pack_off);
  p1.cpk = base + L.pack2_off;
  p1.cpk_mt = T <= 32 ? 1 : 2;

  GemmParams p2 = base_params();
  p2.A0 = base + L.h_off;
  p2.lda = ff_i;
  p2.B0 = wq2_i;
  p2.ldb = d;
  p2.K0 = (int)ff_i;
  p2.M = (int)T;
  p2.N = (int)d;
  p2.C = y_i;
  p2.ldc = d;
  p2.vecA = p2.vecB = 1;
  p2.b_fp8 = 1;
  p2.bscale0 = s2_i;
  attach_split(p2, L.p2, base + L.cnt_off, base + L.part_off, base + L.pack2_off);
  p2.apk_ready = 1;

  hipError_t e = tpk::gemm_bf16(p1, L.p1, sw ? tpk::GK_FWD_SWIGLU : tpk::GK_FWD_ACT, false, s);
  if (e != hipSuccess) return hip_status(e, "tp_mlp_shard_fwd_fp8 (column GEMM)");
  e = tpk::gemm_bf16(p2, L.p2, tpk::GK_FWD_STORE, out_dtype == TP_F32, s);
  return hip_status(e, "tp_mlp_shard_fwd_fp8 (row GEMM)");
}

// ---- mixture of experts (experts sharded in place) --------------------------------

tp_status tp_moe_route(const float* logits, int64_t T, int E, int k, int32_t* idx, float* gate, tp_stream stream) {
  if (!dim_ok(T) || E < 1 || E > tpk::MOE_MAX_E || k < 1 || k > tpk::MOE_MAX_K || k > E || !prod_ok(T, E))
    return fail(TP_ERR_SHAPE, "tp_moe_route: need 1 <= k <= min(E, %d), 1 <= E <= %d", tpk::MOE_MAX_K, tpk::MOE_MAX_E);
  if (T == 0) return TP_OK;
  if (!logits || !idx || !gate) return fail(TP_ERR_NULL, "tp_moe_route: null pointer");
  return hip_status(tpk::moe_route(logits, (int)T, E, k, idx, gate, reinterpret_cast<hipStream_t>(stream)),
                    "tp_moe_route");
}

size_t tp_moe_shard_fwd_workspace(int64_t T, int64_t d, int64_t ff_i, int E, int k) {
  if (!dim_ok(T) || !dim_ok(d) || !dim_ok(ff_i) || E < 1 || E > tpk::MOE_MAX_E || k < 1 || k > tpk::MOE_MAX_K ||
      T == 0)
    return 0;
  return moe_layout(T, d, ff_i, E, k).total;
}

tp_status tp_moe_shard_fwd(const void* x, const int32_t* idx, const float* gate, const void* w1, const void* w_up,
                           const void* w2, void* y_i, void* ws, size_t ws_bytes, int64_t T, int64_t d, int64_t ff_i,
                           int E, int k, tp_dtype out_dtype, tp_stream stream) {
  if (!valid_dtype(out_dtype)) return fail(TP_ERR_DTYPE, "tp_moe_shard_fwd: unknown out_dtype");
  if (!dim_ok(T) || !dim_ok(d) || !dim_ok(ff_i) || E < 1 || E > tpk::MOE_MAX_E || k < 1 || k > tpk::MOE_MAX_K ||
      k > E || !prod_ok(T * k, d) || !prod_ok((int64_t)E * d, ff_i))
    return fail(TP_ERR_SHAPE, "tp_moe_shard_fwd: sizes out of range");
  if (T == 0 || d == 0) return TP_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (ff_i == 0)
    return hip_status(tpk::zero_fill(y_i, (size_t)T * d * esize(out_dtype), s), "tp_moe_shard_fwd (ff_i=0)");
  if (!x || !idx || !gate || !w1 || !w_up || !w2 || !y_i) return fail(TP_ERR_NULL, "tp_moe_shard_fwd: null pointer");
  if (d % 8 || ff_i % 8 || !aligned16(x) || !aligned16(w1) || !aligned16(w_up) || !aligned16(w2))
    return fail(TP_ERR_UNSUPPORTED, "tp_moe_shard_fwd: needs d, ff_i multiples of 8 and 16-byte aligned x, weights");
  const MoeLayout L = moe_layout(T, d, ff_i, E, k);
  if (L.rows > kMaxDim / 8) return fail(TP_ERR_SHAPE, "tp_moe_shard_fwd: too many routed rows");
  if (!ws) return fail(TP_ERR_WORKSPACE, "tp_moe_shard_fwd: workspace required (%zu bytes)", L.total);
  if (ws_bytes < L.total)
    return fail(TP_ERR_WORKSPACE, "tp_moe_shard_fwd: workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  char* base = reinterpret_cast<char*>(ws);
  int* tiles = reinterpret_cast<int*>(base + L.tiles);
  int* pos_of = reinterpret_cast<int*>(base + L.pos);
  int* src = reinterpret_cast<int*>(base + L.src);
  int* dst = reinterpret_cast<int*>(base + L.dst);
  hipError_t e = tpk::moe_group(idx, (int)T, E, k, x, (int)d, (int)L.rows, (int)L.n_tiles,
                                reinterpret_cast<int*>(base + L.offsets), reinterpret_cast<int*>(base + L.cursors),
                                tiles, src, dst, pos_of, L.gather ? base + L.xs : nullptr, s);
  if (e != hipSuccess) return hip_status(e, "tp_moe_shard_fwd (grouping)");

  // grouped gate/up GEMM with the SwiGLU epilogue, MOE_TILE-row tiles, one expert
  // each, reading the routed rows of x through the row table
  GemmPlan plan;
  plan.kernel = tpk::KERNEL_TILED;
  plan.tile = tpk::TILE_256x256;  // BM == MOE_TILE
  plan.splitk = 1;
  GemmParams p1 = base_params();
  p1.A0 = L.gather ? base + L.xs : x;
  p1.a_rows = L.gather ? nullptr : src;
  p1.lda = d;
  p1.B0 = w1;
  p1.B1 = w_up;
  p1.ldb = ff_i;
  p1.K0 = (int)d;
  p1.M = (int)L.rows;
  p1.N = (int)ff_i;
  p1.C = base + L.hs;
  p1.ldc = ff_i;
  p1.act = TP_ACT_SWIGLU;
  p1.vecA = p1.vecB = 1;
  p1.tile_expert = tiles;
  p1.b_expert_stride = d * ff_i;
  if (!tpk::gemm_tile_supported(p1, plan, tpk::GK_FWD_SWIGLU))
    return fail(TP_ERR_UNSUPPORTED, "tp_moe_shard_fwd: no grouped kernel for these operands");
  e = tpk::gemm_tile(p1, plan, tpk::GK_FWD_SWIGLU, false, s);
  if (e != hipSuccess) return hip_status(e, "tp_moe_shard_fwd (gate/up GEMM)");
  // grouped down GEMM, each row stored at its (token, slot) row: bf16 rows
  // for a bf16 output (an intermediate, like h), fp32 rows for an fp32 one
  const bool zs_f32 = out_dtype == TP_F32;
  GemmParams p2 = base_params();
  p2.A0 = base + L.hs;
  p2.lda = ff_i;
  p2.B0 = w2;
  p2.ldb = d;
  p2.K0 = (int)ff_i;
  p2.M = (int)L.rows;
  p2.N = (int)d;
  p2.C = base + L.zs;
  p2.ldc = d;
  p2.vecA = p2.vecB = 1;
  p2.tile_expert = tiles;
  p2.b_expert_stride = ff_i * d;
  p2.c_rows = dst;
  if (!tpk::gemm_tile_supported(p2, plan, tpk::GK_FWD_STORE))
    return fail(TP_ERR_UNSUPPORTED, "tp_moe_shard_fwd: no grouped kernel for these operands");
  // a short contraction (ff_i <= 128) with bf16 rows: one workgroup per row
  // tile walks all of d with its rows of h held in LDS
  if (!zs_f32 && tpk::gemm_walk_supported(p2, T * k)) e = tpk::gemm_walk(p2, s);
  else e = tpk::gemm_tile(p2, plan, tpk::GK_FWD_STORE, zs_f32, s);
  if (e != hipSuccess) return hip_status(e, "tp_moe_shard_fwd (down GEMM)");
  return hip_status(tpk::moe_combine(base + L.zs, zs_f32, pos_of, gate, (int)T, k, (int)d, y_i, out_dtype == TP_F32, s),
                    "tp_moe_shard_fwd (combine)");
}

tp_status tp_fp8_pack_strips(const void* src, void* dst, int64_t K, int64_t N, tp_stream stream) {
  if (!dim_ok(K) || !dim_ok(N) || !prod_ok(K, N)) return fail(TP_ERR_SHAPE, "tp_fp8_pack_strips: sizes out of range");
  if (N % 64) return fail(TP_ERR_SHAPE, "tp_fp8_pack_strips: N=%lld is not a multiple of 64", (long long)N);
  if (K == 0 || N == 0) return TP_OK;
  if (!src || !dst) return fail(TP_ERR_NULL, "tp_fp8_pack_strips: null src or dst");
  if (src == dst) return fail(TP_ERR_SHAPE, "tp_fp8_pack_strips: src and dst must not alias");
  if (!aligned16(src) || !aligned16(dst)) return fail(TP_ERR_UNSUPPORTED, "tp_fp8_pack_strips: unaligned pointers");
  return hip_status(tpk::pack_fp8_strips(src, dst, K, N, reinterpret_cast<hipStream_t>(stream)), "tp_fp8_pack_strips");
}

// ---- sum of partials -------------------------------------------------------------
tp_status tp_partial_sum(const void* const* z, int p, const void* bias, void* y, int64_t T, int64_t N,
                         tp_dtype in_dtype, tp_dtype out_dtype, tp_stream stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return fail(TP_ERR_DTYPE, "tp_partial_sum: unknown dtype");
  if (p < 1 || p > 64) return fail(TP_ERR_SHAPE, "tp_partial_sum: need 1 <= p <= 64 (got %d)", p);
  if (!dim_ok(T) || !dim_ok(N) || !prod_ok(T, N)) return fail(TP_ERR_SHAPE, "tp_partial_sum: sizes out of range");
  if (T == 0 || N == 0) return TP_OK;
  if (!z || !y) return fail(TP_ERR_NULL, "tp_partial_sum: null z or y");
  for (int i = 0; i < p; ++i)
    if (!z[i]) return fail(TP_ERR_NULL, "tp_partial_sum: z[%d] is null", i);
  return hip_status(tpk::partial_sum(z, p, bias, y, T, N, in_dtype == TP_BF16, out_dtype == TP_BF16,
                                     reinterpret_cast<hipStream_t>(stream)),
                    "tp_partial_sum");
}

// ---- sequence-parallel boundary ---------------------------------------------------------
tp_status tp_rs_residual_rmsnorm(const void* const* z, int p, int rank, const void* bias, const void* residual_in,
                                 const void* norm_w, float eps, void* residual_out, void* y, int64_t T, int64_t N,
                                 tp_dtype in_dtype, tp_dtype out_dtype, tp_stream stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(TP_ERR_DTYPE, "tp_rs_residual_rmsnorm: unknown dtype");
  if (p < 1 || p > 64) return fail(TP_ERR_SHAPE, "tp_rs_residual_rmsnorm: need 1 <= p <= 64 (got %d)", p);
  if (rank < 0 || rank >= p) return fail(TP_ERR_SHAPE, "tp_rs_residual_rmsnorm: rank %d outside [0, %d)", rank, p);
  if (!dim_ok(T) || !dim_ok(N) || !prod_ok(T, N)) return fail(TP_ERR_SHAPE, "tp_rs_residual_rmsnorm: sizes out of range");
  if (T % p != 0)
    return fail(TP_ERR_SHAPE, "tp_rs_residual_rmsnorm: T=%lld is not divisible into %d equal row shares",
                (long long)T, p);
  if (N > tpk::RS_NORM_MAX_N)
    return fail(TP_ERR_UNSUPPORTED, "tp_rs_residual_rmsnorm: N=%lld > %lld", (long long)N,
                (long long)tpk::RS_NORM_MAX_N);
  if (!(eps >= 0.0f)) return fail(TP_ERR_SHAPE, "tp_rs_residual_rmsnorm: eps must be >= 0");
  if (T == 0 || N == 0) return TP_OK;
  if (!z || !residual_in || !norm_w || !residual_out || !y)
    return fail(TP_ERR_NULL, "tp_rs_residual_rmsnorm: null z, residual_in, norm_w, residual_out or y");
  for (int i = 0; i < p; ++i)
    if (!z[i]) return fail(TP_ERR_NULL, "tp_rs_residual_rmsnorm: z[%d] is null", i);
  return hip_status(tpk::rs_residual_rmsnorm(z, p, rank, bias, residual_in, norm_w, eps, residual_out, y, T, N,
                                             in_dtype == TP_BF16, out_dtype == TP_BF16,
                                             reinterpret_cast<hipStream_t>(stream)),
                    "tp_rs_residual_rmsnorm");
}

// ---- MLP shard forward ------------------------------------------------------------
size_t tp_mlp_shard_fwd_workspace(int64_t T, int64_t d, int64_t ff_i, tp_dtype dtype, tp_act act) {
  if (!valid_dtype(dtype) || !valid_act(act) || !dim_ok(T) || !dim_ok(d) || !dim_ok(ff_i)) return 0;
  if (T == 0) return 0;
  const size_t a = fwd_layout(T, d, ff_i, dtype, act, true).total;
  const size_t b = fwd_layout(T, d, ff_i, dtype, act, false).total;
  return a > b ? a : b;
}

}  // extern "C"

namespace {

// ---- allocation-free scratch ----------------------------------------------------------
// The forward shard's scratch (split-K arrival counters and partials, h and the
// packed activations) for callers that cannot allocate: a static device array
// per GPU.  Host code never uses the array's name as an address (on the host it
// is only a stand-in symbol); the device address is looked up once per device.
constexpr size_t kNoAllocScratch = TP_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[kNoAllocScratch];

std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch: on the first call on a device, its address
// (hipGetSymbolAddress with that device current) and a cleared counter region
// (a fill kernel on `s`, ahead of the call's own launches on the same stream;
// every call leaves the counters zero again).
tp_status noalloc_scratch(const char* who, hipStream_t s, char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, who);
  if (dev < 0 || dev >= kMaxDevices) return fail(TP_ERR_UNSUPPORTED, "%s: device %d out of range", who, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    e = tpk::zero_fill(ptr, CNT_RESERVE, s);
    if (e != hipSuccess) return hip_status(e, who);
    g_scratch_ptr[dev] = reinterpret_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return TP_OK;
}

// The forward shard behind tp_mlp_shard_fwd (caller workspace) and
// tp_mlp_shard_fwd_noalloc (static scratch; ws is ignored).
tp_status mlp_shard_fwd_impl(const char* who, bool noalloc, const void* x, const void* w1_i, const void* w_up_i,
                             const void* w2_i, void* y_i, void* saved, void* ws, size_t ws_bytes, int64_t T,
                             int64_t d, int64_t ff_i, tp_dtype dtype, tp_dtype out_dtype, tp_act act,
                             tp_stream stream) {
  tp_status st = check_common(dtype, act);
  if (st != TP_OK) return st;
  if (!valid_dtype(out_dtype) || (dtype == TP_F32 && out_dtype != TP_F32))
    return fail(TP_ERR_DTYPE, "%s: out_dtype must be f32 for f32 inputs, bf16 or f32 otherwise", who);
  if (!dim_ok(T) || !dim_ok(d) || !dim_ok(ff_i) || !prod_ok(T, d) || !prod_ok(d, ff_i) || !prod_ok(T, 2 * ff_i))
    return fail(TP_ERR_SHAPE, "%s: sizes out of range", who);
  const bool sw = act == TP_ACT_SWIGLU;
  if (sw != (w_up_i != nullptr)) return fail(TP_ERR_ACT, "%s: w_up_i must be given iff SWIGLU", who);
  if (T == 0 || d == 0) return TP_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (ff_i == 0) {  // empty intermediate: the partial is zero (and saved is empty)
    if (!y_i) return fail(TP_ERR_NULL, "%s: null y_i", who);
    const size_t yb = (size_t)T * d * esize(out_dtype);
    return hip_status(tpk::zero_fill(y_i, yb, s), who);
  }
  if (!x || !w1_i || !w2_i || !y_i) return fail(TP_ERR_NULL, "%s: null x, w1_i, w2_i or y_i", who);
  const bool vec = aligned16(x) && aligned16(w1_i) && (!sw || aligned16(w_up_i)) && aligned16(w2_i) &&
                   d % 8 == 0 && ff_i % 8 == 0;
  const FwdLayout L = fwd_layout(T, d, ff_i, dtype, act, vec);
  if (noalloc) {
    if (L.total > kNoAllocScratch)
      return fail(TP_ERR_WORKSPACE, "%s: these sizes need %zu bytes of scratch; the static scratch holds %zu", who,
                  L.total, kNoAllocScratch);
    char* sp = nullptr;
    st = noalloc_scratch(who, s, &sp);
    if (st != TP_OK) return st;
    ws = sp;
    ws_bytes = kNoAllocScratch;
  } else {
    if (!ws) return fail(TP_ERR_WORKSPACE, "%s: workspace required (%zu bytes)", who, L.total);
    if (ws_bytes < L.total)
      return fail(TP_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu needed", who, ws_bytes, L.total);
  }
  char* base = reinterpret_cast<char*>(ws);
  void* h = base + L.h_off;

  GemmParams p1 = base_params();
  p1.A0 = x;
  p1.lda = d;
  p1.B0 = w1_i;
  p1.B1 = w_up_i;
  p1.ldb = ff_i;
  p1.K0 = (int)d;
  p1.M = (int)T;
  p1.N = (int)ff_i;
  p1.C = h;
  p1.ldc = ff_i;
  p1.act = act;
  if (saved) {
    p1.C2 = saved;
    p1.C3 = sw ? reinterpret_cast<char*>(saved) + ff_i * esize(dtype) : nullptr;
    p1.ldc2 = sw ? 2 * ff_i : ff_i;
  }
  p1.vecA = aligned16(x) && d % 8 == 0;
  p1.vecB = aligned16(w1_i) && (!sw || aligned16(w_up_i)) && ff_i % 8 == 0;
  attach_split(p1, L.p1, base + L.cnt_off, base + L.part_off, base + L.pack_off);
  if (L.fuse_pack) {
    p1.cpk = base + L.pack2_off;
    p1.cpk_mt = T <= 32 ? 1 : 2;
  }

  GemmParams p2 = base_params();
  p2.A0 = h;
  p2.lda = ff_i;
  p2.B0 = w2_i;
  p2.ldb = d;
  p2.K0 = (int)ff_i;
  p2.M = (int)T;
  p2.N = (int)d;
  p2.C = y_i;
  p2.ldc = d;
  p2.vecA = ff_i % 8 == 0;
  p2.vecB = aligned16(w2_i) && d % 8 == 0;
  attach_split(p2, L.p2, base + L.cnt_off, base + L.part_off, base + L.pack2_off);
  p2.apk_ready = L.fuse_pack ? 1 : 0;

  hipError_t e = run_gemm(dtype, p1, L.p1, sw ? tpk::GK_FWD_SWIGLU : tpk::GK_FWD_ACT, false, s);
  if (e != hipSuccess) return hip_status(e, who);
  e = run_gemm(dtype, p2, L.p2, tpk::GK_FWD_STORE, out_dtype == TP_F32, s);
  return hip_status(e, who);
}

}  // namespace

extern "C" {

tp_status tp_mlp_shard_fwd(const void* x, const void* w1_i, const void* w_up_i, const void* w2_i, void* y_i,
                           void* saved, void* ws, size_t ws_bytes, int64_t T, int64_t d, int64_t ff_i, tp_dtype dtype,
                           tp_dtype out_dtype, tp_act act, tp_stream stream) {
  return mlp_shard_fwd_impl("tp_mlp_shard_fwd", false, x, w1_i, w_up_i, w2_i, y_i, saved, ws, ws_bytes, T, d, ff_i,
                            dtype, out_dtype, act, stream);
}

tp_status tp_mlp_shard_fwd_noalloc(const void* x, const void* w1_i, const void* w_up_i, const void* w2_i, void* y_i,
                                   void* saved, int64_t T, int64_t d, int64_t ff_i, tp_dtype dtype,
                                   tp_dtype out_dtype, tp_act act, tp_stream stream) {
  return mlp_shard_fwd_impl("tp_mlp_shard_fwd_noalloc", true, x, w1_i, w_up_i, w2_i, y_i, saved, nullptr, 0, T, d,
                            ff_i, dtype, out_dtype, act, stream);
}

// ---- packed weights (decode-sized calls) ---------------------------------------------
}  // extern "C"

namespace {

constexpr int64_t kPackedMaxT = 64;

// Workspace of the packed-weight entry points:
//   [ split-K counters (>= CNT_RESERVE, zero between calls) ][ packed x ][ packed h ][ split-K partials ]
struct PackedLayout {
  tpk::PackedPlan p1, p2;
  tpk::PackedPlan p1s;  // p1 for a call that stages row-major x (regions sized for both)
  size_t x_off = 0, h_off = 0, part_off = 0, total = 0;
};

size_t counter_region(size_t units) {
  const size_t b = tpk::align_up(units * sizeof(int), 256);
  return b > CNT_RESERVE ? b : CNT_RESERVE;
}

// One GEMM (p1 only; h_off == part_off): x (T, K) -> (T, N).
PackedLayout packed_linear_layout(int64_t T, int64_t K, int64_t N, bool dual) {
  PackedLayout L;
  L.p1 = tpk::plan_packed((int)T, (int)N, (int)K, true, false, dual);
  L.p1s = tpk::plan_packed((int)T, (int)N, (int)K, true, false, dual, true);
  const size_t u = std::max(tpk::packed_units((int)T, (int)N, L.p1), tpk::packed_units((int)T, (int)N, L.p1s));
  const size_t q = std::max(tpk::packed_partial_bytes((int)T, (int)N, dual, L.p1),
                            tpk::packed_partial_bytes((int)T, (int)N, dual, L.p1s));
  L.x_off = counter_region(u);
  L.h_off = L.x_off + tpk::align_up(tpk::packed_act_bytes((int)T, (int)K), 256);
  L.part_off = L.h_off;
  L.total = L.part_off + tpk::align_up(q, 256);
  return L;
}

// The feed-forward shard: x (T, d) -> h (T, ff_i), packed -> y (T, d).
PackedLayout packed_fwd_layout(int64_t T, int64_t d, int64_t ff_i, bool dual) {
  PackedLayout L;
  L.p1 = tpk::plan_packed((int)T, (int)ff_i, (int)d, true, false, dual);
  L.p1s = tpk::plan_packed((int)T, (int)ff_i, (int)d, true, false, dual, true);
  L.p2 = tpk::plan_packed((int)T, (int)d, (int)ff_i, true);
  const size_t u1 = std::max(tpk::packed_units((int)T, (int)ff_i, L.p1), tpk::packed_units((int)T, (int)ff_i, L.p1s)),
               u2 = tpk::packed_units((int)T, (int)d, L.p2);
  const size_t q1 = std::max(tpk::packed_partial_bytes((int)T, (int)ff_i, dual, L.p1),
                             tpk::packed_partial_bytes((int)T, (int)ff_i, dual, L.p1s));
  const size_t q2 = tpk::packed_partial_bytes((int)T, (int)d, false, L.p2);
  L.x_off = counter_region(u1 > u2 ? u1 : u2);
  L.h_off = L.x_off + tpk::align_up(tpk::packed_act_bytes((int)T, (int)d), 256);
  L.part_off = L.h_off + tpk::align_up(tpk::packed_act_bytes((int)T, (int)ff_i), 256);
  L.total = L.part_off + tpk::align_up(q1 > q2 ? q1 : q2, 256);
  return L;
}

tpk::PackedParams packed_params(const void* A, const void* B0, const void* B1, int64_t T, int64_t K, int64_t N,
                                const tpk::PackedPlan& pl, char* ws, const PackedLayout& L) {
  tpk::PackedParams p;
  std::memset(&p, 0, sizeof p);
  p.A = A;
  p.B0 = B0;
  p.B1 = B1;
  p.M = (int)T;
  p.N = (int)N;
  p.K = (int)K;
  p.mt = tpk::packed_mt((int)T);
  p.nkb = (int)((K + 31) / 32);
  p.nstrips = (int)((N + 15) / 16);
  p.splitk = pl.splitk;
  p.counters = reinterpret_cast<int*>(ws);
  p.partials = reinterpret_cast<float*>(ws + L.part_off);
  return p;
}

// Launches that read few activation bytes in all take them straight from
// row-major x (bf16 weights): every workgroup reads its K range of x, so a
// launch reads (strip groups) x K x 32 x mt bytes of fragments, and a
// row-major fragment load touches 16 half lines where a packed one touches 8
// full ones.  Measured at T=64 (packing launch -> row-major reads): o_proj
// K=1024 N=8192 11.5 -> 9.3 us (34 MB of fragments), K=2048 N=2048 12.2 ->
// 9.6 us (17 MB), K=4096 N=1280 12.3 -> 11.8 us (42 MB); slower from 67 MB
// on (K=2048 N=8192 14.3 -> 15.6 us, QKV K=8192 N=1280 15.2 -> 18.1 us, the
// decode gate/up), where the packing launch stays.
//
// Larger launches on bf16 weights with K a multiple of 64 load x in whole
// 128-byte lines (8 rows x 64 columns per load, the same lines per byte as
// the packed copy) and turn them into fragments through LDS, with no packing
// launch either: the decode shard step at T=64 49.7 -> 45.6 us.  They run the
// staged plan (L.p1s: two strips per workgroup from 64 strips on, so QKV at
// T=64 runs 40 groups x 6 K splits, 15.25 -> 14.3 us); one weight fragment
// per k-block (fewer than 64 strips, no gate/up pair) keeps the packing
// launch, where the staging costs more than it saves (QKV with one strip per
// workgroup: 15.2 -> 16.2 us).
//
// Returns the plan the launch runs and sets p.xrm (and p.xstage) where x is
// read in place; otherwise the caller packs x first.
const tpk::PackedPlan& x_source(tpk::PackedParams& p, const PackedLayout& L, const void* x, int64_t K,
                                bool f8 = false) {
  if (K % (f8 ? 64 : 32) != 0 || !aligned16(x)) return L.p1;  // fp8: whole k-pairs
  const int64_t groups = (p.nstrips + L.p1.ns - 1) / L.p1.ns;
  if (groups * K * 32 * p.mt > ((int64_t)48 << 20)) {
    if (f8 || K % 64 != 0 || L.p1s.ns * (p.B1 ? 2 : 1) < 2) return L.p1;
    p.xstage = 1;
    p.splitk = L.p1s.splitk;
  }
  p.xrm = reinterpret_cast<const uint16_t*>(x);
  p.xlda = K;
  return p.xstage ? L.p1s : L.p1;
}

tp_status packed_sizes_ok(const char* who, int64_t T, int64_t K, int64_t N) {
  if (!dim_ok(T) || !dim_ok(K) || !dim_ok(N) || !prod_ok(T, K) || !prod_ok(K, N) || !prod_ok(T, N))
    return fail(TP_ERR_SHAPE, "%s: sizes out of range", who);
  if (T > kPackedMaxT) return fail(TP_ERR_SHAPE, "%s: packed weights serve decode sizes, T <= 64 (T=%lld)", who,
                                   (long long)T);
  return TP_OK;
}

tp_status packed_ws_ok(const char* who, const void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return fail(TP_ERR_WORKSPACE, "%s: workspace required (%zu bytes)", who, need);
  if (ws_bytes < need) return fail(TP_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu needed", who, ws_bytes, need);
  if (!aligned16(ws)) return fail(TP_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned", who);
  return TP_OK;
}

bool rows_vec16(const void* c, int64_t ld, size_t es) { return aligned16(c) && (ld * (int64_t)es) % 16 == 0; }

}  // namespace

extern "C" {

size_t tp_packed_weight_bytes(int64_t K, int64_t N) {
  if (!dim_ok(K) || !dim_ok(N)) return 0;
  return tpk::packed_weight_bytes(K, N);
}

tp_status tp_pack_weight(const void* w, void* w_packed, int64_t K, int64_t N, tp_stream stream) {
  if (!dim_ok(K) || !dim_ok(N) || !prod_ok(K, N)) return fail(TP_ERR_SHAPE, "tp_pack_weight: sizes out of range");
  if (K == 0 || N == 0) return TP_OK;
  if (!w || !w_packed) return fail(TP_ERR_NULL, "tp_pack_weight: null w or w_packed");
  if (!aligned16(w_packed)) return fail(TP_ERR_SHAPE, "tp_pack_weight: w_packed must be 16-byte aligned");
  const bool vec = aligned16(w) && N % 8 == 0;
  return hip_status(tpk::pack_weight16(w, N, (int)K, (int)N, vec, w_packed, reinterpret_cast<hipStream_t>(stream)),
                    "tp_pack_weight");
}

size_t tp_linear_packed_workspace(int64_t T, int64_t K, int64_t N, tp_act act) {
  if (!valid_act(act) || !dim_ok(T) || !dim_ok(K) || !dim_ok(N) || T == 0 || T > kPackedMaxT) return 0;
  return packed_linear_layout(T, K, N, act == TP_ACT_SWIGLU).total;
}

tp_status tp_col_linear_packed(const void* x, const void* w_packed, const void* w_up_packed, const void* bias,
                               void* y, void* ws, size_t ws_bytes, int64_t T, int64_t K, int64_t N_i, tp_act act,
                               tp_stream stream) {
  const char* who = "tp_col_linear_packed";
  if (!valid_act(act)) return fail(TP_ERR_ACT, "%s: unknown act %d", who, act);
  tp_status st = packed_sizes_ok(who, T, K, N_i);
  if (st != TP_OK) return st;
  const bool sw = act == TP_ACT_SWIGLU;
  if (sw && !w_up_packed) return fail(TP_ERR_ACT, "%s: SWIGLU needs w_up_packed", who);
  if (!sw && w_up_packed) return fail(TP_ERR_ACT, "%s: w_up_packed is only used by SWIGLU", who);
  if (sw && bias) return fail(TP_ERR_ACT, "%s: a bias is not defined for SWIGLU", who);
  if (T == 0 || N_i == 0) return TP_OK;
  if ((!x && K > 0) || (!w_packed && K > 0) || !y) return fail(TP_ERR_NULL, "%s: null x, w_packed or y", who);
  if (!aligned16(w_packed) || (sw && !aligned16(w_up_packed)))
    return fail(TP_ERR_SHAPE, "%s: packed weights must be 16-byte aligned", who);
  const PackedLayout L = packed_linear_layout(T, K, N_i, sw);
  st = packed_ws_ok(who, ws, ws_bytes, L.total);
  if (st != TP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(ws);
  tpk::PackedParams p = packed_params(base + L.x_off, w_packed, sw ? w_up_packed : nullptr, T, K, N_i, L.p1, base, L);
  const tpk::PackedPlan& pl = x_source(p, L, x, K);
  if (!p.xrm) {
    const hipError_t e = tpk::pack_act16(x, K, (int)T, (int)K, aligned16(x) && K % 8 == 0, base + L.x_off, s);
    if (e != hipSuccess) return hip_status(e, who);
  }
  p.C = y;
  p.ldc = N_i;
  p.vec_out = rows_vec16(y, N_i, 2);
  p.bias = reinterpret_cast<const uint16_t*>(bias);
  p.act = act;
  return hip_status(tpk::gemm_packed(p, pl, sw ? tpk::GK_FWD_SWIGLU : tpk::GK_FWD_ACT, false, s), who);
}

tp_status tp_row_linear_partial_packed(const void* x_i, const void* w_packed, void* z_i, void* ws, size_t ws_bytes,
                                       int64_t T, int64_t K_i, int64_t N, tp_dtype out_dtype, tp_stream stream) {
  const char* who = "tp_row_linear_partial_packed";
  if (!valid_dtype(out_dtype)) return fail(TP_ERR_DTYPE, "%s: unknown out_dtype", who);
  tp_status st = packed_sizes_ok(who, T, K_i, N);
  if (st != TP_OK) return st;
  if (T == 0 || N == 0) return TP_OK;
  if ((!x_i && K_i > 0) || (!w_packed && K_i > 0) || !z_i) return fail(TP_ERR_NULL, "%s: null x_i, w_packed or z_i", who);
  if (!aligned16(w_packed)) return fail(TP_ERR_SHAPE, "%s: packed weights must be 16-byte aligned", who);
  const PackedLayout L = packed_linear_layout(T, K_i, N, false);
  st = packed_ws_ok(who, ws, ws_bytes, L.total);
  if (st != TP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(ws);
  tpk::PackedParams p = packed_params(base + L.x_off, w_packed, nullptr, T, K_i, N, L.p1, base, L);
  const tpk::PackedPlan& pl = x_source(p, L, x_i, K_i);
  if (!p.xrm) {
    const hipError_t e = tpk::pack_act16(x_i, K_i, (int)T, (int)K_i, aligned16(x_i) && K_i % 8 == 0, base + L.x_off, s);
    if (e != hipSuccess) return hip_status(e, who);
  }
  p.C = z_i;
  p.ldc = N;
  p.vec_out = rows_vec16(z_i, N, esize(out_dtype));
  return hip_status(tpk::gemm_packed(p, pl, tpk::GK_FWD_STORE, out_dtype == TP_F32, s), who);
}

size_t tp_packed_act_bytes(int64_t T, int64_t K) {
  if (!dim_ok(T) || !dim_ok(K) || T == 0 || T > kPackedMaxT) return 0;
  return tpk::packed_act_bytes((int)T, (int)K);
}

tp_status tp_pack_act(const void* x, void* x_packed, int64_t T, int64_t K, tp_stream stream) {
  const char* who = "tp_pack_act";
  tp_status st = packed_sizes_ok(who, T, K, 0);
  if (st != TP_OK) return st;
  if (T == 0 || K == 0) return TP_OK;
  if (!x || !x_packed) return fail(TP_ERR_NULL, "%s: null x or x_packed", who);
  if (!aligned16(x_packed)) return fail(TP_ERR_SHAPE, "%s: x_packed must be 16-byte aligned", who);
  return hip_status(tpk::pack_act16(x, K, (int)T, (int)K, aligned16(x) && K % 8 == 0, x_packed,
                                    reinterpret_cast<hipStream_t>(stream)),
                    who);
}

tp_status tp_linear_packed_gemm(const void* x_packed, const void* w_packed, const void* w_up_packed,
                                const void* bias, void* y, void* ws, size_t ws_bytes, int64_t T, int64_t K,
                                int64_t N, tp_act act, tp_dtype out_dtype, tp_stream stream) {
  const char* who = "tp_linear_packed_gemm";
  if (!valid_act(act)) return fail(TP_ERR_ACT, "%s: unknown act %d", who, act);
  if (!valid_dtype(out_dtype)) return fail(TP_ERR_DTYPE, "%s: unknown out_dtype", who);
  if (out_dtype == TP_F32 && act != TP_ACT_NONE)
    return fail(TP_ERR_DTYPE, "%s: an f32 output is only written without an activation", who);
  tp_status st = packed_sizes_ok(who, T, K, N);
  if (st != TP_OK) return st;
  const bool sw = act == TP_ACT_SWIGLU;
  if (sw != (w_up_packed != nullptr)) return fail(TP_ERR_ACT, "%s: w_up_packed must be given iff SWIGLU", who);
  if (sw && bias) return fail(TP_ERR_ACT, "%s: a bias is not defined for SWIGLU", who);
  if (T == 0 || N == 0) return TP_OK;
  if ((!x_packed && K > 0) || (!w_packed && K > 0) || !y)
    return fail(TP_ERR_NULL, "%s: null x_packed, w_packed or y", who);
  if (!aligned16(x_packed) || !aligned16(w_packed) || (sw && !aligned16(w_up_packed)))
    return fail(TP_ERR_SHAPE, "%s: packed operands must be 16-byte aligned", who);
  const PackedLayout L = packed_linear_layout(T, K, N, sw);
  st = packed_ws_ok(who, ws, ws_bytes, L.total);
  if (st != TP_OK) return st;
  char* base = reinterpret_cast<char*>(ws);
  tpk::PackedParams p = packed_params(x_packed, w_packed, sw ? w_up_packed : nullptr, T, K, N, L.p1, base, L);
  p.C = y;
  p.ldc = N;
  p.vec_out = rows_vec16(y, N, esize(out_dtype));
  p.bias = reinterpret_cast<const uint16_t*>(bias);
  p.act = act;
  const tpk::GemmKind kind = sw ? tpk::GK_FWD_SWIGLU : (act == TP_ACT_NONE && !bias ? tpk::GK_FWD_STORE : tpk::GK_FWD_ACT);
  return hip_status(tpk::gemm_packed(p, L.p1, kind, out_dtype == TP_F32, reinterpret_cast<hipStream_t>(stream)), who);
}

size_t tp_mlp_shard_fwd_packed_workspace(int64_t T, int64_t d, int64_t ff_i, tp_act act) {
  if (!valid_act(act) || !dim_ok(T) || !dim_ok(d) || !dim_ok(ff_i) || T == 0 || T > kPackedMaxT) return 0;
  return packed_fwd_layout(T, d, ff_i, act == TP_ACT_SWIGLU).total;
}

tp_status tp_mlp_shard_fwd_packed(const void* x, const void* w1_packed, const void* w_up_packed,
                                  const void* w2_packed, void* y_i, void* ws, size_t ws_bytes, int64_t T, int64_t d,
                                  int64_t ff_i, tp_dtype out_dtype, tp_act act, tp_stream stream) {
  const char* who = "tp_mlp_shard_fwd_packed";
  if (!valid_act(act)) return fail(TP_ERR_ACT, "%s: unknown act %d", who, act);
  if (!valid_dtype(out_dtype)) return fail(TP_ERR_DTYPE, "%s: unknown out_dtype", who);
  tp_status st = packed_sizes_ok(who, T, d, ff_i);
  if (st != TP_OK) return st;
  const bool sw = act == TP_ACT_SWIGLU;
  if (sw != (w_up_packed != nullptr)) return fail(TP_ERR_ACT, "%s: w_up_packed must be given iff SWIGLU", who);
  if (T == 0 || d == 0) return TP_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (ff_i == 0) {  // empty intermediate: the partial is zero
    if (!y_i) return fail(TP_ERR_NULL, "%s: null y_i", who);
    return hip_status(tpk::zero_fill(y_i, (size_t)T * d * esize(out_dtype), s), who);
  }
  if (!x || !w1_packed || !w2_packed || !y_i) return fail(TP_ERR_NULL, "%s: null x, w1_packed, w2_packed or y_i", who);
  if (!aligned16(w1_packed) || !aligned16(w2_packed) || (sw && !aligned16(w_up_packed)))
    return fail(TP_ERR_SHAPE, "%s: packed weights must be 16-byte aligned", who);
  const PackedLayout L = packed_fwd_layout(T, d, ff_i, sw);
  st = packed_ws_ok(who, ws, ws_bytes, L.total);
  if (st != TP_OK) return st;
  char* base = reinterpret_cast<char*>(ws);
  // column GEMM: h = act(x W1_i [, x W_up_i]) straight into the row GEMM's packed activations
  tpk::PackedParams p1 = packed_params(base + L.x_off, w1_packed, sw ? w_up_packed : nullptr, T, d, ff_i, L.p1,
                                       base, L);
  hipError_t e = hipSuccess;
  const tpk::PackedPlan& pl1 = x_source(p1, L, x, d);
  if (!p1.xrm) {
    e = tpk::pack_act16(x, d, (int)T, (int)d, aligned16(x) && d % 8 == 0, base + L.x_off, s);
    if (e != hipSuccess) return hip_status(e, who);
  }
  p1.cpk = base + L.h_off;
  p1.cpk_mt = tpk::packed_mt((int)T);
  p1.act = act;
  e = tpk::gemm_packed(p1, pl1, sw ? tpk::GK_FWD_SWIGLU : tpk::GK_FWD_ACT, false, s);
  if (e != hipSuccess) return hip_status(e, who);
  // row GEMM: the full-shape partial y_i = h W2_i
  tpk::PackedParams p2 = packed_params(base + L.h_off, w2_packed, nullptr, T, ff_i, d, L.p2, base, L);
  p2.C = y_i;
  p2.ldc = d;
  p2.vec_out = rows_vec16(y_i, d, esize(out_dtype));
  return hip_status(tpk::gemm_packed(p2, L.p2, tpk::GK_FWD_STORE, out_dtype == TP_F32, s), who);
}

// ---- packed fp8 weights (decode-sized calls) -----------------------------------------
}  // extern "C"

namespace {

// Workspace of the packed fp8 entry points: the bf16 packed layout, with the
// packed activations padded to whole 64-row k-pairs (zeros past K).
int64_t kpair_pad(int64_t K) { return (K + 63) / 64 * 64; }

PackedLayout packed8_linear_layout(int64_t T, int64_t K, int64_t N, bool dual) {
  PackedLayout L;
  const int64_t Kp = kpair_pad(K);
  L.p1 = tpk::plan_packed((int)T, (int)N, (int)Kp, true, true, dual);
  L.p1s = L.p1;
  L.x_off = counter_region(tpk::packed_units((int)T, (int)N, L.p1));
  L.h_off = L.x_off + tpk::align_up(tpk::packed_act_bytes((int)T, (int)Kp), 256);
  L.part_off = L.h_off;
  L.total = L.part_off + tpk::align_up(tpk::packed_partial_bytes((int)T, (int)N, dual, L.p1), 256);
  return L;
}

// The feed-forward shard (ff_i a multiple of 64, so h fills whole k-pairs).
PackedLayout packed8_fwd_layout(int64_t T, int64_t d, int64_t ff_i, bool dual) {
  PackedLayout L;
  const int64_t dp = kpair_pad(d);
  L.p1 = tpk::plan_packed((int)T, (int)ff_i, (int)dp, true, true, dual);
  L.p1s = L.p1;
  L.p2 = tpk::plan_packed((int)T, (int)d, (int)ff_i, true, true);
  const size_t u1 = tpk::packed_units((int)T, (int)ff_i, L.p1), u2 = tpk::packed_units((int)T, (int)d, L.p2);
  const size_t q1 = tpk::packed_partial_bytes((int)T, (int)ff_i, dual, L.p1);
  const size_t q2 = tpk::packed_partial_bytes((int)T, (int)d, false, L.p2);
  L.x_off = counter_region(u1 > u2 ? u1 : u2);
  L.h_off = L.x_off + tpk::align_up(tpk::packed_act_bytes((int)T, (int)dp), 256);
  L.part_off = L.h_off + tpk::align_up(tpk::packed_act_bytes((int)T, (int)ff_i), 256);
  L.total = L.part_off + tpk::align_up(q1 > q2 ? q1 : q2, 256);
  return L;
}

tpk::PackedParams packed8_params(const void* A, const void* B0, const float* sc0, const void* B1, const float* sc1,
                                 int64_t T, int64_t K, int64_t N, const tpk::PackedPlan& pl, char* ws,
                                 const PackedLayout& L) {
  tpk::PackedParams p = packed_params(A, B0, B1, T, K, N, pl, ws, L);
  p.nkb = (int)(kpair_pad(K) / 32);
  p.bscale0 = sc0;
  p.bscale1 = sc1;
  return p;
}

}  // namespace

extern "C" {

size_t tp_packed_fp8_weight_bytes(int64_t K, int64_t N) {
  if (!dim_ok(K) || !dim_ok(N)) return 0;
  return tpk::packed_fp8_weight_bytes(K, N);
}

tp_status tp_pack_weight_fp8(const void* codes, void* w_packed, int64_t K, int64_t N, tp_stream stream) {
  const char* who = "tp_pack_weight_fp8";
  if (!dim_ok(K) || !dim_ok(N) || !prod_ok(K, N)) return fail(TP_ERR_SHAPE, "%s: sizes out of range", who);
  if (K == 0 || N == 0) return TP_OK;
  if (!codes || !w_packed) return fail(TP_ERR_NULL, "%s: null codes or w_packed", who);
  if (!aligned16(w_packed)) return fail(TP_ERR_SHAPE, "%s: w_packed must be 16-byte aligned", who);
  const bool vec = aligned16(codes) && N % 16 == 0;
  return hip_status(tpk::pack_weight8(codes, N, (int)K, (int)N, vec, w_packed, reinterpret_cast<hipStream_t>(stream)),
                    who);
}

size_t tp_linear_packed_fp8_workspace(int64_t T, int64_t K, int64_t N, tp_act act) {
  if (!valid_act(act) || !dim_ok(T) || !dim_ok(K) || !dim_ok(N) || T == 0 || T > kPackedMaxT) return 0;
  return packed8_linear_layout(T, K, N, act == TP_ACT_SWIGLU).total;
}

tp_status tp_col_linear_packed_fp8(const void* x, const void* wq_packed, const float* scale, const void* wq_up_packed,
                                   const float* scale_up, const void* bias, void* y, void* ws, size_t ws_bytes,
                                   int64_t T, int64_t K, int64_t N_i, tp_act act, tp_stream stream) {
  const char* who = "tp_col_linear_packed_fp8";
  if (!valid_act(act)) return fail(TP_ERR_ACT, "%s: unknown act %d", who, act);
  tp_status st = packed_sizes_ok(who, T, K, N_i);
  if (st != TP_OK) return st;
  const bool sw = act == TP_ACT_SWIGLU;
  if (sw != (wq_up_packed != nullptr) || sw != (scale_up != nullptr))
    return fail(TP_ERR_ACT, "%s: wq_up_packed and scale_up must be given iff SWIGLU", who);
  if (sw && bias) return fail(TP_ERR_ACT, "%s: a bias is not defined for SWIGLU", who);
  if (T == 0 || N_i == 0) return TP_OK;
  if ((!x && K > 0) || (!wq_packed && K > 0) || !scale || !y)
    return fail(TP_ERR_NULL, "%s: null x, wq_packed, scale or y", who);
  if (!aligned16(wq_packed) || (sw && !aligned16(wq_up_packed)))
    return fail(TP_ERR_SHAPE, "%s: packed weights must be 16-byte aligned", who);
  const PackedLayout L = packed8_linear_layout(T, K, N_i, sw);
  st = packed_ws_ok(who, ws, ws_bytes, L.total);
  if (st != TP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(ws);
  const int nkb = (int)(kpair_pad(K) / 32);
  tpk::PackedParams p = packed8_params(base + L.x_off, wq_packed, scale, sw ? wq_up_packed : nullptr,
                                       sw ? scale_up : nullptr, T, K, N_i, L.p1, base, L);
  x_source(p, L, x, K, true);  // fp8 codes: L.p1
  if (!p.xrm) {
    const hipError_t e = tpk::pack_act16(x, K, (int)T, (int)K, aligned16(x) && K % 8 == 0, base + L.x_off, s, nkb);
    if (e != hipSuccess) return hip_status(e, who);
  }
  p.C = y;
  p.ldc = N_i;
  p.vec_out = rows_vec16(y, N_i, 2);
  p.bias = reinterpret_cast<const uint16_t*>(bias);
  p.act = act;
  const tpk::GemmKind kind = sw ? tpk::GK_FWD_SWIGLU : tpk::GK_FWD_ACT;
  return hip_status(tpk::gemm_packed(p, L.p1, kind, false, s, true), who);
}

tp_status tp_row_linear_partial_packed_fp8(const void* x_i, const void* wq_packed, const float* scale_i, void* z_i,
                                           void* ws, size_t ws_bytes, int64_t T, int64_t K_i, int64_t N,
                                           tp_dtype out_dtype, tp_stream stream) {
  const char* who = "tp_row_linear_partial_packed_fp8";
  if (!valid_dtype(out_dtype)) return fail(TP_ERR_DTYPE, "%s: unknown out_dtype", who);
  tp_status st = packed_sizes_ok(who, T, K_i, N);
  if (st != TP_OK) return st;
  if (T == 0 || N == 0) return TP_OK;
  if ((!x_i && K_i > 0) || (!wq_packed && K_i > 0) || !scale_i || !z_i)
    return fail(TP_ERR_NULL, "%s: null x_i, wq_packed, scale_i or z_i", who);
  if (!aligned16(wq_packed)) return fail(TP_ERR_SHAPE, "%s: packed weights must be 16-byte aligned", who);
  const PackedLayout L = packed8_linear_layout(T, K_i, N, false);
  st = packed_ws_ok(who, ws, ws_bytes, L.total);
  if (st != TP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(ws);
  const int nkb = (int)(kpair_pad(K_i) / 32);
  tpk::PackedParams p = packed8_params(base + L.x_off, wq_packed, scale_i, nullptr, nullptr, T, K_i, N, L.p1, base, L);
  x_source(p, L, x_i, K_i, true);  // fp8 codes: L.p1
  if (!p.xrm) {
    const hipError_t e =
        tpk::pack_act16(x_i, K_i, (int)T, (int)K_i, aligned16(x_i) && K_i % 8 == 0, base + L.x_off, s, nkb);
    if (e != hipSuccess) return hip_status(e, who);
  }
  p.C = z_i;
  p.ldc = N;
  p.vec_out = rows_vec16(z_i, N, esize(out_dtype));
  return hip_status(tpk::gemm_packed(p, L.p1, tpk::GK_FWD_STORE, out_dtype == TP_F32, s, true), who);
}

size_t tp_mlp_shard_fwd_packed_fp8_workspace(int64_t T, int64_t d, int64_t ff_i, tp_act act) {
  if (!valid_act(act) || !dim_ok(T) || !dim_ok(d) || !dim_ok(ff_i) || T == 0 || T > kPackedMaxT || ff_i % 64 != 0)
    return 0;
  return packed8_fwd_layout(T, d, ff_i, act == TP_ACT_SWIGLU).total;
}

tp_status tp_mlp_shard_fwd_packed_fp8(const void* x, const void* wq1_packed, const float* s1_i,
                                      const void* wq_up_packed, const float* s_up_i, const void* wq2_packed,
                                      const float* s2_i, void* y_i, void* ws, size_t ws_bytes, int64_t T, int64_t d,
                                      int64_t ff_i, tp_dtype out_dtype, tp_act act, tp_stream stream) {
  const char* who = "tp_mlp_shard_fwd_packed_fp8";
  if (!valid_act(act)) return fail(TP_ERR_ACT, "%s: unknown act %d", who, act);
  if (!valid_dtype(out_dtype)) return fail(TP_ERR_DTYPE, "%s: unknown out_dtype", who);
  tp_status st = packed_sizes_ok(who, T, d, ff_i);
  if (st != TP_OK) return st;
  if (ff_i % 64 != 0) return fail(TP_ERR_UNSUPPORTED, "%s: ff_i must be a multiple of 64 (ff_i=%lld)", who,
                                  (long long)ff_i);
  const bool sw = act == TP_ACT_SWIGLU;
  if (sw != (wq_up_packed != nullptr) || sw != (s_up_i != nullptr))
    return fail(TP_ERR_ACT, "%s: wq_up_packed and s_up_i must be given iff SWIGLU", who);
  if (T == 0 || d == 0) return TP_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (ff_i == 0) {  // empty intermediate: the partial is zero
    if (!y_i) return fail(TP_ERR_NULL, "%s: null y_i", who);
    return hip_status(tpk::zero_fill(y_i, (size_t)T * d * esize(out_dtype), s), who);
  }
  if (!x || !wq1_packed || !s1_i || !wq2_packed || !s2_i || !y_i)
    return fail(TP_ERR_NULL, "%s: null x, wq1_packed, s1_i, wq2_packed, s2_i or y_i", who);
  if (!aligned16(wq1_packed) || !aligned16(wq2_packed) || (sw && !aligned16(wq_up_packed)))
    return fail(TP_ERR_SHAPE, "%s: packed weights must be 16-byte aligned", who);
  const PackedLayout L = packed8_fwd_layout(T, d, ff_i, sw);
  st = packed_ws_ok(who, ws, ws_bytes, L.total);
  if (st != TP_OK) return st;
  char* base = reinterpret_cast<char*>(ws);
  const int nkb = (int)(kpair_pad(d) / 32);
  // column GEMM: h = act(x W1_i [, x W_up_i]) straight into the row GEMM's packed activations
  tpk::PackedParams p1 = packed8_params(base + L.x_off, wq1_packed, s1_i, sw ? wq_up_packed : nullptr,
                                        sw ? s_up_i : nullptr, T, d, ff_i, L.p1, base, L);
  hipError_t e = hipSuccess;
  x_source(p1, L, x, d, true);  // fp8 codes: L.p1
  if (!p1.xrm) {
    e = tpk::pack_act16(x, d, (int)T, (int)d, aligned16(x) && d % 8 == 0, base + L.x_off, s, nkb);
    if (e != hipSuccess) return hip_status(e, who);
  }
  p1.cpk = base + L.h_off;
  p1.cpk_mt = tpk::packed_mt((int)T);
  p1.act = act;
  e = tpk::gemm_packed(p1, L.p1, sw ? tpk::GK_FWD_SWIGLU : tpk::GK_FWD_ACT, false, s, true);
  if (e != hipSuccess) return hip_status(e, who);
  // row GEMM: the full-shape partial y_i = h W2_i
  tpk::PackedParams p2 = packed8_params(base + L.h_off, wq2_packed, s2_i, nullptr, nullptr, T, ff_i, d, L.p2, base, L);
  p2.C = y_i;
  p2.ldc = d;
  p2.vec_out = rows_vec16(y_i, d, esize(out_dtype));
  return hip_status(tpk::gemm_packed(p2, L.p2, tpk::GK_FWD_STORE, out_dtype == TP_F32, s, true), who);
}

// ---- MLP shard backward --------------------------------------------------------------
size_t tp_mlp_shard_bwd_workspace(int64_t T, int64_t d, int64_t ff_i, tp_dtype dtype, tp_act act) {
  if (!valid_dtype(dtype) || !valid_act(act) || !dim_ok(T) || !dim_ok(d) || !dim_ok(ff_i)) return 0;
  if (T == 0) return 0;
  return bwd_layout(T, d, ff_i, dtype, act).total;
}

tp_status tp_mlp_shard_bwd(const void* x, const void* w1_i, const void* w_up_i, const void* w2_i, const void* saved,
                           const void* dy, void* dw1_i, void* dw_up_i, void* dw2_i, void* dx_i, void* ws,
                           size_t ws_bytes, int64_t T, int64_t d, int64_t ff_i, tp_dtype dtype, tp_act act,
                           tp_stream stream) {
  tp_status st = check_common(dtype, act);
  if (st != TP_OK) return st;
  if (!dim_ok(T) || !dim_ok(d) || !dim_ok(ff_i) || !prod_ok(T, d) || !prod_ok(d, ff_i) || !prod_ok(T, 2 * ff_i))
    return fail(TP_ERR_SHAPE, "tp_mlp_shard_bwd: sizes out of range");
  const bool sw = act == TP_ACT_SWIGLU;
  if (sw != (w_up_i != nullptr) || sw != (dw_up_i != nullptr))
    return fail(TP_ERR_ACT, "tp_mlp_shard_bwd: w_up_i and dw_up_i must be given iff SWIGLU");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t es = esize(dtype);
  if (d == 0) return TP_OK;  // every gradient is empty
  if (ff_i == 0) {           // empty intermediate: weight gradients empty, dx_i zero
    if (!dx_i && T > 0) return fail(TP_ERR_NULL, "tp_mlp_shard_bwd: null dx_i");
    return hip_status(T ? tpk::zero_fill(dx_i, (size_t)T * d * es, s) : hipSuccess, "tp_mlp_shard_bwd (ff_i=0)");
  }
  if (!w1_i || !w2_i || !dw1_i || !dw2_i || (T > 0 && (!x || !saved || !dy || !dx_i)))
    return fail(TP_ERR_NULL, "tp_mlp_shard_bwd: null input or output pointer");
  if (T == 0) {
    // no tokens: the weight gradients are zero, dx_i is empty
    hipError_t e = tpk::zero_fill(dw1_i, (size_t)d * ff_i * es, s);
    if (e == hipSuccess && sw) e = tpk::zero_fill(dw_up_i, (size_t)d * ff_i * es, s);
    if (e == hipSuccess) e = tpk::zero_fill(dw2_i, (size_t)d * ff_i * es, s);
    return hip_status(e, "tp_mlp_shard_bwd (T=0)");
  }
  const BwdLayout L = bwd_layout(T, d, ff_i, dtype, act);
  if (!ws) return fail(TP_ERR_WORKSPACE, "tp_mlp_shard_bwd: workspace required (%zu bytes)", L.total);
  if (ws_bytes < L.total)
    return fail(TP_ERR_WORKSPACE, "tp_mlp_shard_bwd: workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  char* base = reinterpret_cast<char*>(ws);
  char* dgu = base + L.dgu_off;     // (T, 2 ff_i) [dG | dU] for SWIGLU, (T, ff_i) dA otherwise
  char* h = base + L.h_off;         // (T, ff_i) recomputed activation
  char* cnt = base + L.cnt_off;
  char* part = base + L.part_off;
  const int64_t ldg = sw ? 2 * ff_i : ff_i;

  // (a) dh = dy W2^T, epilogue -> dG/dU (or dA) and h
  GemmParams pa = base_params();
  pa.A0 = dy;
  pa.lda = d;
  pa.B0 = w2_i;  // B(k = hidden j, n = f) = w2_i[f * d + j]
  pa.ldb = d;
  pa.K0 = (int)d;
  pa.M = (int)T;
  pa.N = (int)ff_i;
  pa.C = dgu;
  pa.ldc = ldg;
  pa.C2 = sw ? dgu + ff_i * es : nullptr;
  pa.ldc2 = ldg;
  pa.C3 = h;
  pa.ldc3 = ff_i;
  pa.S0 = saved;
  pa.S1 = sw ? reinterpret_cast<const char*>(saved) + ff_i * es : nullptr;
  pa.lds = ldg;
  pa.act = act;
  pa.vecA = aligned16(dy) && d % 8 == 0;
  pa.vecB = aligned16(w2_i) && d % 8 == 0;
  attach_split(pa, L.pa, cnt, part, base + L.pack_off);
  hipError_t e = run_gemm(dtype, pa, L.pa, sw ? tpk::GK_BWD_DH_SWIGLU : tpk::GK_BWD_DH_ACT, false, s);
  if (e != hipSuccess) return hip_status(e, "tp_mlp_shard_bwd (dh GEMM)");

  // (b) dW2 = h^T dy
  GemmParams pb = base_params();
  pb.A0 = h;  // A(m = f, k = t) = h[t * ff_i + f]
  pb.lda = ff_i;
  pb.B0 = dy;  // B(k = t, n = j) = dy[t * d + j]
  pb.ldb = d;
  pb.K0 = (int)T;
  pb.M = (int)ff_i;
  pb.N = (int)d;
  pb.C = dw2_i;
  pb.ldc = d;
  pb.vecA = ff_i % 8 == 0;
  pb.vecB = aligned16(dy) && d % 8 == 0;
  attach_split(pb, L.pb, cnt, part, base + L.pack_off);
  e = run_gemm(dtype, pb, L.pb, tpk::GK_BWD_DW, false, s);
  if (e != hipSuccess) return hip_status(e, "tp_mlp_shard_bwd (dW2 GEMM)");

  // (c) dW1 = x^T dG (and dWup = x^T dU)
  GemmParams pc = base_params();
  pc.A0 = x;  // A(m = j, k = t) = x[t * d + j]
  pc.lda = d;
  pc.B0 = dgu;  // B(k = t, n = f) = dG[t * ldg + f]
  pc.B1 = sw ? dgu + ff_i * es : nullptr;
  pc.ldb = ldg;
  pc.K0 = (int)T;
  pc.M = (int)d;
  pc.N = (int)ff_i;
  pc.C = dw1_i;
  pc.ldc = ff_i;
  pc.C2 = dw_up_i;
  pc.ldc2 = ff_i;
  pc.vecA = aligned16(x) && d % 8 == 0;
  pc.vecB = ff_i % 8 == 0;
  attach_split(pc, L.pc, cnt, part, base + L.pack_off);
  e = run_gemm(dtype, pc, L.pc, sw ? tpk::GK_BWD_DW_DUAL : tpk::GK_BWD_DW, false, s);
  if (e != hipSuccess) return hip_status(e, "tp_mlp_shard_bwd (dW1 GEMM)");

  // (d) dx_i = dG W1^T (+ dU Wup^T): two K segments
  GemmParams pd = base_params();
  pd.A0 = dgu;  // A(m = t, k = f) = dG[t * ldg + f]
  pd.A1 = sw ? dgu + ff_i * es : nullptr;
  pd.lda = ldg;
  pd.B0 = w1_i;  // B(k = f, n = j) = w1_i[j * ff_i + f]
  pd.B1 = w_up_i;
  pd.ldb = ff_i;
  pd.K0 = (int)ff_i;
  pd.K1 = sw ? (int)ff_i : 0;
  pd.M = (int)T;
  pd.N = (int)d;
  pd.C = dx_i;
  pd.ldc = d;
  pd.vecA = ff_i % 8 == 0;
  pd.vecB = aligned16(w1_i) && (!sw || aligned16(w_up_i)) && ff_i % 8 == 0;
  attach_split(pd, L.pd, cnt, part, base + L.pack_off);
  e = run_gemm(dtype, pd, L.pd, tpk::GK_BWD_DX, false, s);
  return hip_status(e, "tp_mlp_shard_bwd (dx GEMM)");
}

size_t tp_linear_shard_bwd_workspace(int64_t T, int64_t K, int64_t N, tp_dtype dtype) {
  if (!valid_dtype(dtype) || !dim_ok(T) || !dim_ok(K) || !dim_ok(N) || T == 0) return 0;
  return lin_bwd_layout(T, K, N, dtype).total;
}

tp_status tp_linear_shard_bwd(const void* x, const void* w, const void* dy, void* dw, void* dx, void* ws,
                              size_t ws_bytes, int64_t T, int64_t K, int64_t N, tp_dtype dtype, tp_stream stream) {
  if (!valid_dtype(dtype)) return fail(TP_ERR_DTYPE, "tp_linear_shard_bwd: unknown dtype %d", dtype);
  if (!dim_ok(T) || !dim_ok(K) || !dim_ok(N) || !prod_ok(T, K) || !prod_ok(K, N) || !prod_ok(T, N))
    return fail(TP_ERR_SHAPE, "tp_linear_shard_bwd: sizes out of range");
  // a pointer to an empty array may be NULL
  if (!dw && !dx && (K * N > 0 || T * K > 0))
    return fail(TP_ERR_NULL, "tp_linear_shard_bwd: neither dw nor dx requested");
  if ((!dy && T * N > 0 && (dw || dx)) || (dw && !x && T * K > 0) || (dx && !w && K * N > 0))
    return fail(TP_ERR_NULL, "tp_linear_shard_bwd: null input pointer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t es = esize(dtype);
  if (T == 0) {
    // no tokens: the weight gradient is zero, dx is empty
    return hip_status(dw ? tpk::zero_fill(dw, (size_t)K * N * es, s) : hipSuccess, "tp_linear_shard_bwd (T=0)");
  }
  if (K == 0) return TP_OK;
  if (N == 0)  // an empty contraction: dx is zero, dW is empty
    return hip_status(dx ? tpk::zero_fill(dx, (size_t)T * K * es, s) : hipSuccess, "tp_linear_shard_bwd (N=0)");
  const LinBwdLayout L = lin_bwd_layout(T, K, N, dtype);
  if (L.total && !ws) return fail(TP_ERR_WORKSPACE, "tp_linear_shard_bwd: workspace required (%zu bytes)", L.total);
  if (ws_bytes < L.total)
    return fail(TP_ERR_WORKSPACE, "tp_linear_shard_bwd: workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  char* base = reinterpret_cast<char*>(ws);
  char* cnt = L.total ? base + L.cnt_off : nullptr;
  char* part = L.total ? base + L.part_off : nullptr;
  char* pack = L.total ? base + L.pack_off : nullptr;
  hipError_t e = hipSuccess;
  if (dw) {
    // dW = x^T dy: A(m = k, k = t) = x[t * K + k], B(k = t, n) = dy[t * N + n]
    GemmParams pw = base_params();
    pw.A0 = x;
    pw.lda = K;
    pw.B0 = dy;
    pw.ldb = N;
    pw.K0 = (int)T;
    pw.M = (int)K;
    pw.N = (int)N;
    pw.C = dw;
    pw.ldc = N;
    pw.vecA = aligned16(x) && K % 8 == 0;
    pw.vecB = aligned16(dy) && N % 8 == 0;
    attach_split(pw, L.pw, cnt, part, pack);
    e = run_gemm(dtype, pw, L.pw, tpk::GK_BWD_DW, false, s);
    if (e != hipSuccess) return hip_status(e, "tp_linear_shard_bwd (dW GEMM)");
  }
  if (dx) {
    // dx = dy W^T: A(m = t, k = n) = dy[t * N + n], B(k = n, n' = k) = w[k * N + n]
    GemmParams px = base_params();
    px.A0 = dy;
    px.lda = N;
    px.B0 = w;
    px.ldb = N;
    px.K0 = (int)N;
    px.M = (int)T;
    px.N = (int)K;
    px.C = dx;
    px.ldc = K;
    px.vecA = aligned16(dy) && N % 8 == 0;
    px.vecB = aligned16(w) && N % 8 == 0;
    attach_split(px, L.px, cnt, part, pack);
    e = run_gemm(dtype, px, L.px, tpk::GK_BWD_DX, false, s);
  }
  return hip_status(e, "tp_linear_shard_bwd (dx GEMM)");
}

tp_status tp_gqa_attention_fwd(const void* qkv, void* out, int64_t T, int n_q, int n_kv, int head_dim, int causal,
                               float scale, tp_stream stream) {
  if (!dim_ok(T) || n_q < 1 || n_kv < 1 || n_q % n_kv != 0 || head_dim < 1)
    return fail(TP_ERR_SHAPE, "tp_gqa_attention_fwd: bad sizes (T=%lld, n_q=%d, n_kv=%d, head_dim=%d)", (long long)T,
                n_q, n_kv, head_dim);
  if (causal != 0 && causal != 1) return fail(TP_ERR_SHAPE, "tp_gqa_attention_fwd: causal must be 0 or 1");
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return fail(TP_ERR_SHAPE, "tp_gqa_attention_fwd: scale must be finite and > 0");
  if (head_dim != tpk::attention_head_dim())
    return fail(TP_ERR_UNSUPPORTED, "tp_gqa_attention_fwd: head_dim %d (only %d is built)", head_dim,
                tpk::attention_head_dim());
  const int64_t width = (int64_t)(n_q + 2 * n_kv) * head_dim;
  // a 64-row key tile of one row stride must stay within 32-bit buffer offsets
  if (width > (1 << 23) || !prod_ok(T, width)) return fail(TP_ERR_SHAPE, "tp_gqa_attention_fwd: sizes out of range");
  if ((T + 63) / 64 * n_q > kMaxDim)  // one workgroup per (query block, head)
    return fail(TP_ERR_SHAPE, "tp_gqa_attention_fwd: too many query blocks x heads for one launch");
  if (T == 0) return TP_OK;
  if (!qkv || !out) return fail(TP_ERR_NULL, "tp_gqa_attention_fwd: null qkv or out");
  if (!aligned16(qkv) || !aligned16(out))
    return fail(TP_ERR_UNSUPPORTED, "tp_gqa_attention_fwd: qkv and out must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return hip_status(tpk::gqa_attention_fwd(qkv, out, (int)T, n_q, n_kv, causal == 1, scale, s), "tp_gqa_attention_fwd");
}

}  // extern "C"
