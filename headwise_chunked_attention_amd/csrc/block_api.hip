// Host engine of the checkpointed pre-norm transformer block behind the C ABI.
//
// The block composes the attention op (its own C entry points, chunked
// heads in one reused workspace) and the sequence-tiled MLP engine with the
// row RMSNorm kernels:
//   a = rmsnorm(x; g_attn)      h = x + attention(a)
//   b = rmsnorm(h; g_mlp)       y = h + mlp(b)
// Activation checkpointing keeps only the block input (talk "Road to
// 5 Million Tokens", the memory-optimization progression; liquidgold.cc
// notes, "Progression of Techniques", items 4 and 5): the backward recomputes
// a and, unless the caller kept it, h.
//
// Workspace (256-byte aligned regions):
//   A   [N][D]   a = rmsnorm(x), the attention's input (forward and backward)
//   DA  [N][D]   the attention's dx (backward)
//   B   [T][D]   one tile of b (the MLP's input)
//   DB  [T][D]   one tile of the MLP's dx (backward)
//   LSE [Hq][N]  fp32, the lse when the caller keeps none
//   O   [Hq][Np][d]  backward from the block input alone: every head's O,
//                kept by the rerun attention forward so that the attention
//                backward does not recompute it (Np = N padded)
//   stage        shared by the attention op and the MLP, which never run at
//                the same time: the larger of their workspaces
// Buffers reused across steps of the backward: dx first holds the
// recomputed attention output, then h (tile by tile), then dh = dL/dh, then
// the final dx; each step reads a row of it before writing that row.
#include <math.h>
#include <string.h>

#include "upipe.h"
#include "host.h"
#include "kernels.h"
#include "mlp.h"

using namespace upipe;
using namespace upipe::host;

namespace {

struct BlockShape {
  upipe_block_shape_t a;  // as given
  mlp::Shape m;
  bool qk_norm;
  int es;
};

struct BlockPlan {
  size_t A, DA, B, DB, lse, O, stage, total;
};

int block_check_shape(int dtype, const upipe_block_shape_t* sh, int qk_norm, BlockShape* out) {
  if (sh == nullptr) return UPIPE_ERR_INVALID_ARG;
  const upipe_block_shape_t& s = *sh;
  int rc = attn_check_args(dtype, s.n_tokens, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.rope_theta,
                           s.chunk_heads, s.qk_norm_eps);
  if (rc) return rc;
  mlp::Shape m;
  if ((rc = mlp::check_shape(dtype, s.n_tokens, s.d_model, s.d_ff, s.tile_tokens, &m))) return rc;
  if (!(s.norm_eps >= 0.f) || !isfinite(s.norm_eps)) return UPIPE_ERR_INVALID_ARG;
  if (s.d_model > ROW_NORM_MAX_D) return UPIPE_ERR_UNSUPPORTED;
  out->a = s;
  out->m = m;
  out->qk_norm = qk_norm != 0;
  out->es = dtype == UPIPE_BF16 ? 2 : 4;
  return UPIPE_OK;
}

size_t attn_ws(const BlockShape& b, upipe_dtype_t dt, int backward) {
  const upipe_block_shape_t& s = b.a;
  return upipe_attn_workspace_bytes(s.n_tokens, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.chunk_heads,
                                    b.qk_norm ? 1 : 0, dt, backward);
}

BlockPlan block_plan(const BlockShape& b, upipe_dtype_t dt, bool backward) {
  BlockPlan p;
  memset(&p, 0, sizeof(p));
  const upipe_block_shape_t& s = b.a;
  const size_t nd = (size_t)s.n_tokens * s.d_model * b.es;
  const size_t td = (size_t)b.m.T * s.d_model * b.es;
  Carver c;
  p.A = c.take(nd);
  if (backward) p.DA = c.take(nd);
  p.B = c.take(td);
  if (backward) p.DB = c.take(td);
  p.lse = c.take((size_t)s.n_q_heads * s.n_tokens * 4);
  if (backward) p.O = c.take((size_t)s.n_q_heads * attn_padded_rows(s.n_tokens) * s.head_dim * b.es);
  size_t stage = attn_ws(b, dt, 0);
  const size_t mw = mlp::plan(b.m, backward).total;
  if (mw > stage) stage = mw;
  if (backward) {
    const size_t ab = attn_ws(b, dt, 1);
    if (ab > stage) stage = ab;
  }
  p.stage = c.take(stage);
  p.total = c.off;
  return p;
}

template <typename T>
int row_norm(const T* x, const T* r, const T* gamma, T* u_out, T* u_out2, T* n_out, int64_t rows, int64_t D,
             float eps, hipStream_t st) {
  RowNorm<T> p;
  memset(&p, 0, sizeof(p));
  p.x = x;
  p.r = r;
  p.gamma = gamma;
  p.u_out = u_out;
  p.u_out2 = u_out2;
  p.n_out = n_out;
  p.rows = rows;
  p.D = D;
  p.eps = eps;
  HIP_TRY(timed(UPIPE_KERNEL_BLOCK_NORM, 0.0, st, [&] { return launch_row_norm<T>(p, st); }));
  return UPIPE_OK;
}

template <typename T>
int row_norm_bwd(const T* u, const T* g, const T* gamma, const T* res, T* out, float* dgamma, int64_t rows,
                 int64_t D, float eps, hipStream_t st) {
  RowNormBwd<T> p;
  memset(&p, 0, sizeof(p));
  p.u = u;
  p.g = g;
  p.gamma = gamma;
  p.res = res;
  p.out = out;
  p.dgamma = dgamma;
  p.rows = rows;
  p.D = D;
  p.eps = eps;
  HIP_TRY(timed(UPIPE_KERNEL_BLOCK_NORM, 0.0, st, [&] { return launch_row_norm_bwd<T>(p, st); }));
  return UPIPE_OK;
}

template <typename T>
int attn_fwd_call(const BlockShape& b, upipe_dtype_t dt, const T* a, const upipe_block_weights_t& w, T* y,
                  float* lse, char* stage, size_t stage_bytes, hipStream_t st) {
  const upipe_block_shape_t& s = b.a;
  return upipe_attn_fwd(dt, s.n_tokens, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.rope_theta,
                        s.chunk_heads, a, w.wq, w.wk, w.wv, w.wo, w.q_norm, w.k_norm, s.qk_norm_eps, y, lse, stage,
                        stage_bytes, st);
}

template <typename T>
int block_fwd_impl(const BlockShape& b, upipe_dtype_t dt, const T* x, const upipe_block_weights_t& w, T* y,
                   T* h_mid, float* lse, char* ws, hipStream_t st) {
  const BlockPlan pl = block_plan(b, dt, false);
  const int64_t N = b.a.n_tokens, D = b.a.d_model, TT = b.m.T;
  const float eps = b.a.norm_eps;
  T* A = reinterpret_cast<T*>(ws + pl.A);
  T* B = reinterpret_cast<T*>(ws + pl.B);
  float* L = lse ? lse : reinterpret_cast<float*>(ws + pl.lse);
  // a = rmsnorm(x); y = attention(a)
  int rc = row_norm<T>(x, nullptr, (const T*)w.attn_norm, nullptr, nullptr, A, N, D, eps, st);
  if (rc) return rc;
  if ((rc = attn_fwd_call<T>(b, dt, A, w, y, L, ws + pl.stage, pl.total - pl.stage, st))) return rc;
  // per tile: h = x + y (into y, and h_mid), b = rmsnorm(h), y = h + mlp(b)
  for (int64_t t0 = 0; t0 < N; t0 += TT) {
    const int64_t rows = N - t0 < TT ? N - t0 : TT;
    T* yt = y + t0 * D;
    if ((rc = row_norm<T>(x + t0 * D, yt, (const T*)w.mlp_norm, yt, h_mid ? h_mid + t0 * D : nullptr, B, rows, D,
                          eps, st)))
      return rc;
    if ((rc = mlp::fwd_tile<T>(b.m, B, rows, (const T*)w.w_gate, (const T*)w.w_up, (const T*)w.w_down, yt, yt,
                               ws + pl.stage, st)))
      return rc;
  }
  return UPIPE_OK;
}

template <typename T>
int block_bwd_impl(const BlockShape& b, upipe_dtype_t dt, const T* x, const upipe_block_weights_t& w,
                   const T* h_mid, const float* lse, const T* dy, T* dx, const upipe_block_grads_t& g, char* ws,
                   hipStream_t st) {
  const BlockPlan pl = block_plan(b, dt, true);
  const upipe_block_shape_t& s = b.a;
  const int64_t N = s.n_tokens, D = s.d_model, TT = b.m.T;
  const float eps = s.norm_eps;
  T* A = reinterpret_cast<T*>(ws + pl.A);
  T* DA = reinterpret_cast<T*>(ws + pl.DA);
  T* B = reinterpret_cast<T*>(ws + pl.B);
  T* DB = reinterpret_cast<T*>(ws + pl.DB);
  char* stage = ws + pl.stage;
  const size_t stage_bytes = pl.total - pl.stage;
  const bool recompute = h_mid == nullptr;
  const T* gm_attn = (const T*)w.attn_norm;
  const T* gm_mlp = (const T*)w.mlp_norm;
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(g.attn_norm, D, 0.f, st); }));
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(g.mlp_norm, D, 0.f, st); }));
  // a = rmsnorm(x); without a kept h, the attention output (into dx) and lse
  int rc = row_norm<T>(x, nullptr, gm_attn, nullptr, nullptr, A, N, D, eps, st);
  if (rc) return rc;
  const float* L = lse;
  T* Okept = nullptr;
  const AttnCall ac = {dt, N, D, s.n_q_heads, s.n_kv_heads, s.head_dim, s.rope_theta, s.chunk_heads, s.qk_norm_eps};
  if (recompute) {
    float* Lw = reinterpret_cast<float*>(ws + pl.lse);
    Okept = reinterpret_cast<T*>(ws + pl.O);
    if ((rc = attn_fwd_keep_o<T>(ac, A, w.wq, w.wk, w.wv, w.wo, w.q_norm, w.k_norm, dx, Lw, Okept, stage,
                                 stage_bytes, st)))
      return rc;
    L = Lw;
  }
  // MLP half, tile by tile: b = rmsnorm(h), db = mlp_bwd(b, dy),
  // dh = dy + rmsnorm_bwd(h, db) (into dx)
  if ((rc = mlp::bwd_prep<T>(b.m, (const T*)w.w_gate, (const T*)w.w_up, (const T*)w.w_down, g.w_gate, g.w_up,
                             g.w_down, stage, st)))
    return rc;
  for (int64_t t0 = 0; t0 < N; t0 += TT) {
    const int64_t rows = N - t0 < TT ? N - t0 : TT;
    T* dxt = dx + t0 * D;
    const T* ht = recompute ? dxt : h_mid + t0 * D;
    if (recompute)  // h = x + attention output, kept in dx for the norm's backward
      rc = row_norm<T>(x + t0 * D, dxt, gm_mlp, dxt, nullptr, B, rows, D, eps, st);
    else
      rc = row_norm<T>(ht, nullptr, gm_mlp, nullptr, nullptr, B, rows, D, eps, st);
    if (rc) return rc;
    if ((rc = mlp::bwd_tile<T>(b.m, B, dy + t0 * D, rows, (const T*)w.w_gate, (const T*)w.w_up, DB, g.w_gate,
                               g.w_up, g.w_down, stage, st)))
      return rc;
    if ((rc = row_norm_bwd<T>(ht, DB, gm_mlp, dy + t0 * D, dxt, g.mlp_norm, rows, D, eps, st))) return rc;
  }
  // attention half: da = attention_bwd(a, dh); dx = dh + rmsnorm_bwd(x, da)
  if (Okept)
    rc = attn_bwd_kept_o<T>(ac, A, w.wq, w.wk, w.wv, w.wo, w.q_norm, w.k_norm, dx, L, Okept, DA, g.wq, g.wk, g.wv,
                            g.wo, g.q_norm, g.k_norm, stage, stage_bytes, st);
  else
    rc = upipe_attn_bwd(dt, N, D, s.n_q_heads, s.n_kv_heads, s.head_dim, s.rope_theta, s.chunk_heads, A, w.wq, w.wk,
                        w.wv, w.wo, w.q_norm, w.k_norm, s.qk_norm_eps, dx, L, DA, g.wq, g.wk, g.wv, g.wo, g.q_norm,
                        g.k_norm, stage, stage_bytes, st);
  if (rc) return rc;
  return row_norm_bwd<T>(x, DA, gm_attn, dx, dx, g.attn_norm, N, D, eps, st);
}

int check_ptrs(const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (ptrs[i] == nullptr) return UPIPE_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (!aligned(ptrs[i], 16)) return UPIPE_ERR_ALIGNMENT;
  return UPIPE_OK;
}

// Optional pointers: alignment only.
int check_opt(const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (ptrs[i] != nullptr && !aligned(ptrs[i], 16)) return UPIPE_ERR_ALIGNMENT;
  return UPIPE_OK;
}

int check_weights(const upipe_block_weights_t* w, bool* qk_norm) {
  if (w == nullptr) return UPIPE_ERR_INVALID_ARG;
  if ((w->q_norm == nullptr) != (w->k_norm == nullptr)) return UPIPE_ERR_INVALID_ARG;
  const void* p[] = {w->attn_norm, w->wq, w->wk, w->wv, w->wo, w->mlp_norm, w->w_gate, w->w_up, w->w_down};
  int rc = check_ptrs(p, 9);
  if (rc) return rc;
  *qk_norm = w->q_norm != nullptr;
  if (*qk_norm) {
    const void* n[] = {w->q_norm, w->k_norm};
    if ((rc = check_ptrs(n, 2))) return rc;
  }
  return UPIPE_OK;
}

int check_ws(const BlockShape& b, upipe_dtype_t dt, bool bwd, const void* ws, size_t bytes) {
  if (ws == nullptr) return UPIPE_ERR_WORKSPACE;
  if (!aligned(ws, REGION_ALIGN)) return UPIPE_ERR_ALIGNMENT;
  if (bytes < block_plan(b, dt, bwd).total) return UPIPE_ERR_WORKSPACE;
  return UPIPE_OK;
}

// ---------------------------------------------------------------------------
// A stack of blocks with the block inputs offloaded to host memory (the
// talk's CPU offload: block inputs leave the GPU between the passes and come
// back, prefetched, for the backward; liquidgold.cc notes, "Progression of
// Techniques", item 5; talk transcript, the part on CPU offloading).
//
// Device buffers, whatever the number of layers: two activation buffers P
// (the forward's block outputs; the backward's prefetched block inputs), two
// gradient buffers G, and one block workspace. Copies run on the caller's
// copy stream, ordered against the compute stream by events:
//   forward   copy of block l's input to host[l] overlaps block l; block l+1,
//             which overwrites that input's buffer, waits for the copy;
//   backward  the input of block l - 2 is fetched into the buffer block l
//             has just finished with, while blocks l - 1 and l - 2 wait for
//             their own inputs only.
// ---------------------------------------------------------------------------
struct StackPlan {
  size_t act[2], grad[2], block, total;
};

StackPlan stack_plan(const BlockShape& b, upipe_dtype_t dt) {
  StackPlan p;
  memset(&p, 0, sizeof(p));
  const size_t nd = (size_t)b.a.n_tokens * b.a.d_model * b.es;
  Carver c;
  p.act[0] = c.take(nd);
  p.act[1] = c.take(nd);
  p.grad[0] = c.take(nd);
  p.grad[1] = c.take(nd);
  size_t bw = block_plan(b, dt, false).total;
  const size_t bb = block_plan(b, dt, true).total;
  if (bb > bw) bw = bb;
  p.block = c.take(bw);
  p.total = c.off;
  return p;
}

// Events of one call, destroyed when the call returns (a recorded event may
// be destroyed before it completes; waits already enqueued keep their meaning).
struct Events {
  hipEvent_t e[6] = {};
  int n = 0;
  ~Events() {
    for (int i = 0; i < n; ++i) hipEventDestroy(e[i]);
  }
  hipError_t make(int count) {
    for (; n < count; ++n) {
      const hipError_t r = hipEventCreateWithFlags(&e[n], hipEventDisableTiming);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
};

template <typename T>
int stack_fwd_impl(const BlockShape& b, upipe_dtype_t dt, int L, const upipe_block_weights_t* w, const T* x, T* y,
                   T* host, char* ws, hipStream_t st, hipStream_t cs) {
  const StackPlan pl = stack_plan(b, dt);
  const size_t nd = (size_t)b.a.n_tokens * b.a.d_model;
  T* P[2] = {reinterpret_cast<T*>(ws + pl.act[0]), reinterpret_cast<T*>(ws + pl.act[1])};
  char* bws = ws + pl.block;
  Events ev;
  HIP_TRY(ev.make(3));
  hipEvent_t ready = ev.e[0], copied[2] = {ev.e[1], ev.e[2]};
  HIP_TRY(hipEventRecord(ready, st));  // x and the workspace, as the caller's stream left them
  const T* in = x;
  for (int l = 0; l < L; ++l) {
    HIP_TRY(hipStreamWaitEvent(cs, ready, 0));
    HIP_TRY(hipMemcpyAsync(host + (size_t)l * nd, in, nd * sizeof(T), hipMemcpyDefault, cs));
    HIP_TRY(hipEventRecord(copied[l % 2], cs));
    T* out = l == L - 1 ? y : P[l % 2];
    // out's buffer holds block l-1's input (from l = 2 on): its copy must be done
    if (l >= 2 && l < L - 1) HIP_TRY(hipStreamWaitEvent(st, copied[(l - 1) % 2], 0));
    int rc = block_fwd_impl<T>(b, dt, in, w[l], out, nullptr, nullptr, bws, st);
    if (rc) return rc;
    HIP_TRY(hipEventRecord(ready, st));
    in = out;
  }
  // the caller's stream covers the last copy: host is complete when it syncs
  HIP_TRY(hipStreamWaitEvent(st, copied[(L - 1) % 2], 0));
  return UPIPE_OK;
}

template <typename T>
int stack_bwd_impl(const BlockShape& b, upipe_dtype_t dt, int L, const upipe_block_weights_t* w, const T* host,
                   const T* dy, T* dx, const upipe_block_grads_t* g, char* ws, hipStream_t st, hipStream_t cs) {
  const StackPlan pl = stack_plan(b, dt);
  const size_t nd = (size_t)b.a.n_tokens * b.a.d_model;
  T* P[2] = {reinterpret_cast<T*>(ws + pl.act[0]), reinterpret_cast<T*>(ws + pl.act[1])};
  T* G[2] = {reinterpret_cast<T*>(ws + pl.grad[0]), reinterpret_cast<T*>(ws + pl.grad[1])};
  char* bws = ws + pl.block;
  Events ev;
  HIP_TRY(ev.make(5));
  hipEvent_t start = ev.e[0], in_ev[2] = {ev.e[1], ev.e[2]}, used[2] = {ev.e[3], ev.e[4]};
  HIP_TRY(hipEventRecord(start, st));
  HIP_TRY(hipStreamWaitEvent(cs, start, 0));  // the workspace is free of the caller's earlier work
  auto fetch = [&](int l) -> hipError_t {
    hipError_t e = hipMemcpyAsync(P[l % 2], host + (size_t)l * nd, nd * sizeof(T), hipMemcpyDefault, cs);
    if (e != hipSuccess) return e;
    return hipEventRecord(in_ev[l % 2], cs);
  };
  HIP_TRY(fetch(L - 1));
  if (L >= 2) HIP_TRY(fetch(L - 2));
  for (int l = L - 1; l >= 0; --l) {
    HIP_TRY(hipStreamWaitEvent(st, in_ev[l % 2], 0));
    const T* dyl = l == L - 1 ? dy : G[(l + 1) % 2];
    T* dxl = l == 0 ? dx : G[l % 2];
    int rc = block_bwd_impl<T>(b, dt, P[l % 2], w[l], nullptr, nullptr, dyl, dxl, g[l], bws, st);
    if (rc) return rc;
    if (l >= 2) {
      HIP_TRY(hipEventRecord(used[l % 2], st));
      HIP_TRY(hipStreamWaitEvent(cs, used[l % 2], 0));
      HIP_TRY(fetch(l - 2));
    }
  }
  return UPIPE_OK;
}

int check_grads(const upipe_block_grads_t* grads, bool qk) {
  if (grads == nullptr) return UPIPE_ERR_INVALID_ARG;
  const void* p[] = {grads->attn_norm, grads->wq, grads->wk, grads->wv, grads->wo, grads->mlp_norm,
                     grads->w_gate, grads->w_up, grads->w_down};
  int rc = check_ptrs(p, 9);
  if (rc) return rc;
  if (qk) {
    const void* n[] = {grads->q_norm, grads->k_norm};
    return check_ptrs(n, 2);
  }
  return (grads->q_norm != nullptr || grads->k_norm != nullptr) ? UPIPE_ERR_INVALID_ARG : UPIPE_OK;
}

// Shape and every layer's weights (and gradients, if given); all layers must
// agree on having q/k norm.
int stack_check(int dtype, const upipe_block_shape_t* shape, int L, const upipe_block_weights_t* w,
                const upipe_block_grads_t* g, BlockShape* b) {
  if (L < 1 || w == nullptr) return UPIPE_ERR_INVALID_ARG;
  bool qk0 = false;
  for (int l = 0; l < L; ++l) {
    bool qk = false;
    int rc = check_weights(&w[l], &qk);
    if (rc) return rc;
    if (l == 0) qk0 = qk;
    if (qk != qk0) return UPIPE_ERR_INVALID_ARG;
    if (g && (rc = check_grads(&g[l], qk))) return rc;
  }
  return block_check_shape(dtype, shape, qk0, b);
}

}  // namespace

extern "C" {

size_t upipe_stack_workspace_bytes(const upipe_block_shape_t* shape, int qk_norm, upipe_dtype_t dtype) {
  BlockShape b;
  if (block_check_shape(dtype, shape, qk_norm, &b)) return 0;
  return stack_plan(b, dtype).total;
}

int upipe_stack_fwd(upipe_dtype_t dtype, const upipe_block_shape_t* shape, int n_layers,
                    const upipe_block_weights_t* weights, const void* x, void* y, void* host_inputs,
                    void* workspace, size_t workspace_bytes, void* stream, void* copy_stream) {
  BlockShape b;
  int rc = stack_check(dtype, shape, n_layers, weights, nullptr, &b);
  if (rc) return rc;
  const void* p[] = {x, y, host_inputs};
  if ((rc = check_ptrs(p, 3))) return rc;
  if (workspace == nullptr) return UPIPE_ERR_WORKSPACE;
  if (!aligned(workspace, REGION_ALIGN)) return UPIPE_ERR_ALIGNMENT;
  if (workspace_bytes < stack_plan(b, dtype).total) return UPIPE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipStream_t cs = copy_stream ? reinterpret_cast<hipStream_t>(copy_stream) : st;
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16)
    return stack_fwd_impl<bf16>(b, dtype, n_layers, weights, (const bf16*)x, (bf16*)y, (bf16*)host_inputs, ws, st,
                                cs);
  return stack_fwd_impl<float>(b, dtype, n_layers, weights, (const float*)x, (float*)y, (float*)host_inputs, ws, st,
                               cs);
}

int upipe_stack_bwd(upipe_dtype_t dtype, const upipe_block_shape_t* shape, int n_layers,
                    const upipe_block_weights_t* weights, const void* host_inputs, const void* dy, void* dx,
                    const upipe_block_grads_t* grads, void* workspace, size_t workspace_bytes, void* stream,
                    void* copy_stream) {
  BlockShape b;
  if (grads == nullptr) return UPIPE_ERR_INVALID_ARG;
  int rc = stack_check(dtype, shape, n_layers, weights, grads, &b);
  if (rc) return rc;
  const void* p[] = {host_inputs, dy, dx};
  if ((rc = check_ptrs(p, 3))) return rc;
  if (workspace == nullptr) return UPIPE_ERR_WORKSPACE;
  if (!aligned(workspace, REGION_ALIGN)) return UPIPE_ERR_ALIGNMENT;
  if (workspace_bytes < stack_plan(b, dtype).total) return UPIPE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipStream_t cs = copy_stream ? reinterpret_cast<hipStream_t>(copy_stream) : st;
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16)
    return stack_bwd_impl<bf16>(b, dtype, n_layers, weights, (const bf16*)host_inputs, (const bf16*)dy, (bf16*)dx,
                                grads, ws, st, cs);
  return stack_bwd_impl<float>(b, dtype, n_layers, weights, (const float*)host_inputs, (const float*)dy,
                               (float*)dx, grads, ws, st, cs);
}

size_t upipe_block_workspace_bytes(const upipe_block_shape_t* shape, int qk_norm, upipe_dtype_t dtype,
                                   int backward) {
  BlockShape b;
  if (block_check_shape(dtype, shape, qk_norm, &b)) return 0;
  return block_plan(b, dtype, backward != 0).total;
}

int upipe_block_fwd(upipe_dtype_t dtype, const upipe_block_shape_t* shape, const void* x,
                    const upipe_block_weights_t* w, void* y, void* h_mid, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  bool qk = false;
  int rc = check_weights(w, &qk);
  if (rc) return rc;
  BlockShape b;
  if ((rc = block_check_shape(dtype, shape, qk, &b))) return rc;
  const void* p[] = {x, y};
  if ((rc = check_ptrs(p, 2))) return rc;
  const void* o[] = {h_mid, lse};
  if ((rc = check_opt(o, 2))) return rc;
  if ((rc = check_ws(b, dtype, false, workspace, workspace_bytes))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16)
    return block_fwd_impl<bf16>(b, dtype, (const bf16*)x, *w, (bf16*)y, (bf16*)h_mid, lse, ws, st);
  return block_fwd_impl<float>(b, dtype, (const float*)x, *w, (float*)y, (float*)h_mid, lse, ws, st);
}

int upipe_block_bwd(upipe_dtype_t dtype, const upipe_block_shape_t* shape, const void* x,
                    const upipe_block_weights_t* w, const void* h_mid, const float* lse, const void* dy, void* dx,
                    const upipe_block_grads_t* grads, void* workspace, size_t workspace_bytes, void* stream) {
  bool qk = false;
  int rc = check_weights(w, &qk);
  if (rc) return rc;
  BlockShape b;
  if ((rc = block_check_shape(dtype, shape, qk, &b))) return rc;
  if (grads == nullptr) return UPIPE_ERR_INVALID_ARG;
  if ((h_mid == nullptr) != (lse == nullptr)) return UPIPE_ERR_INVALID_ARG;
  const void* p[] = {x, dy, dx, grads->attn_norm, grads->wq, grads->wk, grads->wv, grads->wo, grads->mlp_norm,
                     grads->w_gate, grads->w_up, grads->w_down};
  if ((rc = check_ptrs(p, 12))) return rc;
  if (qk) {
    const void* n[] = {grads->q_norm, grads->k_norm};
    if ((rc = check_ptrs(n, 2))) return rc;
  } else if (grads->q_norm != nullptr || grads->k_norm != nullptr) {
    return UPIPE_ERR_INVALID_ARG;
  }
  const void* o[] = {h_mid, lse};
  if ((rc = check_opt(o, 2))) return rc;
  if ((rc = check_ws(b, dtype, true, workspace, workspace_bytes))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16)
    return block_bwd_impl<bf16>(b, dtype, (const bf16*)x, *w, (const bf16*)h_mid, lse, (const bf16*)dy, (bf16*)dx,
                                *grads, ws, st);
  return block_bwd_impl<float>(b, dtype, (const float*)x, *w, (const float*)h_mid, lse, (const float*)dy,
                               (float*)dx, *grads, ws, st);
}

}  // extern "C"
