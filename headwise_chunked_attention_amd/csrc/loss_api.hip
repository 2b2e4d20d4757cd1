// Host engine of the sequence-tiled cross-entropy loss (LM head) behind the C ABI.
//
// The loss is one of the element-wise computations that the talk's memory
// stack tiles along the sequence ("Road to 5 Million Tokens", talk
// transcript, the part after CPU offloading, on Arctic sequence length
// training; liquidgold.cc notes, "Progression of Techniques", item 6): here
// the [N][V] logits never exist. Per tile of rows:
//   forward   one GEMM h_t W^T whose epilogue reduces each 128-column tile of
//             logits to a (max, sum exp) pair per row and picks the target's
//             logit; a small kernel combines the pairs into lse and loss;
//   backward  the same GEMM with an epilogue that writes
//             dz = (softmax - onehot) g for the tile, then dh_t = dz W and
//             dW += dz^T h_t.
#include <math.h>
#include <string.h>

#include "upipe.h"
#include "host.h"
#include "kernels.h"

using namespace upipe;
using namespace upipe::host;

namespace {

constexpr int64_t TILE_ALIGN = 128;

struct LossShape {
  int64_t N, D, V;
  int64_t T;  // rows per tile
  int es;
};

// Forward: part [T][V/128][2] fp32, tgt [T] fp32. Backward: dz [T][V] (io
// dtype) and W^T [D][V].
struct LossPlan {
  size_t part, tgt, dz, w_t, total;
};

int loss_check_shape(int dtype, int64_t N, int64_t D, int64_t V, int64_t tile, LossShape* out) {
  if (dtype != UPIPE_F32 && dtype != UPIPE_BF16) return UPIPE_ERR_INVALID_ARG;
  if (N < 1 || D < 1 || V < 1 || tile < 1) return UPIPE_ERR_INVALID_ARG;
  if (D % 128 || V % 128 || tile % TILE_ALIGN) return UPIPE_ERR_UNSUPPORTED;
  if (N > ((int64_t)1 << 40) || D > ((int64_t)1 << 20) || V > ((int64_t)1 << 24)) return UPIPE_ERR_UNSUPPORTED;
  LossShape s;
  s.N = N;
  s.D = D;
  s.V = V;
  const int64_t whole = round_up(N, TILE_ALIGN);
  s.T = tile < whole ? tile : whole;
  s.es = dtype == UPIPE_BF16 ? 2 : 4;
  *out = s;
  return UPIPE_OK;
}

LossPlan loss_plan(const LossShape& s, bool backward) {
  LossPlan p;
  memset(&p, 0, sizeof(p));
  Carver c;
  if (!backward) {
    p.part = c.take((size_t)s.T * (s.V / 128) * 2 * 4);
    p.tgt = c.take((size_t)s.T * 4);
  } else {
    p.dz = c.take((size_t)s.T * s.V * s.es);
    p.w_t = c.take((size_t)s.V * s.D * s.es);
  }
  p.total = c.off;
  return p;
}

template <typename T>
GemmNT<T> logits_gemm(const LossShape& s, const T* ht, const T* w, int64_t rows) {
  GemmNT<T> g;
  memset(&g, 0, sizeof(g));
  g.a = ht;
  g.lda = s.D;
  g.a_kblk = s.D;
  g.K = s.D;
  g.M = rows;
  g.b[0] = w;
  g.ldb[0] = s.D;
  g.N = s.V;
  g.seg_end[0] = s.V;
  g.nseg = 1;
  return g;
}

template <typename T>
int loss_fwd_impl(const LossShape& s, const T* h, const T* w, const int32_t* targets, float* loss, float* lse,
                  char* ws, hipStream_t st) {
  const LossPlan pl = loss_plan(s, false);
  float* part = reinterpret_cast<float*>(ws + pl.part);
  float* tgt = reinterpret_cast<float*>(ws + pl.tgt);
  for (int64_t t0 = 0; t0 < s.N; t0 += s.T) {
    const int64_t rows = s.N - t0 < s.T ? s.N - t0 : s.T;
    // a target outside [0, V) leaves its logit NaN, and so its loss
    HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(tgt, rows, NAN, st); }));
    GemmNT<T> g = logits_gemm<T>(s, h + t0 * s.D, w, rows);
    g.ce.targets = targets + t0;
    g.ce.part = part;
    g.ce.tgt = tgt;
    HIP_TRY(timed(UPIPE_KERNEL_LOSS_GEMM, 2.0 * rows * s.V * s.D, st,
                  [&] { return launch_gemm_nt<T>(g, EPI_CE, 128, st); }));
    HIP_TRY(timed(UPIPE_KERNEL_LOSS_GEMM, 0.0, st,
                  [&] { return launch_ce_reduce(part, tgt, rows, s.V / 128, lse + t0, loss + t0, st); }));
  }
  return UPIPE_OK;
}

template <typename T>
int loss_bwd_impl(const LossShape& s, const T* h, const T* w, const int32_t* targets, const float* lse,
                  const float* gl, T* dh, float* dw, char* ws, hipStream_t st) {
  const LossPlan pl = loss_plan(s, true);
  T* dz = reinterpret_cast<T*>(ws + pl.dz);
  T* wt = reinterpret_cast<T*>(ws + pl.w_t);
  const int64_t D = s.D, V = s.V;
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(dw, V * D, 0.f, st); }));
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_transpose<T>(w, V, D, D, wt, V, st); }));
  for (int64_t t0 = 0; t0 < s.N; t0 += s.T) {
    const int64_t rows = s.N - t0 < s.T ? s.N - t0 : s.T;
    const T* ht = h + t0 * D;
    // dz = (softmax(h W^T) - onehot) g for the tile
    GemmNT<T> g = logits_gemm<T>(s, ht, w, rows);
    g.ce.targets = targets + t0;
    g.ce.lse = lse + t0;
    g.ce.g = gl + t0;
    g.ce.dz = dz;
    g.ce.ldz = V;
    HIP_TRY(timed(UPIPE_KERNEL_LOSS_GEMM, 2.0 * rows * V * D, st,
                  [&] { return launch_gemm_nt<T>(g, EPI_CE_BWD, 128, st); }));
    // dh_t = dz W
    GemmNT<T> g2;
    memset(&g2, 0, sizeof(g2));
    g2.a = dz;
    g2.lda = V;
    g2.a_kblk = V;
    g2.K = V;
    g2.M = rows;
    g2.b[0] = wt;
    g2.ldb[0] = V;
    g2.N = D;
    g2.seg_end[0] = D;
    g2.nseg = 1;
    g2.c = dh + t0 * D;
    g2.ldc = D;
    HIP_TRY(timed(UPIPE_KERNEL_LOSS_GEMM, 2.0 * rows * D * V, st,
                  [&] { return launch_gemm_nt<T>(g2, EPI_STORE, 128, st); }));
    // dW += dz^T h_t
    GemmTN<T> g3;
    memset(&g3, 0, sizeof(g3));
    g3.a = dz;
    g3.lda = V;
    g3.b = ht;
    g3.b_nblk = D;
    g3.ldb = D;
    g3.M = V;
    g3.N = D;
    g3.K = rows;
    g3.out[0] = dw;
    g3.seg_end[0] = D;
    g3.nseg = 1;
    g3.ldm = D;
    g3.ldn = 1;
    const int64_t tiles = (V / 128) * (D / 128);
    int64_t splits = 1024 / (tiles > 0 ? tiles : 1);
    if (splits < 1) splits = 1;
    g3.ksplit = round_up((rows + splits - 1) / splits, 64);
    HIP_TRY(timed(UPIPE_KERNEL_LOSS_WGRAD, 2.0 * V * D * rows, st, [&] { return launch_gemm_tn<T>(g3, 128, st); }));
  }
  return UPIPE_OK;
}

int loss_check_ptrs(const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (ptrs[i] == nullptr) return UPIPE_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (!aligned(ptrs[i], 16)) return UPIPE_ERR_ALIGNMENT;
  return UPIPE_OK;
}

int loss_check_ws(const LossShape& s, bool bwd, const void* ws, size_t bytes) {
  if (ws == nullptr) return UPIPE_ERR_WORKSPACE;
  if (!aligned(ws, REGION_ALIGN)) return UPIPE_ERR_ALIGNMENT;
  if (bytes < loss_plan(s, bwd).total) return UPIPE_ERR_WORKSPACE;
  return UPIPE_OK;
}

}  // namespace

extern "C" {

size_t upipe_loss_workspace_bytes(int64_t n_tokens, int64_t d_model, int64_t vocab, int64_t tile_tokens,
                                  upipe_dtype_t dtype, int backward) {
  LossShape s;
  if (loss_check_shape(dtype, n_tokens, d_model, vocab, tile_tokens, &s)) return 0;
  return loss_plan(s, backward != 0).total;
}

int upipe_loss_fwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int64_t vocab, int64_t tile_tokens,
                   const void* h, const void* w, const int32_t* targets, float* loss, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  LossShape s;
  int rc = loss_check_shape(dtype, n_tokens, d_model, vocab, tile_tokens, &s);
  if (rc) return rc;
  const void* ptrs[] = {h, w, targets, loss, lse};
  if ((rc = loss_check_ptrs(ptrs, 5))) return rc;
  if ((rc = loss_check_ws(s, false, workspace, workspace_bytes))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16)
    return loss_fwd_impl<bf16>(s, (const bf16*)h, (const bf16*)w, targets, loss, lse, ws, st);
  return loss_fwd_impl<float>(s, (const float*)h, (const float*)w, targets, loss, lse, ws, st);
}

int upipe_loss_bwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int64_t vocab, int64_t tile_tokens,
                   const void* h, const void* w, const int32_t* targets, const float* lse, const float* g,
                   void* dh, float* dw, void* workspace, size_t workspace_bytes, void* stream) {
  LossShape s;
  int rc = loss_check_shape(dtype, n_tokens, d_model, vocab, tile_tokens, &s);
  if (rc) return rc;
  const void* ptrs[] = {h, w, targets, lse, g, dh, dw};
  if ((rc = loss_check_ptrs(ptrs, 7))) return rc;
  if ((rc = loss_check_ws(s, true, workspace, workspace_bytes))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16)
    return loss_bwd_impl<bf16>(s, (const bf16*)h, (const bf16*)w, targets, lse, g, (bf16*)dh, dw, ws, st);
  return loss_bwd_impl<float>(s, (const float*)h, (const float*)w, targets, lse, g, (float*)dh, dw, ws, st);
}

}  // extern "C"
