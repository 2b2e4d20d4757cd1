// Host engine of the sequence-tiled gated-SiLU MLP behind the C ABI.
//
// The element-wise parts of the model are tiled along the sequence so that
// no intermediate is as long as the sequence (Arctic sequence length
// training in "Road to 5 Million Tokens", talk transcript, the part after CPU
// offloading; liquidgold.cc notes, "Progression of Techniques", item 6). For
// the MLP y = (silu(x Wg^T) * (x Wu^T)) Wd^T that means: tile_tokens rows at a
// time, with the [tile][d_ff] intermediates in one workspace that every tile
// reuses. Per tile:
//   forward   a = silu(h) * u from one GEMM whose 128-column tiles hold 64 gate
//             and 64 up features (the epilogue forms a), then y_t = a Wd^T;
//   backward  h|u recomputed the same way, then da = dy_t Wd with an
//             epilogue that forms dh, du and a, the weight-gradient GEMMs
//             (fp32 atomics into dWd, dWg, dWu) and dx_t = [dh du] [Wg; Wu].
#include <string.h>

#include "upipe.h"
#include "host.h"
#include "kernels.h"
#include "mlp.h"

using namespace upipe;
using namespace upipe::host;

namespace upipe {
namespace mlp {

namespace {

constexpr int64_t TILE_ALIGN = 128;  // tile rows are whole GEMM row tiles

template <typename T>
GemmNT<T> nt_base(const T* a, int64_t lda, int64_t K, int64_t M) {
  GemmNT<T> g;
  memset(&g, 0, sizeof(g));
  g.a = a;
  g.lda = lda;
  g.a_kblk = K;
  g.K = K;
  g.M = M;
  g.nseg = 1;
  return g;
}

// out[m * ldm + n] += sum over the tile's rows of rows[t][m] * cols[t][n]
template <typename T>
int wgrad(const T* rows, int64_t ld_rows, int64_t M, const T* cols, int64_t N, int64_t ntok, float* out,
          hipStream_t st) {
  GemmTN<T> g;
  memset(&g, 0, sizeof(g));
  g.a = rows;
  g.lda = ld_rows;
  g.b = cols;
  g.b_nblk = N;
  g.ldb = N;
  g.M = M;
  g.N = N;
  g.K = ntok;
  g.out[0] = out;
  g.seg_end[0] = N;
  g.nseg = 1;
  g.ldm = N;
  g.ldn = 1;
  const int64_t tiles = (M / 128) * (N / 128);
  int64_t splits = 1024 / (tiles > 0 ? tiles : 1);
  if (splits < 1) splits = 1;
  g.ksplit = round_up((ntok + splits - 1) / splits, 64);
  HIP_TRY(timed(UPIPE_KERNEL_MLP_WGRAD, 2.0 * M * N * ntok, st, [&] { return launch_gemm_tn<T>(g, 128, st); }));
  return UPIPE_OK;
}

}  // namespace

int check_shape(int dtype, int64_t N, int64_t D, int64_t F, int64_t tile, Shape* out) {
  if (dtype != UPIPE_F32 && dtype != UPIPE_BF16) return UPIPE_ERR_INVALID_ARG;
  if (N < 1 || D < 1 || F < 1 || tile < 1) return UPIPE_ERR_INVALID_ARG;
  if (D % 128 || F % 128 || tile % TILE_ALIGN) return UPIPE_ERR_UNSUPPORTED;
  if (N > ((int64_t)1 << 40) || D > ((int64_t)1 << 20) || F > ((int64_t)1 << 20)) return UPIPE_ERR_UNSUPPORTED;
  Shape s;
  s.N = N;
  s.D = D;
  s.F = F;
  const int64_t whole = round_up(N, TILE_ALIGN);
  s.T = tile < whole ? tile : whole;
  s.es = dtype == UPIPE_BF16 ? 2 : 4;
  *out = s;
  return UPIPE_OK;
}

Plan plan(const Shape& s, bool backward) {
  Plan p;
  memset(&p, 0, sizeof(p));
  Carver c;
  const size_t tf = (size_t)s.T * s.F * s.es;  // one [T][F] tile buffer
  p.a = c.take(tf);
  if (backward) {
    p.hu = c.take(2 * tf);
    p.dh = c.take(tf);
    p.du = c.take(tf);
    p.wd_t = c.take((size_t)s.F * s.D * s.es);
    p.wgu_t = c.take((size_t)2 * s.F * s.D * s.es);
  }
  p.total = c.off;
  return p;
}

template <typename T>
int fwd_tile(const Shape& s, const T* x, int64_t rows, const T* wg, const T* wu, const T* wd, T* y,
             const T* add, char* ws, hipStream_t st) {
  const Plan pl = plan(s, false);
  T* A = reinterpret_cast<T*>(ws + pl.a);
  // a = silu(x Wg^T) * (x Wu^T)
  GemmNT<T> g1 = nt_base<T>(x, s.D, s.D, rows);
  g1.b[0] = wg;
  g1.b[1] = wu;
  g1.ldb[0] = s.D;
  g1.N = 2 * s.F;
  g1.seg_end[0] = g1.N;
  g1.glu.a = A;
  g1.glu.ldf = s.F;
  HIP_TRY(timed(UPIPE_KERNEL_MLP_GEMM, 2.0 * rows * g1.N * s.D, st,
                [&] { return launch_gemm_nt<T>(g1, EPI_GLU, 128, st); }));
  // y = a Wd^T (+ add)
  GemmNT<T> g2 = nt_base<T>(A, s.F, s.F, rows);
  g2.b[0] = wd;
  g2.ldb[0] = s.F;
  g2.N = s.D;
  g2.seg_end[0] = s.D;
  g2.c = y;
  g2.ldc = s.D;
  g2.add = add;
  g2.ld_add = s.D;
  HIP_TRY(timed(UPIPE_KERNEL_MLP_GEMM, 2.0 * rows * s.D * s.F, st,
                [&] { return launch_gemm_nt<T>(g2, EPI_STORE, 128, st); }));
  return UPIPE_OK;
}

template <typename T>
int bwd_prep(const Shape& s, const T* wg, const T* wu, const T* wd, float* dwg, float* dwu, float* dwd,
             char* ws, hipStream_t st) {
  const Plan pl = plan(s, true);
  T* WdT = reinterpret_cast<T*>(ws + pl.wd_t);
  T* WguT = reinterpret_cast<T*>(ws + pl.wgu_t);
  const int64_t F = s.F, D = s.D;
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(dwg, F * D, 0.f, st); }));
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(dwu, F * D, 0.f, st); }));
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(dwd, F * D, 0.f, st); }));
  // Wd^T [F][D]; [Wg^T | Wu^T] [D][2F]
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_transpose<T>(wd, D, F, F, WdT, D, st); }));
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_transpose<T>(wg, F, D, D, WguT, 2 * F, st); }));
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_transpose<T>(wu, F, D, D, WguT + F, 2 * F, st); }));
  return UPIPE_OK;
}

template <typename T>
int bwd_tile(const Shape& s, const T* xt, const T* dyt, int64_t rows, const T* wg, const T* wu, T* dx,
             float* dwg, float* dwu, float* dwd, char* ws, hipStream_t st) {
  const Plan pl = plan(s, true);
  T* A = reinterpret_cast<T*>(ws + pl.a);
  T* HU = reinterpret_cast<T*>(ws + pl.hu);
  T* DH = reinterpret_cast<T*>(ws + pl.dh);
  T* DU = reinterpret_cast<T*>(ws + pl.du);
  T* WdT = reinterpret_cast<T*>(ws + pl.wd_t);
  T* WguT = reinterpret_cast<T*>(ws + pl.wgu_t);
  const int64_t F = s.F, D = s.D;
  // h|u of the tile, recomputed from x
  GemmNT<T> g1 = nt_base<T>(xt, D, D, rows);
  g1.b[0] = wg;
  g1.b[1] = wu;
  g1.ldb[0] = D;
  g1.N = 2 * F;
  g1.seg_end[0] = g1.N;
  g1.glu.hu = HU;
  g1.glu.ldf = F;
  HIP_TRY(timed(UPIPE_KERNEL_MLP_GEMM, 2.0 * rows * g1.N * D, st,
                [&] { return launch_gemm_nt<T>(g1, EPI_GLU, 128, st); }));
  // da = dy_t Wd, and from it dh, du (and a for dWd)
  GemmNT<T> g2 = nt_base<T>(dyt, D, D, rows);
  g2.b[0] = WdT;
  g2.ldb[0] = D;
  g2.N = F;
  g2.seg_end[0] = F;
  g2.glu.hu = HU;
  g2.glu.a = A;
  g2.glu.dh = DH;
  g2.glu.du = DU;
  g2.glu.ldf = F;
  HIP_TRY(timed(UPIPE_KERNEL_MLP_GEMM, 2.0 * rows * F * D, st,
                [&] { return launch_gemm_nt<T>(g2, EPI_GLU_BWD, 128, st); }));
  // dWd += dy_t^T a, dWg += dh^T x_t, dWu += du^T x_t
  int rc = wgrad<T>(dyt, D, D, A, F, rows, dwd, st);
  if (rc) return rc;
  rc = wgrad<T>(DH, F, F, xt, D, rows, dwg, st);
  if (rc) return rc;
  rc = wgrad<T>(DU, F, F, xt, D, rows, dwu, st);
  if (rc) return rc;
  // dx_t = [dh | du] [Wg; Wu]
  GemmNT<T> g3 = nt_base<T>(DH, F, 2 * F, rows);
  g3.a_kblk = F;
  g3.a_kblk_stride = DU - DH;
  g3.b[0] = WguT;
  g3.ldb[0] = 2 * F;
  g3.N = D;
  g3.seg_end[0] = D;
  g3.c = dx;
  g3.ldc = D;
  HIP_TRY(timed(UPIPE_KERNEL_MLP_GEMM, 2.0 * rows * D * 2 * F, st,
                [&] { return launch_gemm_nt<T>(g3, EPI_STORE, 128, st); }));
  return UPIPE_OK;
}

#define UPIPE_MLP_INST(T)                                                                                     \
  template int fwd_tile<T>(const Shape&, const T*, int64_t, const T*, const T*, const T*, T*, const T*, char*, \
                           hipStream_t);                                                                      \
  template int bwd_prep<T>(const Shape&, const T*, const T*, const T*, float*, float*, float*, char*,          \
                           hipStream_t);                                                                      \
  template int bwd_tile<T>(const Shape&, const T*, const T*, int64_t, const T*, const T*, T*, float*, float*,  \
                           float*, char*, hipStream_t);
UPIPE_MLP_INST(bf16)
UPIPE_MLP_INST(float)
#undef UPIPE_MLP_INST

}  // namespace mlp
}  // namespace upipe

namespace {

using upipe::mlp::Shape;

template <typename T>
int mlp_fwd_impl(const Shape& s, const T* x, const T* wg, const T* wu, const T* wd, T* y, char* ws,
                 hipStream_t st) {
  for (int64_t t0 = 0; t0 < s.N; t0 += s.T) {
    const int64_t rows = s.N - t0 < s.T ? s.N - t0 : s.T;
    const int rc = upipe::mlp::fwd_tile<T>(s, x + t0 * s.D, rows, wg, wu, wd, y + t0 * s.D, nullptr, ws, st);
    if (rc) return rc;
  }
  return UPIPE_OK;
}

template <typename T>
int mlp_bwd_impl(const Shape& s, const T* x, const T* wg, const T* wu, const T* wd, const T* dy, T* dx,
                 float* dwg, float* dwu, float* dwd, char* ws, hipStream_t st) {
  int rc = upipe::mlp::bwd_prep<T>(s, wg, wu, wd, dwg, dwu, dwd, ws, st);
  if (rc) return rc;
  for (int64_t t0 = 0; t0 < s.N; t0 += s.T) {
    const int64_t rows = s.N - t0 < s.T ? s.N - t0 : s.T;
    rc = upipe::mlp::bwd_tile<T>(s, x + t0 * s.D, dy + t0 * s.D, rows, wg, wu, dx + t0 * s.D, dwg, dwu, dwd,
                                 ws, st);
    if (rc) return rc;
  }
  return UPIPE_OK;
}

int mlp_check_ptrs(const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (ptrs[i] == nullptr) return UPIPE_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (!aligned(ptrs[i], 16)) return UPIPE_ERR_ALIGNMENT;
  return UPIPE_OK;
}

int mlp_check_ws(const Shape& s, bool bwd, const void* ws, size_t bytes) {
  if (ws == nullptr) return UPIPE_ERR_WORKSPACE;
  if (!aligned(ws, REGION_ALIGN)) return UPIPE_ERR_ALIGNMENT;
  if (bytes < upipe::mlp::plan(s, bwd).total) return UPIPE_ERR_WORKSPACE;
  return UPIPE_OK;
}

}  // namespace

extern "C" {

size_t upipe_mlp_workspace_bytes(int64_t n_tokens, int64_t d_model, int64_t d_ff, int64_t tile_tokens,
                                 upipe_dtype_t dtype, int backward) {
  Shape s;
  if (upipe::mlp::check_shape(dtype, n_tokens, d_model, d_ff, tile_tokens, &s)) return 0;
  return upipe::mlp::plan(s, backward != 0).total;
}

int upipe_mlp_fwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int64_t d_ff, int64_t tile_tokens,
                  const void* x, const void* w_gate, const void* w_up, const void* w_down, void* y,
                  void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = upipe::mlp::check_shape(dtype, n_tokens, d_model, d_ff, tile_tokens, &s);
  if (rc) return rc;
  const void* ptrs[] = {x, w_gate, w_up, w_down, y};
  if ((rc = mlp_check_ptrs(ptrs, 5))) return rc;
  if ((rc = mlp_check_ws(s, false, workspace, workspace_bytes))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16)
    return mlp_fwd_impl<bf16>(s, (const bf16*)x, (const bf16*)w_gate, (const bf16*)w_up, (const bf16*)w_down,
                              (bf16*)y, ws, st);
  return mlp_fwd_impl<float>(s, (const float*)x, (const float*)w_gate, (const float*)w_up, (const float*)w_down,
                             (float*)y, ws, st);
}

int upipe_mlp_bwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int64_t d_ff, int64_t tile_tokens,
                  const void* x, const void* w_gate, const void* w_up, const void* w_down, const void* dy,
                  void* dx, float* dw_gate, float* dw_up, float* dw_down, void* workspace,
                  size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = upipe::mlp::check_shape(dtype, n_tokens, d_model, d_ff, tile_tokens, &s);
  if (rc) return rc;
  const void* ptrs[] = {x, w_gate, w_up, w_down, dy, dx, dw_gate, dw_up, dw_down};
  if ((rc = mlp_check_ptrs(ptrs, 9))) return rc;
  if ((rc = mlp_check_ws(s, true, workspace, workspace_bytes))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16)
    return mlp_bwd_impl<bf16>(s, (const bf16*)x, (const bf16*)w_gate, (const bf16*)w_up, (const bf16*)w_down,
                              (const bf16*)dy, (bf16*)dx, dw_gate, dw_up, dw_down, ws, st);
  return mlp_bwd_impl<float>(s, (const float*)x, (const float*)w_gate, (const float*)w_up, (const float*)w_down,
                             (const float*)dy, (float*)dx, dw_gate, dw_up, dw_down, ws, st);
}

}  // extern "C"
