// Host engine behind the C ABI: argument validation, the workspace plan and
// the chunk loop that enqueues the gfx950 kernels.
//
// The chunk loop is the method itself: the heads one GPU owns are split into
// chunks of `chunk_heads` query heads that run one after another; each chunk
// recomputes its Q (and, at the first chunk of a kv group, that group's K and
// V), runs attention over the full sequence, stores its partial result into
// y, and the next chunk reuses the same buffers ("500 万トークンへの道 — Max
// Ryabinin (Together AI) の Untied Ulysses", section "Untied Ulysses (UPipe) —
// head 単位のチャンク化"; "Road to 5 Million Tokens", section "Primary
// Contribution"). Only per-chunk buffers live in the workspace, so its size
// grows with chunk_heads and not with the number of heads.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "upipe.h"
#include "host.h"
#include "kernels.h"

using namespace upipe;
using namespace upipe::host;

namespace upipe {
namespace host {
Profiler g_prof;
}  // namespace host
}  // namespace upipe

namespace {

// Scratch of upipe_attn_fwd_noalloc. In host code `scratch` names a host-side
// stand-in, not device memory: kernels and copies get the per-device address
// that noalloc_scratch() looks up once per device.
__device__ __align__(256) char scratch[UPIPE_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// This device's address of `scratch` (looked up on the first call with the
// device current), or null when the lookup fails.
void* noalloc_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

constexpr int64_t ROW_PAD = 256;   // token rows of per-head buffers are padded to this

struct Shape {
  int64_t N, D, Np;
  int Hq, Hkv, d, C, G, kvC;
  bool norm;
  int es;  // element size of the io dtype
};

// Workspace regions (byte offsets). Forward uses q, k|v, o.
// Backward aliases: the dq of a chunk overwrites q, dk|dv overwrite k|v.
struct Plan {
  size_t q, uq, k, v, uk, dout, o, delta, dq_acc, dk_acc, dv_acc, wo_t, wqkv_t;
  size_t total;
};

Plan make_plan(const Shape& s, bool backward) {
  Plan p;
  memset(&p, 0, sizeof(p));
  const size_t head = (size_t)s.Np * s.d;  // elements of one [Np][d] head buffer
  Carver c;
  // Q, then K, then V: contiguous heads of stride Np*d (the backward's dx
  // product reads dq|dk|dv, which alias them, as one operand)
  p.q = c.take(head * s.C * s.es);
  p.k = c.take(head * 2 * s.kvC * s.es);  // K then V (backward: dk|dv alias them)
  p.v = p.k + head * s.kvC * s.es;
  if (!backward) {
    p.o = c.take(head * s.C * s.es);
    p.total = c.off;
    return p;
  }
  if (s.norm) p.uq = c.take(head * s.C * s.es);
  if (s.norm) p.uk = c.take(head * s.kvC * s.es);
  p.dout = c.take(head * s.C * s.es);
  p.o = c.take(head * s.C * s.es);
  p.delta = c.take((size_t)s.Np * s.C * 4);
  p.dq_acc = c.take(head * s.C * 4);
  p.dk_acc = c.take(head * s.kvC * 4);
  p.dv_acc = c.take(head * s.kvC * 4);
  p.wo_t = c.take((size_t)s.C * s.d * s.D * s.es);
  // [D][C*d + 2*kvC*d]: Wq_c^T columns, then Wk_g^T, then Wv_g^T
  p.wqkv_t = c.take((size_t)(s.C + 2 * s.kvC) * s.d * s.D * s.es);
  p.total = c.off;
  return p;
}

int check_shape(int dtype, int64_t N, int64_t D, int Hq, int Hkv, int d, int C, Shape* out) {
  if (dtype != UPIPE_F32 && dtype != UPIPE_BF16) return UPIPE_ERR_INVALID_ARG;
  if (N < 1 || D < 1 || Hq < 1 || Hkv < 1 || C < 1 || d < 1) return UPIPE_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return UPIPE_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return UPIPE_ERR_UNSUPPORTED;
  if (D % 128 != 0) return UPIPE_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (Hq % C != 0) return UPIPE_ERR_UNSUPPORTED;
  if (C % G != 0 && G % C != 0) return UPIPE_ERR_UNSUPPORTED;
  if (N > ((int64_t)1 << 40) || D > ((int64_t)1 << 20)) return UPIPE_ERR_UNSUPPORTED;
  Shape s;
  s.N = N;
  s.D = D;
  s.Np = round_up(N, ROW_PAD);
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.d = d;
  s.C = C;
  s.G = G;
  s.kvC = C > G ? C / G : 1;
  s.norm = false;
  s.es = dtype == UPIPE_BF16 ? 2 : 4;
  *out = s;
  return UPIPE_OK;
}

// Visible (query, key) pairs of causal attention over N tokens.
double causal_pairs(int64_t N) { return 0.5 * (double)N * (double)(N + 1); }

template <typename T>
GemmNT<T> gemm_base() {
  GemmNT<T> g;
  memset(&g, 0, sizeof(g));
  g.nseg = 1;
  return g;
}

// Projection of rows x[N][D] onto the heads described by up to 3 segments.
template <typename T>
int run_projection(const Shape& s, const T* x, int nseg, const T* const* w, const int* nheads,
                   const HeadOut<T>* ho, float eps, double log2_theta, hipStream_t st) {
  GemmNT<T> g = gemm_base<T>();
  g.a = x;
  g.lda = s.D;
  g.a_kblk = s.D;
  g.a_kblk_stride = 0;
  int64_t n = 0;
  for (int i = 0; i < nseg; ++i) {
    g.b[i] = w[i];
    g.ldb[i] = s.D;
    n += (int64_t)nheads[i] * s.d;
    g.seg_end[i] = n;
    g.ho[i] = ho[i];
  }
  g.nseg = nseg;
  g.M = s.N;
  g.N = n;
  g.K = s.D;
  g.Np = s.Np;
  g.eps = eps;
  g.log2_theta = log2_theta;
  HIP_TRY(timed(UPIPE_KERNEL_PROJECTION, 2.0 * g.M * g.N * g.K, st,
                [&] { return launch_gemm_nt<T>(g, EPI_HEADS, s.d, st); }));
  return UPIPE_OK;
}

// out[N][D] (+)= A_heads[nheads][Np][d] (as [N][nheads*d]) x B^T, B(n,k) = b + n*ldb + k
template <typename T>
int run_heads_times_wt(const Shape& s, const T* a_heads, int nheads, const T* b, int64_t ldb, T* out,
                       int accumulate, hipStream_t st) {
  GemmNT<T> g = gemm_base<T>();
  g.a = a_heads;
  g.lda = s.d;
  g.a_kblk = s.d;
  g.a_kblk_stride = s.Np * s.d;
  g.b[0] = b;
  g.ldb[0] = ldb;
  g.seg_end[0] = s.D;
  g.M = s.N;
  g.N = s.D;
  g.K = (int64_t)nheads * s.d;
  g.c = out;
  g.ldc = s.D;
  g.accumulate = accumulate;
  HIP_TRY(timed(UPIPE_KERNEL_OUT_GEMM, 2.0 * g.M * g.N * g.K, st,
                [&] { return launch_gemm_nt<T>(g, EPI_ACCUM, 128, st); }));
  return UPIPE_OK;
}

// Weight gradient out[m*ldm + n*ldn] += sum_tok rows[tok][m] * heads[n/d][tok][n%d],
// with the heads split into up to 3 segments of seg_heads[i] heads, each with
// its own output. The token sum is split over workgroups; with part == null
// the splits are added with fp32 atomics, else (deterministic) they go to
// part (part_bytes of free workspace) and are added in split order, with as
// many splits as part holds.
template <typename T>
int run_weight_grad_segs(const Shape& s, const T* rows, const T* heads, int nseg, const int* seg_heads,
                         float* const* outs, int64_t ldm, int64_t ldn, hipStream_t st, float* part = nullptr,
                         size_t part_bytes = 0) {
  GemmTN<T> g;
  memset(&g, 0, sizeof(g));
  g.a = rows;
  g.lda = s.D;
  g.b = heads;
  g.b_nblk = s.d;
  g.b_nblk_stride = s.Np * s.d;
  g.ldb = s.d;
  g.M = s.D;
  int64_t n = 0;
  bool all128 = true;
  for (int i = 0; i < nseg; ++i) {
    n += (int64_t)seg_heads[i] * s.d;
    g.seg_end[i] = n;
    g.out[i] = outs[i];
    all128 = all128 && ((int64_t)seg_heads[i] * s.d) % 128 == 0;
  }
  g.nseg = nseg;
  g.N = n;
  g.K = s.N;
  const int bn = all128 ? 128 : 64;  // n tiles never straddle two segments
  const int64_t tiles = (g.M / 128) * (g.N / bn);
  int64_t splits = 1024 / (tiles > 0 ? tiles : 1);
  if (part) {
    const int64_t fit = (int64_t)(part_bytes / ((size_t)g.M * g.N * 4));
    if (splits > fit) splits = fit;
    g.part = part;
  }
  if (splits < 1) splits = 1;
  g.ksplit = round_up((s.N + splits - 1) / splits, 64);
  g.ldm = ldm;
  g.ldn = ldn;
  HIP_TRY(timed(UPIPE_KERNEL_WGRAD, 2.0 * g.M * g.N * g.K, st, [&] { return launch_gemm_tn<T>(g, bn, st); }));
  return UPIPE_OK;
}

template <typename T>
int run_weight_grad(const Shape& s, const T* rows, const T* heads, int nheads, float* out, int64_t ldm,
                    int64_t ldn, hipStream_t st, float* part = nullptr, size_t part_bytes = 0) {
  return run_weight_grad_segs<T>(s, rows, heads, 1, &nheads, &out, ldm, ldn, st, part, part_bytes);
}

template <typename T>
int attn_fwd_impl(const Shape& s, double theta, const T* x, const T* wq, const T* wk, const T* wv,
                  const T* wo, const T* qn, const T* kn, float eps, T* y, float* lse, char* ws,
                  hipStream_t st, T* o_keep = nullptr) {
  const Plan pl = make_plan(s, false);
  T* Q = reinterpret_cast<T*>(ws + pl.q);
  T* K = reinterpret_cast<T*>(ws + pl.k);
  T* V = reinterpret_cast<T*>(ws + pl.v);
  T* Ows = reinterpret_cast<T*>(ws + pl.o);
  const double l2t = log2(theta);
  const int64_t head = s.Np * s.d;
  const int nh = s.C < s.G ? s.C : s.G;  // q heads of the chunk per kv head
  const float q_scale = (float)(1.4426950408889634 / sqrt((double)s.d));
  for (int c0 = 0; c0 < s.Hq; c0 += s.C) {
    const int g0 = c0 / s.G;
    const bool new_kv = (c0 % s.G) == 0;
    // the chunk's O: the reused workspace buffer, or its heads of the kept O
    T* O = o_keep ? o_keep + (int64_t)c0 * head : Ows;
    const T* w[3] = {wq + (int64_t)c0 * s.d * s.D, wk + (int64_t)g0 * s.d * s.D, wv + (int64_t)g0 * s.d * s.D};
    const int nheads[3] = {s.C, s.kvC, s.kvC};
    HeadOut<T> ho[3];
    memset(ho, 0, sizeof(ho));
    ho[0].rm = Q;
    ho[0].gamma = qn;
    ho[0].rope = 1;
    ho[0].scale = q_scale;  // Q K^T is then the softmax exponent in log2 units
    ho[1].rm = K;
    ho[1].gamma = kn;
    ho[1].rope = 1;
    ho[1].scale = 1.f;
    ho[2].rm = V;
    ho[2].scale = 1.f;
    int rc = run_projection<T>(s, x, new_kv ? 3 : 1, w, nheads, ho, eps, l2t, st);
    if (rc) return rc;
    for (int j = 0; j < s.kvC; ++j) {
      AttnFwd<T> a;
      memset(&a, 0, sizeof(a));
      a.q = Q + (int64_t)j * nh * head;
      a.k = K + (int64_t)j * head;
      a.v = V + (int64_t)j * head;
      a.o = O + (int64_t)j * nh * head;
      a.lse = lse + (int64_t)(c0 + j * nh) * s.N;
      a.lse_stride = s.N;
      a.N = s.N;
      a.Np = s.Np;
      a.nh = nh;
      HIP_TRY(timed(UPIPE_KERNEL_ATTN_FWD, 4.0 * s.d * nh * causal_pairs(s.N), st,
                    [&] { return launch_attn_fwd<T>(a, s.d, 0, st); }));
    }
    rc = run_heads_times_wt<T>(s, O, s.C, wo + (int64_t)c0 * s.d, (int64_t)s.Hq * s.d, y, c0 > 0, st);
    if (rc) return rc;
  }
  return UPIPE_OK;
}

template <typename T>
int attn_bwd_impl(const Shape& s, double theta, const T* x, const T* wq, const T* wk, const T* wv,
                  const T* wo, const T* qn, const T* kn, float eps, const T* dy, const float* lse,
                  T* dx, float* dwq, float* dwk, float* dwv, float* dwo, float* dqn, float* dkn,
                  char* ws, hipStream_t st, const T* o_kept = nullptr, bool det = false) {
  const Plan pl = make_plan(s, true);
  T* Q = reinterpret_cast<T*>(ws + pl.q);
  T* Uq = s.norm ? reinterpret_cast<T*>(ws + pl.uq) : nullptr;
  T* K = reinterpret_cast<T*>(ws + pl.k);
  T* V = reinterpret_cast<T*>(ws + pl.v);
  T* Uk = s.norm ? reinterpret_cast<T*>(ws + pl.uk) : nullptr;
  T* dO = reinterpret_cast<T*>(ws + pl.dout);
  T* Ows = reinterpret_cast<T*>(ws + pl.o);
  float* Delta = reinterpret_cast<float*>(ws + pl.delta);
  float* dQa = reinterpret_cast<float*>(ws + pl.dq_acc);
  float* dKa = reinterpret_cast<float*>(ws + pl.dk_acc);
  float* dVa = reinterpret_cast<float*>(ws + pl.dv_acc);
  T* WoT = reinterpret_cast<T*>(ws + pl.wo_t);
  // one row of WqkvT is [Wq_c^T | Wk_g^T | Wv_g^T]; Q, K, V heads are contiguous
  // in the workspace in the same order, so dx takes all three in one product
  T* WqkvT = reinterpret_cast<T*>(ws + pl.wqkv_t);
  const double l2t = log2(theta);
  const int64_t head = s.Np * s.d;
  const int64_t Cd = (int64_t)s.C * s.d, kvd = (int64_t)s.kvC * s.d;
  const int64_t ldw = Cd + 2 * kvd;  // row stride of WqkvT
  const int nh = s.C < s.G ? s.C : s.G;
  // q is stored times log2(e)/sqrt(d) and dO times 1/sqrt(d) (see kernels.h);
  // the dK/dV kernel undoes those factors on its results
  const float q_scale = (float)(1.4426950408889634 / sqrt((double)s.d));
  const float do_scale = (float)(1.0 / sqrt((double)s.d));
  const float dk_mul = (float)(sqrt((double)s.d) * 0.6931471805599453);
  const float dv_mul = (float)sqrt((double)s.d);
  // Free workspace borrowed by the fixed-order reductions. The dq accumulator
  // is free while the weight gradients run (dWo before the dQ kernel fills
  // it, the others after the dq finish has consumed it): deterministic mode
  // keeps the split-K partial tiles there. dO and O are free once the
  // attention backward of the chunk is done: the dgamma partials of the
  // RMSNorm backward go there.
  float* part = det ? dQa : nullptr;
  const size_t part_bytes = det ? (size_t)head * s.C * 4 : 0;
  float* dg_part = reinterpret_cast<float*>(ws + pl.dout);
  const int64_t dg_waves = (int64_t)((pl.o + (size_t)head * s.C * s.es - pl.dout) / ((size_t)s.d * 4));

  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(dwq, (int64_t)s.Hq * s.d * s.D, 0.f, st); }));
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(dwk, (int64_t)s.Hkv * s.d * s.D, 0.f, st); }));
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(dwv, (int64_t)s.Hkv * s.d * s.D, 0.f, st); }));
  HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(dwo, (int64_t)s.Hq * s.d * s.D, 0.f, st); }));
  if (s.norm) {
    HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(dqn, s.d, 0.f, st); }));
    HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_fill_f32(dkn, s.d, 0.f, st); }));
  }

  for (int c0 = 0; c0 < s.Hq; c0 += s.C) {
    const int g0 = c0 / s.G;
    const bool new_kv = (c0 % s.G) == 0;
    const bool last_kv = ((c0 + s.C) % s.G) == 0;
    // weight slices transposed for the products that contract over their rows
    HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_transpose<T>(wo + (int64_t)c0 * s.d, s.D, Cd, (int64_t)s.Hq * s.d, WoT, s.D, st); }));
    HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_transpose<T>(wq + (int64_t)c0 * s.d * s.D, Cd, s.D, s.D, WqkvT, ldw, st); }));
    if (new_kv) {
      HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_transpose<T>(wk + (int64_t)g0 * s.d * s.D, kvd, s.D, s.D, WqkvT + Cd, ldw, st); }));
      HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_transpose<T>(wv + (int64_t)g0 * s.d * s.D, kvd, s.D, s.D, WqkvT + Cd + kvd, ldw, st); }));
    }
    // recompute the chunk's projections
    {
      const T* w[3] = {wq + (int64_t)c0 * s.d * s.D, wk + (int64_t)g0 * s.d * s.D, wv + (int64_t)g0 * s.d * s.D};
      const int nheads[3] = {s.C, s.kvC, s.kvC};
      HeadOut<T> ho[3];
      memset(ho, 0, sizeof(ho));
      ho[0].rm = Q;
      ho[0].pre = Uq;
      ho[0].gamma = qn;
      ho[0].rope = 1;
      ho[0].scale = q_scale;
      ho[1].rm = K;
      ho[1].pre = Uk;
      ho[1].gamma = kn;
      ho[1].rope = 1;
      ho[1].scale = 1.f;
      ho[2].rm = V;
      ho[2].scale = 1.f;
      int rc = run_projection<T>(s, x, new_kv ? 3 : 1, w, nheads, ho, eps, l2t, st);
      if (rc) return rc;
    }
    // dO_c = dY Wo_c  (as dY (Wo_c^T)^T)
    {
      const T* w[1] = {WoT};
      const int nheads[1] = {s.C};
      HeadOut<T> ho[1];
      memset(ho, 0, sizeof(ho));
      ho[0].rm = dO;
      ho[0].scale = do_scale;
      int rc = run_projection<T>(s, dy, 1, w, nheads, ho, eps, l2t, st);
      if (rc) return rc;
    }
    // recompute O_c from the saved LSE, and Delta = rowsum(dO o O); with O
    // kept by the forward, only Delta
    const T* O = o_kept ? o_kept + (int64_t)c0 * head : Ows;
    if (o_kept)
      HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st,
                    [&] { return launch_row_dot<T>(dO, O, (int64_t)s.C * s.Np, s.d, Delta, st); }));
    for (int j = 0; j < s.kvC && !o_kept; ++j) {
      AttnFwd<T> a;
      memset(&a, 0, sizeof(a));
      a.q = Q + (int64_t)j * nh * head;
      a.k = K + (int64_t)j * head;
      a.v = V + (int64_t)j * head;
      a.o = Ows + (int64_t)j * nh * head;
      a.lse = const_cast<float*>(lse) + (int64_t)(c0 + j * nh) * s.N;
      a.lse_stride = s.N;
      a.dout = dO + (int64_t)j * nh * head;
      a.delta = Delta + (int64_t)j * nh * s.Np;
      a.N = s.N;
      a.Np = s.Np;
      a.nh = nh;
      HIP_TRY(timed(UPIPE_KERNEL_ATTN_RECOMPUTE, 4.0 * s.d * nh * causal_pairs(s.N), st,
                    [&] { return launch_attn_fwd<T>(a, s.d, 1, st); }));
    }
    // dWo[:, chunk] = dY^T O_c
    int rc = run_weight_grad<T>(s, dy, O, s.C, dwo + (int64_t)c0 * s.d, (int64_t)s.Hq * s.d, 1, st, part, part_bytes);
    if (rc) return rc;
    // attention backward: dK/dV (key-stationary) and dQ (query-stationary)
    for (int j = 0; j < s.kvC; ++j) {
      AttnBwd<T> b;
      memset(&b, 0, sizeof(b));
      b.q = Q + (int64_t)j * nh * head;
      b.k = K + (int64_t)j * head;
      b.v = V + (int64_t)j * head;
      b.dout = dO + (int64_t)j * nh * head;
      b.lse = lse + (int64_t)(c0 + j * nh) * s.N;
      b.lse_stride = s.N;
      b.delta = Delta + (int64_t)j * nh * s.Np;
      b.dq = dQa + (int64_t)j * nh * head;
      b.dk_acc = dKa + (int64_t)j * head;
      b.dv_acc = dVa + (int64_t)j * head;
      b.N = s.N;
      b.Np = s.Np;
      b.nh = nh;
      b.accumulate = new_kv ? 0 : 1;
      b.dk_mul = dk_mul;
      b.dv_mul = dv_mul;
      b.no_head_split = det ? 1 : 0;
      HIP_TRY(timed(UPIPE_KERNEL_ATTN_BWD_DKDV, 8.0 * s.d * nh * causal_pairs(s.N), st,
                    [&] { return launch_attn_bwd_dkdv<T>(b, s.d, st); }));
      HIP_TRY(timed(UPIPE_KERNEL_ATTN_BWD_DQ, 6.0 * s.d * nh * causal_pairs(s.N), st,
                    [&] { return launch_attn_bwd_dq<T>(b, s.d, st); }));
    }
    // dq: RoPE transpose (+ RMSNorm backward), into the Q buffer
    {
      GradFinish<T> f;
      memset(&f, 0, sizeof(f));
      f.gacc = dQa;
      f.u = Uq;
      f.gamma = qn;
      f.dgamma = dqn;
      f.out = Q;
      f.rope = 1;
      f.nh = s.C;
      f.N = s.N;
      f.Np = s.Np;
      f.eps = eps;
      f.log2_theta = l2t;
      f.dg_part = dg_part;
      f.dg_waves = dg_waves;
      HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_grad_finish<T>(f, s.d, st); }));
    }
    const bool group_done = last_kv || s.C >= s.G;  // dk/dv of the kv group are complete
    if (!group_done) {
      rc = run_weight_grad<T>(s, x, Q, s.C, dwq + (int64_t)c0 * s.d * s.D, 1, s.D, st, part, part_bytes);
      if (rc) return rc;
      rc = run_heads_times_wt<T>(s, Q, s.C, WqkvT, ldw, dx, c0 > 0, st);
      if (rc) return rc;
    } else {
      GradFinish<T> f;
      memset(&f, 0, sizeof(f));
      f.gacc = dKa;
      f.u = Uk;
      f.gamma = kn;
      f.dgamma = dkn;
      f.out = K;
      f.rope = 1;
      f.nh = s.kvC;
      f.N = s.N;
      f.Np = s.Np;
      f.eps = eps;
      f.log2_theta = l2t;
      f.dg_part = dg_part;
      f.dg_waves = dg_waves;
      HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_grad_finish<T>(f, s.d, st); }));
      GradFinish<T> fv;
      memset(&fv, 0, sizeof(fv));
      fv.gacc = dVa;
      fv.out = V;
      fv.nh = s.kvC;
      fv.N = s.N;
      fv.Np = s.Np;
      HIP_TRY(timed(UPIPE_KERNEL_OTHER, 0.0, st, [&] { return launch_grad_finish<T>(fv, s.d, st); }));
      // dWq_c, dWk_g, dWv_g from one pass over x: [dq_c | dk_g | dv_g] are contiguous heads
      {
        const int seg_heads[3] = {s.C, s.kvC, s.kvC};
        float* const outs[3] = {dwq + (int64_t)c0 * s.d * s.D, dwk + (int64_t)g0 * s.d * s.D,
                                dwv + (int64_t)g0 * s.d * s.D};
        rc = run_weight_grad_segs<T>(s, x, Q, 3, seg_heads, outs, 1, s.D, st, part, part_bytes);
        if (rc) return rc;
      }
      // dx (+)= [dq_c | dk_g | dv_g] [Wq_c; Wk_g; Wv_g] in one pass over dx
      rc = run_heads_times_wt<T>(s, Q, s.C + 2 * s.kvC, WqkvT, ldw, dx, c0 > 0, st);
      if (rc) return rc;
    }
  }
  return UPIPE_OK;
}

int check_common(int dtype, int64_t N, int64_t D, int Hq, int Hkv, int d, double theta, int C,
                 const void* qn, const void* kn, float eps, Shape* s) {
  int rc = check_shape(dtype, N, D, Hq, Hkv, d, C, s);
  if (rc) return rc;
  if (!(theta > 0.0) || !isfinite(theta)) return UPIPE_ERR_INVALID_ARG;
  if ((qn == nullptr) != (kn == nullptr)) return UPIPE_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return UPIPE_ERR_INVALID_ARG;
  s->norm = qn != nullptr;
  return UPIPE_OK;
}

int check_ptrs(const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (ptrs[i] == nullptr) return UPIPE_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (!aligned(ptrs[i], 16)) return UPIPE_ERR_ALIGNMENT;
  return UPIPE_OK;
}

int check_ws(const Shape& s, bool bwd, const void* ws, size_t bytes) {
  if (ws == nullptr) return UPIPE_ERR_WORKSPACE;
  if (!aligned(ws, REGION_ALIGN)) return UPIPE_ERR_ALIGNMENT;
  if (bytes < make_plan(s, bwd).total) return UPIPE_ERR_WORKSPACE;
  return UPIPE_OK;
}

}  // namespace

namespace upipe {
int64_t attn_padded_rows(int64_t N) { return round_up(N, ROW_PAD); }

template <typename T>
int attn_fwd_keep_o(const AttnCall& c, const void* x, const void* wq, const void* wk, const void* wv, const void* wo,
                    const void* qn, const void* kn, void* y, float* lse, T* o_keep, void* ws, size_t bytes,
                    hipStream_t st) {
  Shape s;
  int rc = check_common(c.dtype, c.N, c.D, c.Hq, c.Hkv, c.d, c.theta, c.C, qn, kn, c.eps, &s);
  if (rc) return rc;
  const void* ptrs[] = {x, wq, wk, wv, wo, y, lse, o_keep};
  if ((rc = check_ptrs(ptrs, 8))) return rc;
  if ((rc = check_ws(s, false, ws, bytes))) return rc;
  return attn_fwd_impl<T>(s, c.theta, (const T*)x, (const T*)wq, (const T*)wk, (const T*)wv, (const T*)wo,
                          (const T*)qn, (const T*)kn, c.eps, (T*)y, lse, (char*)ws, st, o_keep);
}

template <typename T>
int attn_bwd_kept_o(const AttnCall& c, const void* x, const void* wq, const void* wk, const void* wv, const void* wo,
                    const void* qn, const void* kn, const void* dy, const float* lse, const T* o_kept, void* dx,
                    float* dwq, float* dwk, float* dwv, float* dwo, float* dqn, float* dkn, void* ws, size_t bytes,
                    hipStream_t st) {
  Shape s;
  int rc = check_common(c.dtype, c.N, c.D, c.Hq, c.Hkv, c.d, c.theta, c.C, qn, kn, c.eps, &s);
  if (rc) return rc;
  const void* ptrs[] = {x, wq, wk, wv, wo, dy, lse, o_kept, dx, dwq, dwk, dwv, dwo};
  if ((rc = check_ptrs(ptrs, 13))) return rc;
  if (s.norm) {
    const void* np[] = {dqn, dkn};
    if ((rc = check_ptrs(np, 2))) return rc;
  }
  if ((rc = check_ws(s, true, ws, bytes))) return rc;
  return attn_bwd_impl<T>(s, c.theta, (const T*)x, (const T*)wq, (const T*)wk, (const T*)wv, (const T*)wo,
                          (const T*)qn, (const T*)kn, c.eps, (const T*)dy, lse, (T*)dx, dwq, dwk, dwv, dwo, dqn, dkn,
                          (char*)ws, st, o_kept);
}

template int attn_fwd_keep_o<bf16>(const AttnCall&, const void*, const void*, const void*, const void*,
                                   const void*, const void*, const void*, void*, float*, bf16*, void*, size_t,
                                   hipStream_t);
template int attn_fwd_keep_o<float>(const AttnCall&, const void*, const void*, const void*, const void*,
                                    const void*, const void*, const void*, void*, float*, float*, void*, size_t,
                                    hipStream_t);
template int attn_bwd_kept_o<bf16>(const AttnCall&, const void*, const void*, const void*, const void*,
                                   const void*, const void*, const void*, const void*, const float*, const bf16*,
                                   void*, float*, float*, float*, float*, float*, float*, void*, size_t, hipStream_t);
template int attn_bwd_kept_o<float>(const AttnCall&, const void*, const void*, const void*, const void*,
                                    const void*, const void*, const void*, const void*, const float*, const float*,
                                    void*, float*, float*, float*, float*, float*, float*, void*, size_t,
                                    hipStream_t);

int attn_check_args(int dtype, int64_t N, int64_t D, int Hq, int Hkv, int d, double theta, int C, float eps) {
  Shape s;
  const int rc = check_shape(dtype, N, D, Hq, Hkv, d, C, &s);
  if (rc) return rc;
  if (!(theta > 0.0) || !isfinite(theta)) return UPIPE_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return UPIPE_ERR_INVALID_ARG;
  return UPIPE_OK;
}
}  // namespace upipe

extern "C" {

size_t upipe_attn_workspace_bytes(int64_t n_tokens, int64_t d_model, int n_q_heads, int n_kv_heads,
                                  int head_dim, int chunk_heads, int qk_norm, upipe_dtype_t dtype,
                                  int backward) {
  Shape s;
  if (check_shape(dtype, n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, chunk_heads, &s)) return 0;
  s.norm = qk_norm != 0;
  return make_plan(s, backward != 0).total;
}

int upipe_choose_chunk_heads(int64_t n_tokens, int64_t d_model, int n_q_heads, int n_kv_heads, int head_dim,
                             int qk_norm, upipe_dtype_t dtype, int backward, size_t budget_bytes,
                             size_t* ws_bytes) {
  Shape s;
  // chunk_heads = 1 is a valid chunking for every accepted shape, so this
  // reports exactly the shape errors the entry points would
  const int rc = check_shape(dtype, n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, 1, &s);
  if (rc) return rc;
  for (int c = n_q_heads; c >= 1; --c) {
    if (check_shape(dtype, n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, c, &s)) continue;
    s.norm = qk_norm != 0;
    const size_t need = make_plan(s, backward != 0).total;
    if (need <= budget_bytes) {
      if (ws_bytes) *ws_bytes = need;
      return c;
    }
  }
  return UPIPE_ERR_WORKSPACE;
}

int upipe_attn_fwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int n_q_heads, int n_kv_heads,
                   int head_dim, double rope_theta, int chunk_heads, const void* x, const void* wq,
                   const void* wk, const void* wv, const void* wo, const void* q_norm_w,
                   const void* k_norm_w, float norm_eps, void* y, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  Shape s;
  int rc = check_common(dtype, n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads,
                        q_norm_w, k_norm_w, norm_eps, &s);
  if (rc) return rc;
  const void* ptrs[] = {x, wq, wk, wv, wo, y, lse};
  if ((rc = check_ptrs(ptrs, 7))) return rc;
  if (s.norm) {
    const void* np[] = {q_norm_w, k_norm_w};
    if ((rc = check_ptrs(np, 2))) return rc;
  }
  if ((rc = check_ws(s, false, workspace, workspace_bytes))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16)
    return attn_fwd_impl<bf16>(s, rope_theta, (const bf16*)x, (const bf16*)wq, (const bf16*)wk,
                               (const bf16*)wv, (const bf16*)wo, (const bf16*)q_norm_w,
                               (const bf16*)k_norm_w, norm_eps, (bf16*)y, lse, ws, st);
  return attn_fwd_impl<float>(s, rope_theta, (const float*)x, (const float*)wq, (const float*)wk,
                              (const float*)wv, (const float*)wo, (const float*)q_norm_w,
                              (const float*)k_norm_w, norm_eps, (float*)y, lse, ws, st);
}

int upipe_attn_fwd_noalloc(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int n_q_heads, int n_kv_heads,
                           int head_dim, double rope_theta, int chunk_heads, const void* x, const void* wq,
                           const void* wk, const void* wv, const void* wo, const void* q_norm_w,
                           const void* k_norm_w, float norm_eps, void* y, float* lse, void* stream) {
  Shape s;
  int rc = check_common(dtype, n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads,
                        q_norm_w, k_norm_w, norm_eps, &s);
  if (rc) return rc;
  const void* ptrs[] = {x, wq, wk, wv, wo, y, lse};
  if ((rc = check_ptrs(ptrs, 7))) return rc;
  if (s.norm) {
    const void* np[] = {q_norm_w, k_norm_w};
    if ((rc = check_ptrs(np, 2))) return rc;
  }
  if (make_plan(s, false).total > UPIPE_NOALLOC_SCRATCH_BYTES) return UPIPE_ERR_SCRATCH;
  char* ws = reinterpret_cast<char*>(noalloc_scratch());
  if (!ws) return UPIPE_ERR_HIP;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == UPIPE_BF16)
    return attn_fwd_impl<bf16>(s, rope_theta, (const bf16*)x, (const bf16*)wq, (const bf16*)wk,
                               (const bf16*)wv, (const bf16*)wo, (const bf16*)q_norm_w,
                               (const bf16*)k_norm_w, norm_eps, (bf16*)y, lse, ws, st);
  return attn_fwd_impl<float>(s, rope_theta, (const float*)x, (const float*)wq, (const float*)wk,
                              (const float*)wv, (const float*)wo, (const float*)q_norm_w,
                              (const float*)k_norm_w, norm_eps, (float*)y, lse, ws, st);
}

static int attn_bwd_entry(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int n_q_heads, int n_kv_heads,
                          int head_dim, double rope_theta, int chunk_heads, const void* x, const void* wq,
                          const void* wk, const void* wv, const void* wo, const void* q_norm_w,
                          const void* k_norm_w, float norm_eps, const void* dy, const float* lse, void* dx,
                          float* dwq, float* dwk, float* dwv, float* dwo, float* dq_norm_w, float* dk_norm_w,
                          void* workspace, size_t workspace_bytes, void* stream, bool det) {
  Shape s;
  int rc = check_common(dtype, n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads,
                        q_norm_w, k_norm_w, norm_eps, &s);
  if (rc) return rc;
  const void* ptrs[] = {x, wq, wk, wv, wo, dy, lse, dx, dwq, dwk, dwv, dwo};
  if ((rc = check_ptrs(ptrs, 12))) return rc;
  if (s.norm) {
    const void* np[] = {q_norm_w, k_norm_w, dq_norm_w, dk_norm_w};
    if ((rc = check_ptrs(np, 4))) return rc;
  } else if (dq_norm_w != nullptr || dk_norm_w != nullptr) {
    return UPIPE_ERR_INVALID_ARG;
  }
  if ((rc = check_ws(s, true, workspace, workspace_bytes))) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == UPIPE_BF16)
    return attn_bwd_impl<bf16>(s, rope_theta, (const bf16*)x, (const bf16*)wq, (const bf16*)wk,
                               (const bf16*)wv, (const bf16*)wo, (const bf16*)q_norm_w,
                               (const bf16*)k_norm_w, norm_eps, (const bf16*)dy, lse, (bf16*)dx, dwq,
                               dwk, dwv, dwo, dq_norm_w, dk_norm_w, ws, st, nullptr, det);
  return attn_bwd_impl<float>(s, rope_theta, (const float*)x, (const float*)wq, (const float*)wk,
                              (const float*)wv, (const float*)wo, (const float*)q_norm_w,
                              (const float*)k_norm_w, norm_eps, (const float*)dy, lse, (float*)dx, dwq,
                              dwk, dwv, dwo, dq_norm_w, dk_norm_w, ws, st, nullptr, det);
}

int upipe_attn_bwd(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int n_q_heads, int n_kv_heads,
                   int head_dim, double rope_theta, int chunk_heads, const void* x, const void* wq,
                   const void* wk, const void* wv, const void* wo, const void* q_norm_w,
                   const void* k_norm_w, float norm_eps, const void* dy, const float* lse, void* dx,
                   float* dwq, float* dwk, float* dwv, float* dwo, float* dq_norm_w, float* dk_norm_w,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd_entry(dtype, n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads, x, wq,
                        wk, wv, wo, q_norm_w, k_norm_w, norm_eps, dy, lse, dx, dwq, dwk, dwv, dwo, dq_norm_w,
                        dk_norm_w, workspace, workspace_bytes, stream, false);
}

int upipe_attn_bwd_deterministic(upipe_dtype_t dtype, int64_t n_tokens, int64_t d_model, int n_q_heads,
                                 int n_kv_heads, int head_dim, double rope_theta, int chunk_heads, const void* x,
                                 const void* wq, const void* wk, const void* wv, const void* wo,
                                 const void* q_norm_w, const void* k_norm_w, float norm_eps, const void* dy,
                                 const float* lse, void* dx, float* dwq, float* dwk, float* dwv, float* dwo,
                                 float* dq_norm_w, float* dk_norm_w, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return attn_bwd_entry(dtype, n_tokens, d_model, n_q_heads, n_kv_heads, head_dim, rope_theta, chunk_heads, x, wq,
                        wk, wv, wo, q_norm_w, k_norm_w, norm_eps, dy, lse, dx, dwq, dwk, dwv, dwo, dq_norm_w,
                        dk_norm_w, workspace, workspace_bytes, stream, true);
}

const char* upipe_strerror(int code) {
  switch (code) {
    case UPIPE_OK: return "success";
    case UPIPE_ERR_INVALID_ARG: return "invalid argument (null pointer, non-positive size or bad head counts)";
    case UPIPE_ERR_UNSUPPORTED: return "unsupported shape (head_dim must be 64 or 128, d_model a multiple of 128, "
                                       "chunk_heads must divide n_q_heads and divide or be a multiple of the GQA group)";
    case UPIPE_ERR_WORKSPACE: return "workspace missing or smaller than upipe_attn_workspace_bytes()";
    case UPIPE_ERR_ALIGNMENT: return "misaligned pointer (tensors need 16 bytes, the workspace 256 bytes)";
    case UPIPE_ERR_HIP: return "a HIP kernel launch failed";
    case UPIPE_ERR_SCRATCH: return "upipe_attn_fwd_noalloc: the forward workspace of these sizes exceeds the "
                                   "built-in scratch (UPIPE_NOALLOC_SCRATCH_BYTES); use upipe_attn_fwd";
    default: return "unknown error code";
  }
}

int upipe_version(void) { return 100; }

int upipe_device_peak(int device, double* bf16_dense_tflops, int* compute_units, int* clock_khz) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return UPIPE_ERR_HIP;
  if (bf16_dense_tflops) *bf16_dense_tflops = (double)prop.multiProcessorCount * prop.clockRate * 1e3 * 4096.0 / 1e12;
  if (compute_units) *compute_units = prop.multiProcessorCount;
  if (clock_khz) *clock_khz = prop.clockRate;
  return UPIPE_OK;
}

int upipe_profile_start(void) {
  g_prof.on = true;
  return UPIPE_OK;
}

int upipe_profile_stop(double* total_ms, int64_t* launches, double* flops, int n_kinds) {
  g_prof.on = false;
  for (int k = 0; k < n_kinds; ++k) {
    if (total_ms) total_ms[k] = 0.0;
    if (launches) launches[k] = 0;
    if (flops) flops[k] = 0.0;
  }
  int rc = UPIPE_OK;
  for (const ProfRec& r : g_prof.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      rc = UPIPE_ERR_HIP;
    } else if (r.kind < n_kinds) {
      if (total_ms) total_ms[r.kind] += ms;
      if (launches) launches[r.kind] += 1;
      if (flops) flops[r.kind] += r.flops;
    }
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  return rc;
}

}  // extern "C"
