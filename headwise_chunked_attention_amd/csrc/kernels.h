// Host-side launch interface of the gfx950 kernels (argument blocks + launchers).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;

namespace upipe {

enum { EPI_ACCUM = 0, EPI_HEADS = 1, EPI_STORE = 2, EPI_GLU = 3, EPI_GLU_BWD = 4, EPI_CE = 5, EPI_CE_BWD = 6 };

// Where one group of heads produced by a projection GEMM goes. A head is one
// N-tile of the GEMM (BN == head_dim).
template <typename T>
struct HeadOut {
  T* rm;           // [heads][Np][d] row-major, or null
  T* pre;          // [heads][Np][d] values before norm/RoPE, or null
  const T* gamma;  // [d] RMSNorm weight (norm applied iff non-null)
  int rope;        // rotate (i, i + d/2) pairs by pos * theta^(-2i/d)
  float scale;     // multiplies the values stored to rm (after norm and RoPE)
};

// Gated-SiLU MLP epilogues (BN = 128; F = ldf features).
// EPI_GLU: the B operand is gated: tile t (128 columns of C) takes rows
//   64t .. 64t+63 of b[0] (the gate weight) and then the same rows of b[1]
//   (the up weight), so it holds h and u of the same 64 features. It writes
//     a[m][64t + j] = silu(h) * u          if a is set (forward), and/or
//     hu[m][128t + c] = C[m][c]             if hu is set (h block, u block).
// EPI_GLU_BWD: C = da over features n (ordinary B); reads h, u from hu and
//   writes dh = da * u * silu'(h), du = da * silu(h), a = silu(h) * u.
// All rows m < M; a, dh, du have row stride ldf, hu 2 * ldf.
template <typename T>
struct GluOut {
  T* a;
  T* hu;
  T* dh;
  T* du;
  int64_t ldf;
};

// Cross-entropy epilogues over logits C = h W^T (BN = 128; rows m < M).
// EPI_CE: per row and 128-column tile t, part[(m * N/128 + t) * 2 + {0, 1}] =
//   (max of the tile's logits, sum of exp(logit - that max)); and
//   tgt[m] = C[m][targets[m]] from the tile that holds the target.
// EPI_CE_BWD: dz[m * ldz + n] = (exp(C[m][n] - lse[m]) - [n == targets[m]]) * g[m].
template <typename T>
struct CeOut {
  const int32_t* targets;
  float* part;
  float* tgt;
  const float* lse;
  const float* g;
  T* dz;
  int64_t ldz;
};

// C[m][n] = sum_k A(m,k) B(n,k), both operands contiguous along k.
//   A(m,k) = a + (k / a_kblk) * a_kblk_stride + m * lda + (k % a_kblk)
//   B(n,k) = b[s] + (n - seg_begin(s)) * ldb[s] + k for the segment s holding n
// EPI_ACCUM:  c[m * ldc + n] = (accumulate ? c : 0) + C   (rows m < M)
// EPI_STORE:  c[m * ldc + n] = C (+ add[m * ld_add + n] if add; add may be c)
//             (rows m < M); long k (128-byte k rows)
// EPI_HEADS:  head-wise epilogue per segment (see HeadOut), rows m < Np.
// EPI_GLU, EPI_GLU_BWD: see GluOut. EPI_CE, EPI_CE_BWD: see CeOut.
template <typename T>
struct GemmNT {
  const T* a;
  int64_t lda;
  int64_t a_kblk;
  int64_t a_kblk_stride;
  const T* b[3];
  int64_t ldb[3];
  int64_t seg_end[3];  // cumulative end of each segment along N
  int nseg;
  int64_t M, N, K;
  T* c;
  int64_t ldc;
  int accumulate;
  HeadOut<T> ho[3];
  int64_t Np;
  float eps;
  double log2_theta;
  GluOut<T> glu;
  CeOut<T> ce;
  const T* add;
  int64_t ld_add;
};

// out[m*ldm + n*ldn] += sum_{k in split} A(k,m) B(k,n)   (fp32 atomics)
//   A(k,m) = a + k * lda + m
//   B(k,n) = b + (n / b_nblk) * b_nblk_stride + k * ldb + (n % b_nblk)
template <typename T>
struct GemmTN {
  const T* a;
  int64_t lda;
  const T* b;
  int64_t b_nblk;
  int64_t b_nblk_stride;
  int64_t ldb;
  int64_t M, N, K;
  int64_t ksplit;
  // output column n of segment s (n < seg_end[s]) goes to
  // out[s] + m * ldm + (n - seg_begin(s)) * ldn; segments hold whole n tiles
  float* out[3];
  int64_t seg_end[3];
  int nseg;
  int64_t ldm, ldn;
  // with several k splits: null = add each split's tile into out with fp32
  // atomics (order unspecified); else each split stores its tile to
  // part[split][M][N] and launch_gemm_tn adds the splits into out in split
  // order (bitwise reproducible)
  float* part;
};

// Causal GQA attention forward over one kv head and `nh` q heads.
//   q, o   [nh][Np][D]     k, v [Np][D]
//   lse    [nh] rows of stride lse_stride (caller's [Hq][N]), fp32
// mode 0: online softmax, writes o (normalised) and lse.
// mode 1: reads lse, writes o and delta[h][i] = sum_d dO[h][i][d] * O[h][i][d].
template <typename T>
// The attention kernels take q pre-multiplied by log2(e)/sqrt(D) (so Q K^T
// is the softmax exponent in log2 units) and, in the backward, dout
// pre-multiplied by 1/sqrt(D) (so dO V^T is dP/sqrt(D)); the projection
// epilogue stores them that way. delta is then rowsum(dout o O) of that dout.
struct AttnFwd {
  const T* q;
  const T* k;
  const T* v;
  T* o;
  float* lse;
  int64_t lse_stride;
  const T* dout;  // mode 1
  float* delta;   // mode 1, [nh][Np]
  int64_t N, Np;
  int nh;
};

// Causal GQA attention backward over one kv head and `nh` q heads.
//   q, dout [nh][Np][D]; k, v [Np][D]; lse [nh] rows of stride lse_stride;
//   delta [nh][Np] (= rowsum(dO o O));
//   dk_acc, dv_acc [Np][D] fp32: written, or added to when accumulate (dK/dV kernel);
//   dq [nh][Np][D] fp32: written (dQ kernel).
template <typename T>
struct AttnBwd {
  const T* q;
  const T* k;
  const T* v;
  const T* dout;
  const float* lse;
  int64_t lse_stride;
  const float* delta;
  float* dq;
  float* dk_acc;
  float* dv_acc;
  int64_t N, Np;
  int nh;
  int accumulate;
  float dk_mul;  // sqrt(D) ln 2: dK from the pre-scaled q (see below)
  float dv_mul;  // sqrt(D): dV from the pre-scaled dout
  int no_head_split;  // 1: one workgroup per key block (no fp32 atomics)
};

// Per-row gradient finish for heads stored [nh][Np][D]:
//   g = rope^T(gacc) if rope; g = rmsnorm_bwd(u, gamma, g) if gamma (dgamma += ...);
//   out = g in io dtype; rows >= N are written as zero.
template <typename T>
struct GradFinish {
  const float* gacc;
  const T* u;
  const T* gamma;
  float* dgamma;
  T* out;
  int rope;
  int nh;
  int64_t N, Np;
  float eps;
  double log2_theta;
  // dgamma: each wave stores its partial sums to dg_part[wave][D] (room for
  // dg_waves waves), and launch_grad_finish adds them into dgamma in wave order
  float* dg_part;
  int64_t dg_waves;
};

// RMSNorm over rows of D elements (row stride D), optionally after a residual add:
//   u = x + r (r may be null), rounded to the io dtype;
//   u_out, u_out2 = u (either may be null, u_out may alias x or r);
//   n_out = gamma * u / sqrt(mean(u^2) + eps).
template <typename T>
struct RowNorm {
  const T* x;
  const T* r;
  const T* gamma;
  T* u_out;
  T* u_out2;
  T* n_out;
  int64_t rows, D;
  float eps;
};

// Backward of RowNorm's n_out for upstream gradient g, plus a residual gradient:
//   out = res + rstd (gamma g - uh sum(gamma g uh) / D),  uh = u rstd  (res may be null);
//   dgamma[c] += sum over rows of g uh (fp32 atomics). out may alias u, g or res.
template <typename T>
struct RowNormBwd {
  const T* u;
  const T* g;
  const T* gamma;
  const T* res;
  T* out;
  float* dgamma;
  int64_t rows, D;
  float eps;
};

// Largest D the row kernels take: each thread keeps its share of a row in registers.
constexpr int64_t ROW_NORM_MAX_D = 8192;

template <typename T> hipError_t launch_row_norm(const RowNorm<T>& p, hipStream_t s);
template <typename T> hipError_t launch_row_norm_bwd(const RowNormBwd<T>& p, hipStream_t s);
template <typename T> hipError_t launch_gemm_nt(const GemmNT<T>& p, int epi, int bn, hipStream_t s);
template <typename T> hipError_t launch_gemm_tn(const GemmTN<T>& p, int bn, hipStream_t s);
template <typename T> hipError_t launch_attn_fwd(const AttnFwd<T>& p, int head_dim, int mode, hipStream_t s);
template <typename T> hipError_t launch_attn_bwd_dkdv(const AttnBwd<T>& p, int head_dim, hipStream_t s);
template <typename T> hipError_t launch_attn_bwd_dq(const AttnBwd<T>& p, int head_dim, hipStream_t s);
template <typename T> hipError_t launch_grad_finish(const GradFinish<T>& p, int head_dim, hipStream_t s);
template <typename T>
hipError_t launch_transpose(const T* src, int64_t rows, int64_t cols, int64_t ld_src, T* dst,
                            int64_t ld_dst, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);
// out[r] = sum_k a[r * d + k] * b[r * d + k] for rows r < rows (d = 64 or 128), fp32.
template <typename T>
hipError_t launch_row_dot(const T* a, const T* b, int64_t rows, int d, float* out, hipStream_t s);
// Per row m < rows: lse[m] = log sum over the ntiles tiles of the row's
// (max, sum exp) partials; loss[m] = lse[m] - tgt[m].
hipError_t launch_ce_reduce(const float* part, const float* tgt, int64_t rows, int64_t ntiles, float* lse,
                            float* loss, hipStream_t s);

}  // namespace upipe
