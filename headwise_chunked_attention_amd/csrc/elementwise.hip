// Element-wise and data-movement kernels of the chunk loop: the gradient
// finish of the rotated/normalised heads (RoPE transpose, RMSNorm backward,
// cast), weight-slice transposes and fp32 fills; the row RMSNorm of the
// transformer block (forward with a fused residual add, and backward).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace upipe {

namespace {

DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// One wave per row; lane i < D/2 owns the rotary pair (i, i + D/2).
//   dt = R(-a) g   (transpose of the rotation applied in the forward)
//   du = r (gamma dt - uh * sum(gamma dt uh) / D),  uh = u r,  r = (mean u^2 + eps)^-1/2
//   dgamma += dt * uh
template <typename T, int D>
__global__ __launch_bounds__(256) void grad_finish_kernel(const GradFinish<T> p) {
  const int l = lane_id();
  const bool act = l < D / 2;
  const int i = act ? l : 0;
  const int64_t nrows = (int64_t)p.nh * p.Np;
  const int64_t wstride = (int64_t)gridDim.x * 4;
  float dg0 = 0.f, dg1 = 0.f;
  double omega = 0.0;
  if (p.rope) omega = exp2(-(2.0 * i / D) * p.log2_theta);
  for (int64_t row = (int64_t)blockIdx.x * 4 + wave_id(); row < nrows; row += wstride) {
    const int64_t tok = row % p.Np;
    T* out = p.out + row * D;
    if (tok >= p.N) {
      if (act) {
        out[i] = from_f<T>(0.f);
        out[i + D / 2] = from_f<T>(0.f);
      }
      continue;
    }
    const float* g = p.gacc + row * D;
    float t0 = act ? g[i] : 0.f, t1 = act ? g[i + D / 2] : 0.f;
    if (p.rope) {
      double sd, cd;
      sincos((double)tok * omega, &sd, &cd);
      const float c = (float)cd, s = (float)sd;
      const float a = t0 * c + t1 * s;
      const float b = -t0 * s + t1 * c;
      t0 = a;
      t1 = b;
    }
    if (p.gamma) {
      const T* u = p.u + row * D;
      const float u0 = act ? to_f<T>(u[i]) : 0.f, u1 = act ? to_f<T>(u[i + D / 2]) : 0.f;
      const float ss = wave_sum(u0 * u0 + u1 * u1);
      const float rr = 1.0f / sqrtf(ss / (float)D + p.eps);
      const float uh0 = u0 * rr, uh1 = u1 * rr;
      const float gh0 = act ? to_f<T>(p.gamma[i]) * t0 : 0.f;
      const float gh1 = act ? to_f<T>(p.gamma[i + D / 2]) * t1 : 0.f;
      const float dot = wave_sum(gh0 * uh0 + gh1 * uh1);
      dg0 += t0 * uh0;
      dg1 += t1 * uh1;
      t0 = rr * (gh0 - uh0 * dot / (float)D);
      t1 = rr * (gh1 - uh1 * dot / (float)D);
    }
    if (act) {
      out[i] = from_f<T>(t0);
      out[i + D / 2] = from_f<T>(t1);
    }
  }
  if (p.gamma && p.dgamma && act) {
    // this wave's partial sums; dgamma_reduce_kernel adds them in wave order
    float* part = p.dg_part + ((int64_t)blockIdx.x * 4 + wave_id()) * D;
    part[i] = dg0;
    part[i + D / 2] = dg1;
  }
}

// dgamma[i] += sum over waves w = 0, 1, ... of part[w][i], in that order.
__global__ __launch_bounds__(128) void dgamma_reduce_kernel(const float* part, int64_t waves, int d, float* dgamma) {
  const int i = threadIdx.x;
  if (i >= d) return;
  float acc = 0.f;
  for (int64_t w = 0; w < waves; ++w) acc += part[w * d + i];
  dgamma[i] += acc;
}

// Sum over the 256 threads of a block; every thread gets the total. red holds
// one partial per wave; the trailing barrier lets the caller reuse red.
template <int NVAL>
DEV void block_sum(float (&v)[NVAL], float (*red)[4]) {
#pragma unroll
  for (int k = 0; k < NVAL; ++k) v[k] = wave_sum(v[k]);
  if (lane_id() == 0)
#pragma unroll
    for (int k = 0; k < NVAL; ++k) red[k][threadIdx.x >> 6] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NVAL; ++k) v[k] = red[k][0] + red[k][1] + red[k][2] + red[k][3];
  __syncthreads();
}

// Row RMSNorm: one 256-thread block per row (grid-stride over rows). Thread t
// owns the 16-byte vectors t, t + 256, ... of the row (NV of them, the last
// ones possibly past D), kept in registers between the reduction and the store.
template <typename T, int NV>
__global__ __launch_bounds__(256) void row_norm_kernel(const RowNorm<T> p) {
  constexpr int VEC = 16 / (int)sizeof(T);
  __shared__ float red[1][4];
  const int tid = threadIdx.x;
  float gm[NV][VEC];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t c = (int64_t)(tid + j * 256) * VEC;
    if (c < p.D) ld16_f<T>(p.gamma + c, gm[j]);
  }
  for (int64_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
    const int64_t base = row * p.D;
    float u[NV][VEC];
    float ss[1] = {0.f};
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t c = (int64_t)(tid + j * 256) * VEC;
      if (c >= p.D) continue;
      ld16_f<T>(p.x + base + c, u[j]);
      if (p.r) {
        float t[VEC];
        ld16_f<T>(p.r + base + c, t);
#pragma unroll
        for (int e = 0; e < VEC; ++e) u[j][e] += t[e];
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        u[j][e] = to_f<T>(from_f<T>(u[j][e]));  // the value the io dtype stores
        ss[0] += u[j][e] * u[j][e];
      }
    }
    block_sum<1>(ss, red);
    const float rs = 1.0f / sqrtf(ss[0] / (float)p.D + p.eps);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t c = (int64_t)(tid + j * 256) * VEC;
      if (c >= p.D) continue;
      if (p.u_out) st16_f<T>(p.u_out + base + c, u[j]);
      if (p.u_out2) st16_f<T>(p.u_out2 + base + c, u[j]);
      float n[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) n[e] = gm[j][e] * (u[j][e] * rs);
      st16_f<T>(p.n_out + base + c, n);
    }
  }
}

// Row RMSNorm backward, same thread layout; dgamma partials stay in registers
// over the block's rows and are added once per block.
template <typename T, int NV>
__global__ __launch_bounds__(256) void row_norm_bwd_kernel(const RowNormBwd<T> p) {
  constexpr int VEC = 16 / (int)sizeof(T);
  __shared__ float red[2][4];
  const int tid = threadIdx.x;
  float gm[NV][VEC], dg[NV][VEC];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t c = (int64_t)(tid + j * 256) * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) dg[j][e] = 0.f;
    if (c < p.D) ld16_f<T>(p.gamma + c, gm[j]);
  }
  const float inv_d = 1.0f / (float)p.D;
  for (int64_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
    const int64_t base = row * p.D;
    float u[NV][VEC], g[NV][VEC], rv[NV][VEC];
    float s[2] = {0.f, 0.f};  // sum u^2, sum gamma g u
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t c = (int64_t)(tid + j * 256) * VEC;
      if (c >= p.D) continue;
      ld16_f<T>(p.u + base + c, u[j]);
      ld16_f<T>(p.g + base + c, g[j]);
      if (p.res) ld16_f<T>(p.res + base + c, rv[j]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        s[0] += u[j][e] * u[j][e];
        s[1] += gm[j][e] * g[j][e] * u[j][e];
      }
    }
    block_sum<2>(s, red);
    const float rs = 1.0f / sqrtf(s[0] * inv_d + p.eps);
    const float k = rs * (s[1] * rs) * inv_d;  // rstd * sum(gamma g uh) / D
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t c = (int64_t)(tid + j * 256) * VEC;
      if (c >= p.D) continue;
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float uh = u[j][e] * rs;
        o[e] = rs * gm[j][e] * g[j][e] - uh * k + (p.res ? rv[j][e] : 0.f);
        dg[j][e] += g[j][e] * uh;
      }
      st16_f<T>(p.out + base + c, o);
    }
  }
  if (p.dgamma) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t c = (int64_t)(tid + j * 256) * VEC;
      if (c >= p.D) continue;
#pragma unroll
      for (int e = 0; e < VEC; ++e) atomicAdd(p.dgamma + c + e, dg[j][e]);
    }
  }
}

// dst[c][r] = src[r][c] for a rows x cols block, 32 x 32 tiles through LDS.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* src, int64_t rows, int64_t cols,
                                                        int64_t ld_src, T* dst, int64_t ld_dst) {
  __shared__ float tile[32][33];
  const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int k = ty; k < 32; k += 8) {
    const int64_t r = r0 + k, c = c0 + tx;
    tile[k][tx] = (r < rows && c < cols) ? to_f<T>(src[r * ld_src + c]) : 0.f;
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int64_t c = c0 + k, r = r0 + tx;
    if (r < rows && c < cols) dst[c * ld_dst + r] = from_f<T>(tile[tx][k]);
  }
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

// One wave per row: out[r] = a[r] . b[r] over d <= 128 elements (each lane
// takes d / 64 of them).
template <typename T>
__global__ __launch_bounds__(256) void row_dot_kernel(const T* a, const T* b, int64_t rows, int d, float* out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= rows) return;
  float v = 0.f;
  for (int k = l; k < d; k += 64) v += to_f<T>(a[row * d + k]) * to_f<T>(b[row * d + k]);
  v = wave_sum(v);
  if (l == 0) out[row] = v;
}

// One wave per row: combine the row's per-tile (max, sum exp) partials.
__global__ __launch_bounds__(256) void ce_reduce_kernel(const float* part, const float* tgt, int64_t rows,
                                                        int64_t ntiles, float* lse, float* loss) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= rows) return;
  const float* pr = part + row * ntiles * 2;
  float mx = -INFINITY;
  for (int64_t t = l; t < ntiles; t += 64) mx = fmaxf(mx, pr[t * 2]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float se = 0.f;
  for (int64_t t = l; t < ntiles; t += 64) se += pr[t * 2 + 1] * expf(pr[t * 2] - mx);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) se += __shfl_xor(se, o);
  if (l == 0) {
    const float v = mx + logf(se);
    lse[row] = v;
    loss[row] = v - tgt[row];
  }
}

}  // namespace

hipError_t launch_ce_reduce(const float* part, const float* tgt, int64_t rows, int64_t ntiles, float* lse,
                            float* loss, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(ce_reduce_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, part, tgt, rows, ntiles,
                     lse, loss);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_grad_finish(const GradFinish<T>& p, int head_dim, hipStream_t s) {
  const int64_t rows = (int64_t)p.nh * p.Np;
  int64_t blocks = (rows + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  const bool dg = p.gamma && p.dgamma;
  if (dg) {
    // four waves per block, each with its own row of partial sums
    if (!p.dg_part || p.dg_waves < 4) return hipErrorInvalidValue;
    if (blocks > p.dg_waves / 4) blocks = p.dg_waves / 4;
  }
  if (blocks < 1) return hipSuccess;
  if (head_dim == 64)
    hipLaunchKernelGGL((grad_finish_kernel<T, 64>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else if (head_dim == 128)
    hipLaunchKernelGGL((grad_finish_kernel<T, 128>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !dg) return e;
  hipLaunchKernelGGL(dgamma_reduce_kernel, dim3(1), dim3(128), 0, s, p.dg_part, blocks * 4, head_dim, p.dgamma);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_transpose(const T* src, int64_t rows, int64_t cols, int64_t ld_src, T* dst,
                            int64_t ld_dst, hipStream_t s) {
  const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  hipLaunchKernelGGL((transpose_kernel<T>), grid, dim3(256), 0, s, src, rows, cols, ld_src, dst, ld_dst);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// Vectors per thread for rows of D elements: the smallest of 1, 2, 4, 8 that covers D.
template <typename T>
int row_norm_nv(int64_t D) {
  const int64_t per = 256 * (16 / (int64_t)sizeof(T));
  for (int nv = 1; nv <= 8; nv *= 2)
    if (D <= per * nv) return nv;
  return 0;
}

template <typename T>
hipError_t launch_row_norm(const RowNorm<T>& p, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  if (p.D <= 0 || p.D % (16 / (int64_t)sizeof(T)) || p.D > ROW_NORM_MAX_D) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(p.rows < 8192 ? p.rows : 8192);
  switch (row_norm_nv<T>(p.D)) {
    case 1: hipLaunchKernelGGL((row_norm_kernel<T, 1>), dim3(grid), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((row_norm_kernel<T, 2>), dim3(grid), dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((row_norm_kernel<T, 4>), dim3(grid), dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((row_norm_kernel<T, 8>), dim3(grid), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_row_norm_bwd(const RowNormBwd<T>& p, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  if (p.D <= 0 || p.D % (16 / (int64_t)sizeof(T)) || p.D > ROW_NORM_MAX_D) return hipErrorInvalidValue;
  // fewer blocks than the forward: each block adds its dgamma partials once
  const unsigned grid = (unsigned)(p.rows < 1024 ? p.rows : 1024);
  switch (row_norm_nv<T>(p.D)) {
    case 1: hipLaunchKernelGGL((row_norm_bwd_kernel<T, 1>), dim3(grid), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((row_norm_bwd_kernel<T, 2>), dim3(grid), dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((row_norm_bwd_kernel<T, 4>), dim3(grid), dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((row_norm_bwd_kernel<T, 8>), dim3(grid), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_row_dot(const T* a, const T* b, int64_t rows, int d, float* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d < 1 || d > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL((row_dot_kernel<T>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a, b, rows, d, out);
  return hipGetLastError();
}

template hipError_t launch_row_dot<bf16>(const bf16*, const bf16*, int64_t, int, float*, hipStream_t);
template hipError_t launch_row_dot<float>(const float*, const float*, int64_t, int, float*, hipStream_t);
template hipError_t launch_row_norm<bf16>(const RowNorm<bf16>&, hipStream_t);
template hipError_t launch_row_norm<float>(const RowNorm<float>&, hipStream_t);
template hipError_t launch_row_norm_bwd<bf16>(const RowNormBwd<bf16>&, hipStream_t);
template hipError_t launch_row_norm_bwd<float>(const RowNormBwd<float>&, hipStream_t);
template hipError_t launch_grad_finish<bf16>(const GradFinish<bf16>&, int, hipStream_t);
template hipError_t launch_grad_finish<float>(const GradFinish<float>&, int, hipStream_t);
template hipError_t launch_transpose<bf16>(const bf16*, int64_t, int64_t, int64_t, bf16*, int64_t, hipStream_t);
template hipError_t launch_transpose<float>(const float*, int64_t, int64_t, int64_t, float*, int64_t, hipStream_t);

}  // namespace upipe
