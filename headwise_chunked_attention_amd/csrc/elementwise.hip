// Element-wise and data-movement kernels of the chunk loop: the gradient
// finish of the rotated/normalised heads (RoPE transpose, RMSNorm backward,
// cast), weight-slice transposes and fp32 fills.
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
    atomicAdd(p.dgamma + i, dg0);
    atomicAdd(p.dgamma + i + D / 2, dg1);
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
  if (blocks < 1) return hipSuccess;
  if (head_dim == 64)
    hipLaunchKernelGGL((grad_finish_kernel<T, 64>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else if (head_dim == 128)
    hipLaunchKernelGGL((grad_finish_kernel<T, 128>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    return hipErrorInvalidValue;
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

template hipError_t launch_grad_finish<bf16>(const GradFinish<bf16>&, int, hipStream_t);
template hipError_t launch_grad_finish<float>(const GradFinish<float>&, int, hipStream_t);
template hipError_t launch_transpose<bf16>(const bf16*, int64_t, int64_t, int64_t, bf16*, int64_t, hipStream_t);
template hipError_t launch_transpose<float>(const float*, int64_t, int64_t, int64_t, float*, int64_t, hipStream_t);

}  // namespace upipe
