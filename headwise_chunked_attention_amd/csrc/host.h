// Host-side helpers shared by the C ABI implementations: workspace carving,
// alignment checks and the opt-in per-kernel timing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace upipe {
namespace host {

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

constexpr size_t REGION_ALIGN = 256;  // every workspace region starts at this alignment

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t at = off;
    off += (bytes + REGION_ALIGN - 1) / REGION_ALIGN * REGION_ALIGN;
    return at;
  }
};

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ---- opt-in per-kernel timing ------------------------------------------
struct ProfRec {
  int kind;
  double flops;
  hipEvent_t a, b;
};
struct Profiler {
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
extern Profiler g_prof;  // one per process (defined with the attention entry points)

// Enqueue one kernel through `launch`, bracketed by events when timing is on.
template <class F>
hipError_t timed(int kind, double flops, hipStream_t st, F&& launch) {
  if (!g_prof.on) return launch();
  hipEvent_t a = g_prof.get(), b = g_prof.get();
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, st);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, st);
  g_prof.recs.push_back({kind, flops, a, b});
  return e;
}

}  // namespace host

// The attention entry points' checks of their scalar arguments (shape,
// rope_theta, q/k norm epsilon): UPIPE_OK or the code they would return.
int attn_check_args(int dtype, int64_t N, int64_t D, int Hq, int Hkv, int d, double theta, int C, float eps);

// Token rows of the attention engine's per-head buffers (N padded).
int64_t attn_padded_rows(int64_t N);

// Scalar arguments of one attention call.
struct AttnCall {
  int dtype;
  int64_t N, D;
  int Hq, Hkv, d;
  double theta;
  int C;
  float eps;  // q/k norm
};

// The attention forward that also keeps every head's O in o_keep
// ([Hq][attn_padded_rows(N)][d], io dtype), and the backward that takes that O
// instead of recomputing it (Delta = rowsum(dO o O) from it, and dWo). Same
// checks, workspace and results as upipe_attn_fwd / upipe_attn_bwd.
template <typename T>
int attn_fwd_keep_o(const AttnCall& c, const void* x, const void* wq, const void* wk, const void* wv, const void* wo,
                    const void* qn, const void* kn, void* y, float* lse, T* o_keep, void* ws, size_t bytes,
                    hipStream_t st);
template <typename T>
int attn_bwd_kept_o(const AttnCall& c, const void* x, const void* wq, const void* wk, const void* wv, const void* wo,
                    const void* qn, const void* kn, const void* dy, const float* lse, const T* o_kept, void* dx,
                    float* dwq, float* dwk, float* dwv, float* dwo, float* dqn, float* dkn, void* ws, size_t bytes,
                    hipStream_t st);

}  // namespace upipe

#define HIP_TRY(x)                                 \
  do {                                             \
    if ((x) != hipSuccess) return UPIPE_ERR_HIP;   \
  } while (0)
