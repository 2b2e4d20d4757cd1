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

}  // namespace upipe

#define HIP_TRY(x)                                 \
  do {                                             \
    if ((x) != hipSuccess) return UPIPE_ERR_HIP;   \
  } while (0)
