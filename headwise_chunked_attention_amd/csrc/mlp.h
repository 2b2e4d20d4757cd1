// Engine of the sequence-tiled gated-SiLU MLP, shared by its own C entry
// points and by the transformer block, which runs the MLP one sequence tile
// at a time on the tile's normed input.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace upipe {
namespace mlp {

struct Shape {
  int64_t N, D, F;
  int64_t T;  // rows per tile (and of the tile buffers)
  int es;
};

// Workspace regions (byte offsets). Forward: a. Backward: a, h|u, dh, du
// (du right after dh: the dx product reads [dh | du] as one operand) and the
// transposed weights Wd^T [F][D] and [Wg^T | Wu^T] [D][2F].
struct Plan {
  size_t a, hu, dh, du, wd_t, wgu_t, total;
};

int check_shape(int dtype, int64_t N, int64_t D, int64_t F, int64_t tile, Shape* out);
Plan plan(const Shape& s, bool backward);

// y[0 .. rows) = mlp(x[0 .. rows)) (+ add[0 .. rows) if add; add may be y);
// x, y, add have row stride D; rows <= s.T.
template <typename T>
int fwd_tile(const Shape& s, const T* x, int64_t rows, const T* wg, const T* wu, const T* wd, T* y,
             const T* add, char* ws, hipStream_t st);

// Zero the weight gradients and write the transposed weights into the
// workspace; once, before the tiles of a backward pass.
template <typename T>
int bwd_prep(const Shape& s, const T* wg, const T* wu, const T* wd, float* dwg, float* dwu, float* dwd,
             char* ws, hipStream_t st);

// One tile of the backward: dx[0 .. rows) and the tile's share of the weight
// gradients (added). x, dy, dx have row stride D; rows <= s.T.
template <typename T>
int bwd_tile(const Shape& s, const T* x, const T* dy, int64_t rows, const T* wg, const T* wu, T* dx,
             float* dwg, float* dwu, float* dwd, char* ws, hipStream_t st);

}  // namespace mlp
}  // namespace upipe
