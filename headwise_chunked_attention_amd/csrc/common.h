// Device helpers shared by the gfx950 kernels: element types, MFMA fragments,
// LDS tile geometry.
//
// MFMA operand convention used throughout (v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_32x32x2f32, both with a 32x32 fp32 accumulator):
//   A operand: lane l supplies row m = l % 32 and the 8 k-values 8*(l/32)..+7
//              of a 16-wide k step;
//   B operand: lane l supplies column n = l % 32 and the same 8 k-values;
//   C/D:       lane l holds column n = l % 32, rows 8*i + 4*(l/32) + j at
//              accumulator index 4*i + j (i, j in 0..3).
// A "Frag" is those 8 k-values of one lane. For bf16 one 32x32x16 MFMA
// consumes a Frag pair; for fp32 eight 32x32x2 MFMAs do (instruction t takes
// element t of each half-wave, so the two half-waves cover k = t and 8 + t).
// Because a contraction does not care how k is numbered, a C tile whose rows
// are the contraction index can feed the next MFMA directly as a B operand:
// step s (16 rows) of the tile is accumulator elements 8*s .. 8*s+7, whose
// physical rows are 16*s + 8*(e/4) + 4*(l/32) + (e%4) for element e. The
// matching A operand then reads those same rows (two runs of 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define DEV __device__ __forceinline__

DEV int lane_id() { return (int)(threadIdx.x & 63); }
DEV int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

// 8 contiguous elements at p (16-byte aligned for bf16, 16-byte aligned halves for fp32).
template <typename T> DEV Frag<T> ld_frag(const T* p);
template <> DEV Frag<bf16> ld_frag<bf16>(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
template <> DEV Frag<float> ld_frag<float>(const float* p) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f;
}

// elements 0..3 from p0 and 4..7 from p1 (each run of 4 contiguous).
template <typename T> DEV Frag<T> ld_frag2(const T* p0, const T* p1);
template <> DEV Frag<bf16> ld_frag2<bf16>(const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  Frag<bf16> f;
  f.v = (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}
template <> DEV Frag<float> ld_frag2<float>(const float* p0, const float* p1) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p0);
  f.hi = *reinterpret_cast<const f32x4*>(p1);
  return f;
}

// Accumulator elements 8*s .. 8*s+7 of a C tile as a B (or A) operand, times mul.
template <typename T> DEV Frag<T> frag_from_acc(const f32x16& c, int s, float mul);
template <> DEV Frag<bf16> frag_from_acc<bf16>(const f32x16& c, int s, float mul) {
  Frag<bf16> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)(c[8 * s + e] * mul);
  return f;
}
template <> DEV Frag<float> frag_from_acc<float>(const f32x16& c, int s, float mul) {
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.lo[e] = c[8 * s + e] * mul;
    f.hi[e] = c[8 * s + 4 + e] * mul;
  }
  return f;
}

// A * B + c0 over one 16-wide k step, into a new accumulator (c0 is kept).
template <typename T> DEV f32x16 mma_first(const Frag<T>& a, const Frag<T>& b, const f32x16& c0);
template <> DEV f32x16 mma_first<bf16>(const Frag<bf16>& a, const Frag<bf16>& b, const f32x16& c0) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c0, 0, 0, 0);
}
template <> DEV f32x16 mma_first<float>(const Frag<float>& a, const Frag<float>& b, const f32x16& c0) {
  f32x16 c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[0], b.lo[0], c0, 0, 0, 0);
#pragma unroll
  for (int i = 1; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[i], b.lo[i], c, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[i], b.hi[i], c, 0, 0, 0);
  return c;
}

// c += A * B over one 16-wide k step.
template <typename T> DEV void mma(f32x16& c, const Frag<T>& a, const Frag<T>& b);
template <> DEV void mma<bf16>(f32x16& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
template <> DEV void mma<float>(f32x16& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int t = 0; t < 4; ++t) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[t], b.lo[t], c, 0, 0, 0);
#pragma unroll
  for (int t = 0; t < 4; ++t) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[t], b.hi[t], c, 0, 0, 0);
}

DEV f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ---- scalar conversions -------------------------------------------------
template <typename T> DEV float to_f(T v);
template <> DEV float to_f<float>(float v) { return v; }
template <> DEV float to_f<bf16>(bf16 v) { return (float)v; }
template <typename T> DEV T from_f(float v);
template <> DEV float from_f<float>(float v) { return v; }
template <> DEV bf16 from_f<bf16>(float v) { return (bf16)v; }

// 16-byte vector of T: VEC elements.
template <typename T> struct Vec16 { static constexpr int N = 16 / sizeof(T); };

// Load VEC (=16/sizeof(T)) elements from 16-byte aligned p as floats.
template <typename T> DEV void ld16_f(const T* p, float* out);
template <> DEV void ld16_f<bf16>(const bf16* p, float* out) {
  bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
}
template <> DEV void ld16_f<float>(const float* p, float* out) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = v[i];
}
template <typename T> DEV void st16_f(T* p, const float* in);
template <> DEV void st16_f<bf16>(bf16* p, const float* in) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)in[i];
  *reinterpret_cast<bf16x8*>(p) = v;
}
template <> DEV void st16_f<float>(float* p, const float* in) {
  f32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = in[i];
  *reinterpret_cast<f32x4*>(p) = v;
}

// Raw 16-byte copy unit.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// VEC (=16/sizeof(T)) elements held in a raw 16-byte register value, as floats.
template <typename T> DEV void raw16_to_f(u32x4 r, float* out);
template <> DEV void raw16_to_f<bf16>(u32x4 r, float* out) {
  const bf16x8 v = __builtin_bit_cast(bf16x8, r);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = (float)v[i];
}
template <> DEV void raw16_to_f<float>(u32x4 r, float* out) {
  const f32x4 v = __builtin_bit_cast(f32x4, r);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = v[i];
}
DEV u32x4 ld_raw16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
DEV void st_raw16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
DEV u32x4 zero_raw16() { return (u32x4){0u, 0u, 0u, 0u}; }

// LDS row stride (in elements) for a tile with `cols` columns: 16 bytes of
// padding per row so consecutive rows start 4 banks apart.
template <typename T> constexpr int lds_stride(int cols) { return cols + 16 / (int)sizeof(T); }

DEV float wave_max_pair(float v) { return fmaxf(v, __shfl_xor(v, 32)); }
DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- LDS tile layout --------------------------------------------------------
// A row-major tile of COLS elements per row. bf16 tiles with 64 or 128 columns
// are stored without padding and their 16-byte chunks are XOR-swizzled by row:
// chunk c of row r lives at chunk position c ^ swz(r). swz is chosen so that
// both access patterns of the kernels are free of bank conflicts:
//   * 16-byte row reads of 16 consecutive rows at one chunk (MFMA operands);
//   * column reads (ds_read_b64_tr_b16) touching 4 consecutive rows and 4
//     consecutive chunks.
// Other tiles keep 16 bytes of padding per row and no swizzle.
template <typename T, int COLS>
struct Tile {
  static constexpr int ROW_BYTES = COLS * (int)sizeof(T);
  static constexpr bool SWZ = sizeof(T) == 2 && (ROW_BYTES == 256 || ROW_BYTES == 128);
  static constexpr int STRIDE = SWZ ? COLS : COLS + 16 / (int)sizeof(T);
  static constexpr int E = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int ELEMS(int rows) { return rows * STRIDE; }
  DEV static int swz(int row) {
    if constexpr (ROW_BYTES == 256) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
  // element offset of (row, col); col may point inside a 16-byte chunk
  DEV static int idx(int row, int col) {
    if constexpr (!SWZ) return row * STRIDE + col;
    else return row * STRIDE + (((col / E) ^ swz(row)) * E) + (col % E);
  }
};

// ---- column reads from LDS tiles -------------------------------------------
// For lane l, the four values X[k0 + j][c0 + 16*((l >> 4) & 1) + (l & 15)],
// j = 0..3, of a tile X in LDS: a column segment of 4 rows. On gfx950 this is
// one ds_read_b64_tr_b16 for bf16: within each 16-lane group, lane L points at
// the 4 elements X[k0 + L/4][cbase + 4*(L%4) .. +3], and the hardware hands
// lane i the column cbase + i of that 4 x 16 block (verified on the device).
template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

typedef short i16x4 __attribute__((ext_vector_type(4)));

template <class L, typename T> DEV typename Vec4<T>::type ld_col4(const T* X, int k0, int c0);
template <class L> DEV bf16x4 ld_col4_bf16(const bf16* X, int k0, int c0) {
  const int l = lane_id(), Ln = l & 15;
  const bf16* p = X + L::idx(k0 + (Ln >> 2), c0 + 16 * ((l >> 4) & 1) + 4 * (Ln & 3));
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}
template <class L> DEV f32x4 ld_col4_f32(const float* X, int k0, int c0) {
  const int l = lane_id();
  const int c = c0 + 16 * ((l >> 4) & 1) + (l & 15);
  return (f32x4){X[L::idx(k0, c)], X[L::idx(k0 + 1, c)], X[L::idx(k0 + 2, c)], X[L::idx(k0 + 3, c)]};
}
template <class L, typename T> DEV typename Vec4<T>::type ld_col4(const T* X, int k0, int c0) {
  if constexpr (sizeof(T) == 2) return ld_col4_bf16<L>(X, k0, c0);
  else return ld_col4_f32<L>(X, k0, c0);
}

// Column reads at precomputed lane offsets. A bf16 swizzled tile's swizzle
// depends only on the low four bits of the row, so ld_col4(X, R + k, c0) with
// R a multiple of 16 and k < 16 reads X + R * STRIDE + (the lane offset of
// ld_col4(X, k, c0)): the lane offsets of the few (k, c0) a loop uses can be
// computed once, and R * STRIDE becomes an immediate offset of the read.
template <class L, int NJ>
struct Col4Plan {
  int off[2][NJ];  // lane element offsets for k = 4 * (lane / 32) + 8x, c0 = 32j
  DEV void init() {
    static_assert(L::SWZ, "bf16 swizzled tiles only");
    const int l = lane_id(), Ln = l & 15, h = l >> 5;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int j = 0; j < NJ; ++j) off[x][j] = L::idx(4 * h + 8 * x + (Ln >> 2), j * 32 + 16 * ((l >> 4) & 1) + 4 * (Ln & 3));
  }
};
DEV bf16x4 ld_col4_at(const bf16* X, int off) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(X + off));
  return __builtin_bit_cast(bf16x4, v);
}

template <typename T> DEV Frag<T> frag_from_col4(typename Vec4<T>::type lo, typename Vec4<T>::type hi);
template <> DEV Frag<bf16> frag_from_col4<bf16>(bf16x4 a, bf16x4 b) {
  Frag<bf16> f;
  f.v = (bf16x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}
template <> DEV Frag<float> frag_from_col4<float>(f32x4 a, f32x4 b) {
  Frag<float> f;
  f.lo = a;
  f.hi = b;
  return f;
}

// Workgroup barrier that orders LDS only. __syncthreads() also fences global
// memory, which makes every wave wait for all of its outstanding global loads
// and atomics at each barrier; the kernels here never exchange global data
// between the threads of a workgroup, so an LDS-scoped fence is enough.
DEV void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- direct global -> LDS tile loads (bf16 swizzled tiles) ------------------
// One wave instruction moves 64 x 16 bytes from global memory straight into
// 1 KB of contiguous LDS (lane l lands at byte 16*l of the wave's LDS base):
// for a swizzled tile that is rows [r0, r0 + 1024/ROW_BYTES) with lane l
// filling physical chunk l % CPR of row r0 + l / CPR, so it fetches logical
// chunk (l % CPR) ^ swz(row). No registers hold the data and the LDS writes
// happen asynchronously; completion is tracked by vmcnt.
//
// The instruction is issued from inline assembly on purpose. Issued through
// the compiler builtin, every later LDS transpose read gets a conservative
// vmcnt(0) wait in front of it (the compiler cannot tell that the read does
// not touch the bytes in flight), which stalls each step until the next tile
// has arrived. Callers load only into LDS stages that no wave reads in the
// meantime and wait for vmcnt(0) before the barrier that publishes the stage.
// M0 (the LDS base of the instruction) is saved and restored around it; the
// s_nop is the wait state required between an M0 write and an LDS DMA.
DEV void lds_dma16(const void* gptr, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds_addr)
      : "memory");
}

template <class L, typename T>
DEV void dma_tile_rows(const T* src, int64_t src_ld, T* lds_tile, int row0) {
  static_assert(L::SWZ, "direct loads need the unpadded swizzled layout");
  constexpr int CPR = L::ROW_BYTES / 16;  // 16-byte chunks per row
  const int l = lane_id();
  const int row = row0 + l / CPR;
  const int chunk = (l % CPR) ^ L::swz(row);
  const T* g = src + (int64_t)row * src_ld + chunk * L::E;
  const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T*)(lds_tile + row0 * L::STRIDE);
  lds_dma16(g, __builtin_amdgcn_readfirstlane(lds));
}

// Wait for this wave's outstanding vector-memory operations (direct LDS loads included).
DEV void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0), expcnt(7), lgkmcnt(15)

// ---- XCD-aware block order ----------------------------------------------------
// The dispatcher hands workgroup b to XCD b % 8, and each XCD has its own L2.
// Blocks that share operands should run on the same XCD at the same time, so a
// logical block index is assigned in groups of 8 consecutive logical blocks
// per XCD: hardware block b (XCD b % 8, its (b / 8)-th block there) gets
// logical block (slot / 8) * 64 + xcd * 8 + slot % 8. Every XCD still walks
// the logical order from first to last (heavy-first schedules stay balanced).
// Bijective on [0, n); a tail of fewer than 64 blocks keeps its index.
DEV int64_t xcd_remap(int64_t b, int64_t n) {
  constexpr int64_t X = 8, G = 8;
  const int64_t full = n - n % (X * G);
  if (b >= full) return b;
  const int64_t xcd = b % X, slot = b / X;
  return (slot / G) * (X * G) + xcd * G + (slot % G);
}
