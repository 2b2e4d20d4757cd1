// Projection GEMMs of the chunk loop on gfx950 MFMA.
//
// gemm_nt: C = A B^T with both operands contiguous along k. Used for the
//   chunk's Q/K/V projection (x Wq_c^T, with the per-head RMSNorm + RoPE
//   epilogue), for y (+)= O_c Wo_c^T, for dO_c = dY Wo_c and for
//   dx (+)= dq_c Wq_c. 128 x BN tile, 4 waves in 2 x 2, each wave 64 x BN/2 of
//   32x32 MFMA tiles, k staged through LDS in 128-byte rows (double buffer).
// gemm_tn: out += A^T B with both operands contiguous along the free dims and
//   k = tokens; the weight gradients (dWq = dq^T x, dWo = dY^T O, ...). Each
//   workgroup takes one 128 x BN output tile over one slice of the tokens
//   (split-K), keeps its token-major tiles row-major in LDS, reads the MFMA
//   operands as columns, and adds its partial sum into the fp32 output with
//   atomics.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace upipe {

namespace {

constexpr int BM = 128;
constexpr int NTHREADS = 256;

// KB bytes of k per tile row; LDS rows padded by 16 bytes (16 rows of one
// 16-byte column then hit 16 distinct bank groups).
template <typename T, int KB = 128> struct GemmGeo {
  static constexpr int BK = KB / (int)sizeof(T);
  static constexpr int SK = lds_stride<T>(BK);
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int CPR = BK / VEC;  // 16-byte chunks per tile row
};
// The accumulating products (y/dx, K = a few heads) are bound by the
// read-modify-write of their output: 64-byte k rows and a two-pass epilogue
// keep their LDS at 40 KB, so three workgroups share a CU. The projections
// (K = d_model) keep 128-byte rows (fewer k steps and barriers).
template <int EPI> constexpr int nt_kb() { return EPI == EPI_ACCUM ? 64 : 128; }
// gate/up halves of a gated B tile
template <int EPI> constexpr bool nt_gated() { return EPI == EPI_GLU; }
constexpr int EPI_ROWS = BM / 2;  // rows per epilogue pass
constexpr float LOG2E_F = 1.4426950408889634f;
// 1 / (1 + e^-z) from the hardware exp2 and reciprocal (about 1 ulp each)
DEV float fast_sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-z * LOG2E_F)); }

template <typename T, int BN, int EPI>
constexpr int gemm_smem_bytes() {
  constexpr int main_bytes = 2 * (BM + BN) * GemmGeo<T, nt_kb<EPI>()>::SK * (int)sizeof(T);
  constexpr int epi_bytes = EPI_ROWS * (BN + 4) * 4;
  return main_bytes > epi_bytes ? main_bytes : epi_bytes;
}

// One 16-wide k step of a 2 x 2 wave grid over a BM x BN tile held in LDS as
// As[m][k], Bs[n][k] (row stride SK).
// The wave's A and B fragments of k step ks (16 k) of a tile in LDS.
template <typename T, int BN>
struct TileFrags {
  Frag<T> a[2], b[BN / 64];
};

template <typename T, int BN>
DEV void load_frags(const T* As, const T* Bs, int SK, int ks, int wm, int wn, TileFrags<T, BN>& f) {
  const int l = lane_id();
  const int r = l & 31, h = l >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) f.a[mt] = ld_frag(As + (wm * 64 + mt * 32 + r) * SK + ks * 16 + 8 * h);
#pragma unroll
  for (int nt = 0; nt < BN / 64; ++nt) f.b[nt] = ld_frag(Bs + (wn * (BN / 2) + nt * 32 + r) * SK + ks * 16 + 8 * h);
}

// All k steps of one LDS tile, the fragments of step ks + 1 read before the
// MFMAs of step ks are issued (their LDS latency overlaps those MFMAs).
template <typename T, int BN, int KS>
DEV void mma_tile(const T* As, const T* Bs, int SK, int wm, int wn, f32x16 (&acc)[2][BN / 64]) {
  TileFrags<T, BN> f[2];
  load_frags<T, BN>(As, Bs, SK, 0, wm, wn, f[0]);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) load_frags<T, BN>(As, Bs, SK, ks + 1, wm, wn, f[(ks + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of this step's MFMAs
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < BN / 64; ++nt) mma(acc[mt][nt], f[ks & 1].a[mt], f[ks & 1].b[nt]);
  }
}

// Accumulators -> fp32 LDS tile Cs[rows][BN + 4]; row0 is the tile row of
// Cs row 0 (the waves of other rows skip).
template <int BN>
DEV void acc_to_lds(float* Cs, int row0, int nrows, int wm, int wn, const f32x16 (&acc)[2][BN / 64]) {
  constexpr int NTW = BN / 64, SC = BN + 4;
  if (wm * 64 + 64 <= row0 || wm * 64 >= row0 + nrows) return;
  const int l = lane_id();
  const int col0 = wn * (BN / 2) + (l & 31), h = l >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          Cs[(wm * 64 + mt * 32 + 8 * i + 4 * h + j - row0) * SC + col0 + nt * 32] = acc[mt][nt][4 * i + j];
}

// Per-thread row pointers of the A and B k tiles (fixed over k; a k tile
// adds an offset). Rows of A past M read row M - 1, so no load depends on a
// branch. B rows 0 .. BN/2-1
// come from blo, rows BN/2 .. BN-1 from bhi (the same pointer plus BN/2
// rows, except for a gated tile).
template <typename T, int BN, class G>
struct NtPtrs {
  const T* a[BM * G::CPR / NTHREADS];
  const T* b[BN * G::CPR / NTHREADS];
};

template <typename T, int BN, class G>
DEV void nt_ptrs(const GemmNT<T>& p, const T* blo, const T* bhi, int64_t ldb, int64_t m0, NtPtrs<T, BN, G>& q) {
  constexpr int VEC = G::VEC, CPR = G::CPR;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < BM * CPR / NTHREADS; ++i) {
    const int c = tid + i * NTHREADS;
    const int64_t m = min(m0 + c / CPR, p.M - 1);
    q.a[i] = p.a + m * p.lda + (c % CPR) * VEC;
  }
#pragma unroll
  for (int i = 0; i < BN * CPR / NTHREADS; ++i) {
    const int c = tid + i * NTHREADS;
    const int row = c / CPR;
    q.b[i] = (row < BN / 2 ? blo + row * ldb : bhi + (row - BN / 2) * ldb) + (c % CPR) * VEC;
  }
}

// One k tile into registers: A at element offset aoff (its k block and
// column), B at column k0.
template <typename T, int BN, class G>
DEV void nt_load_tile(const NtPtrs<T, BN, G>& q, int64_t aoff, int64_t k0, u32x4 (&ra)[BM * G::CPR / NTHREADS],
                      u32x4 (&rb)[BN * G::CPR / NTHREADS]) {
#pragma unroll
  for (int i = 0; i < BM * G::CPR / NTHREADS; ++i) ra[i] = ld_raw16(q.a[i] + aoff);
#pragma unroll
  for (int i = 0; i < BN * G::CPR / NTHREADS; ++i) rb[i] = ld_raw16(q.b[i] + k0);
}

// The same load with the addresses formed per call (no pointer registers
// held across the k loop: the accumulating products have few k tiles and
// need the registers for occupancy).
template <typename T, int BN, class G>
DEV void nt_load_tile_direct(const GemmNT<T>& p, const T* blo, const T* bhi, int64_t ldb, int64_t m0, int64_t aoff,
                             int64_t k0, u32x4 (&ra)[BM * G::CPR / NTHREADS], u32x4 (&rb)[BN * G::CPR / NTHREADS]) {
  constexpr int VEC = G::VEC, CPR = G::CPR;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < BM * CPR / NTHREADS; ++i) {
    const int c = tid + i * NTHREADS;
    ra[i] = ld_raw16(p.a + aoff + min(m0 + c / CPR, p.M - 1) * p.lda + (c % CPR) * VEC);
  }
#pragma unroll
  for (int i = 0; i < BN * CPR / NTHREADS; ++i) {
    const int c = tid + i * NTHREADS;
    const int row = c / CPR;
    const T* base = row < BN / 2 ? blo + row * ldb : bhi + (row - BN / 2) * ldb;
    rb[i] = ld_raw16(base + k0 + (c % CPR) * VEC);
  }
}

template <typename T, int BN, class G>
DEV void nt_store_tile(T* As, T* Bs, const u32x4 (&ra)[BM * G::CPR / NTHREADS], const u32x4 (&rb)[BN * G::CPR / NTHREADS]) {
  constexpr int VEC = G::VEC, SK = G::SK, CPR = G::CPR;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < BM * CPR / NTHREADS; ++i) {
    const int c = tid + i * NTHREADS;
    st_raw16(As + (c / CPR) * SK + (c % CPR) * VEC, ra[i]);
  }
#pragma unroll
  for (int i = 0; i < BN * CPR / NTHREADS; ++i) {
    const int c = tid + i * NTHREADS;
    st_raw16(Bs + (c / CPR) * SK + (c % CPR) * VEC, rb[i]);
  }
}

// One epilogue pass of the plain-store, gated-SiLU and cross-entropy
// epilogues over tile rows mr0 .. mr0+ROWS-1 (global row numbers), read from
// the fp32 staging tile Cs[ROWS][BN + 4] by NTH threads.
template <typename T, int BN, int EPI, int ROWS, int NTH>
DEV void epi_pass(const GemmNT<T>& p, const float* Cs, int64_t mr0, int64_t n0, int tid) {
  constexpr int VEC = 16 / (int)sizeof(T), SC = BN + 4;
  if constexpr (EPI == EPI_STORE) {
#pragma unroll
    for (int i = 0; i < ROWS * BN / VEC / NTH; ++i) {
      const int c = tid + i * NTH;
      const int row = c / (BN / VEC), cv = c % (BN / VEC);
      const int64_t m = mr0 + row;
      if (m >= p.M) continue;
      float v[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = Cs[row * SC + cv * VEC + e];
      if (p.add) {  // residual: read before the store, so add may be c itself
        float o[VEC];
        ld16_f<T>(p.add + m * p.ld_add + n0 + cv * VEC, o);
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] += o[e];
      }
      st16_f<T>(p.c + m * p.ldc + n0 + cv * VEC, v);
    }
  } else if constexpr (EPI == EPI_GLU) {
    const GluOut<T>& g = p.glu;
    if (g.a) {  // a = silu(h) * u for the tile's 64 features
      for (int c = tid; c < ROWS * (BN / 2) / VEC; c += NTH) {
        const int row = c / (BN / 2 / VEC), cv = c % (BN / 2 / VEC);
        const int64_t m = mr0 + row;
        if (m >= p.M) continue;
        float v[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float hh = Cs[row * SC + cv * VEC + e], uu = Cs[row * SC + BN / 2 + cv * VEC + e];
          v[e] = hh * fast_sigmoid(hh) * uu;
        }
        st16_f<T>(g.a + m * g.ldf + n0 / 2 + cv * VEC, v);
      }
    }
    if (g.hu) {  // h and u as computed, in blocks of 64 features: h block, then u block
      for (int c = tid; c < ROWS * BN / VEC; c += NTH) {
        const int row = c / (BN / VEC), cv = c % (BN / VEC);
        const int64_t m = mr0 + row;
        if (m >= p.M) continue;
        float v[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] = Cs[row * SC + cv * VEC + e];
        // tile column cc: feature n0/2 + cc % (BN/2), h for cc < BN/2, else u
        const int cc = cv * VEC, f = cc % (BN / 2);
        st16_f<T>(g.hu + m * 2 * g.ldf + n0 + (f / 64) * 128 + (cc >= BN / 2 ? 64 : 0) + f % 64, v);
      }
    }
  } else if constexpr (EPI == EPI_GLU_BWD) {
    // C = da over features n0 .. n0+BN-1; h, u of feature f sit at columns
    // 128 (f / 64) + f % 64 and that + 64 of hu
    const GluOut<T>& g = p.glu;
    for (int c = tid; c < ROWS * BN / VEC; c += NTH) {
      const int row = c / (BN / VEC), cv = c % (BN / VEC);
      const int64_t m = mr0 + row;
      if (m >= p.M) continue;
      const int64_t f0 = n0 + cv * VEC;
      const T* hp = g.hu + m * 2 * g.ldf + (f0 / 64) * 128 + f0 % 64;
      float hh[VEC], uu[VEC], dh[VEC], du[VEC], av[VEC];
      ld16_f<T>(hp, hh);
      ld16_f<T>(hp + 64, uu);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float da = Cs[row * SC + cv * VEC + e];
        const float sg = fast_sigmoid(hh[e]);
        const float sh = hh[e] * sg;
        dh[e] = da * uu[e] * (sg * (1.0f + hh[e] * (1.0f - sg)));
        du[e] = da * sh;
        av[e] = sh * uu[e];
      }
      st16_f<T>(g.dh + m * g.ldf + f0, dh);
      st16_f<T>(g.du + m * g.ldf + f0, du);
      st16_f<T>(g.a + m * g.ldf + f0, av);
    }
  } else if constexpr (EPI == EPI_CE) {
    // four threads per row, 32 logits each of every 128-column part of the
    // tile: the part's row max and sum of exp(logit - max), and the target's
    // logit where the part holds it
    static_assert(ROWS * 4 == NTH && BN % 128 == 0, "four threads per row");
    const CeOut<T>& ce = p.ce;
    const int row = tid >> 2, qq = tid & 3;
    const int64_t m = mr0 + row;
#pragma unroll
    for (int hb = 0; hb < BN / 128; ++hb) {
      const float* cr = Cs + row * SC + hb * 128 + qq * 32;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 32; ++j) mx = fmaxf(mx, cr[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      float se = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) se += fast_exp2((cr[j] - mx) * LOG2E_F);
      se += __shfl_xor(se, 1);
      se += __shfl_xor(se, 2);
      if (m < p.M) {
        const int64_t n1 = n0 + hb * 128;
        if (qq == 0) {
          float* pp = ce.part + (m * (p.N / 128) + n1 / 128) * 2;
          pp[0] = mx;
          pp[1] = se;
        }
        const int64_t t = (int64_t)ce.targets[m] - n1 - qq * 32;
        if (t >= 0 && t < 32) ce.tgt[m] = cr[t];
      }
    }
  } else if constexpr (EPI == EPI_CE_BWD) {
    const CeOut<T>& ce = p.ce;
    for (int c = tid; c < ROWS * BN / VEC; c += NTH) {
      const int row = c / (BN / VEC), cv = c % (BN / VEC);
      const int64_t m = mr0 + row;
      if (m >= p.M) continue;
      const float l = ce.lse[m], gg = ce.g[m];
      const int64_t tcol = (int64_t)ce.targets[m] - n0 - cv * VEC;
      float v[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float pr = fast_exp2((Cs[row * SC + cv * VEC + e] - l) * LOG2E_F) - (tcol == e ? 1.0f : 0.0f);
        v[e] = pr * gg;
      }
      st16_f<T>(ce.dz + m * ce.ldz + n0 + cv * VEC, v);
    }
  }
}

template <typename T, int BN, int EPI>
__global__ __launch_bounds__(NTHREADS) void gemm_nt_kernel(const GemmNT<T> p) {
  using G = GemmGeo<T, nt_kb<EPI>()>;
  constexpr int BK = G::BK, SK = G::SK, VEC = G::VEC;
  constexpr int NTW = BN / 64, SC = BN + 4;
  __shared__ __attribute__((aligned(16))) char smem[gemm_smem_bytes<T, BN, EPI>()];
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + 2 * BM * SK;

  // Consecutive blocks run on one XCD and share the operand of the slower
  // index in its L2: the n tiles of one m tile share that A tile, or (when A
  // is the smaller operand, M < N) the m tiles of one n tile share that B
  // tile, so that the larger operand is streamed from HBM once.
  const int64_t ntn = p.N / BN;
  const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  int64_t mtile, ntile;
  if (p.M < p.N) {
    const int64_t mtn = gridDim.x / ntn;
    mtile = bid % mtn;
    ntile = bid / mtn;
  } else {
    mtile = bid / ntn;
    ntile = bid % ntn;
  }
  const int64_t m0 = mtile * BM, n0 = ntile * BN;
  int seg = 0;
  while (seg + 1 < p.nseg && n0 >= p.seg_end[seg]) ++seg;
  const int64_t seg_begin = seg ? p.seg_end[seg - 1] : 0;
  const int64_t ldb = p.ldb[seg];
  const int64_t nrow0 = n0 - seg_begin;
  const T* blo;
  const T* bhi;
  if constexpr (nt_gated<EPI>()) {
    static_assert(BN == 128, "gated tiles hold 64 gate and 64 up rows");
    blo = p.b[0] + (n0 / 2) * ldb;
    bhi = p.b[1] + (n0 / 2) * ldb;
  } else {
    blo = p.b[seg] + nrow0 * ldb;
    bhi = blo + (BN / 2) * ldb;
  }

  const int w = wave_id();
  const int wm = w >> 1, wn = w & 1;
  f32x16 acc[2][NTW];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = zero16();

  const int tid = threadIdx.x;
  constexpr int CPR = G::CPR;
  // EPI_ACCUM: the old values of the first epilogue pass's rows are fetched
  // before the k loop (K is short here, so their latency would otherwise be
  // exposed), those of the second pass when the epilogue starts
  constexpr int CH = EPI == EPI_ACCUM ? EPI_ROWS * BN / VEC / NTHREADS : 1;
  u32x4 old[CH];
  auto load_old = [&](int pass) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + i * NTHREADS;
      const int row = pass * EPI_ROWS + c / (BN / VEC), cv = c % (BN / VEC);
      const int64_t m = m0 + row;
      old[i] = (p.accumulate && m < p.M) ? ld_raw16(p.c + m * p.ldc + n0 + cv * VEC) : zero_raw16();
    }
  };
  if constexpr (EPI == EPI_ACCUM) load_old(0);

  // Register-staged k tiles, NPF of them in flight: at step kt the tiles
  // kt+1 .. kt+NPF are loading into register slots while tile kt is in LDS.
  // Two slots for the bf16 products with long k (every epilogue but the
  // accumulating one), which wait on HBM; one for the accumulating product
  // (only a few k tiles) and for fp32.
  constexpr int NPF = (sizeof(T) == 2 && EPI != EPI_ACCUM) ? 2 : 1;
  constexpr int RA = BM * CPR / NTHREADS, RB = BN * CPR / NTHREADS;
  u32x4 ra[NPF][RA], rb[NPF][RB];
  const int64_t nk = p.K / BK;
  // A's offset of the k tile loaded last (its k block times the block
  // stride, plus k within the block), stepped one tile at a time: the blocks
  // hold whole k tiles, so no division
  int64_t a_tile = 0, a_blk = 0, a_kin = 0;
  auto a_next = [&]() {
    if (a_tile + 1 < nk) {
      ++a_tile;
      a_kin += BK;
      if (a_kin == p.a_kblk) {
        a_kin = 0;
        a_blk += p.a_kblk_stride;
      }
    }
  };
  NtPtrs<T, BN, G> q;  // with several slots (long k): row pointers set up once
  if constexpr (NPF > 1) nt_ptrs<T, BN, G>(p, blo, bhi, ldb, m0, q);
  auto load = [&](u32x4(&a)[RA], u32x4(&b)[RB]) {
    if constexpr (NPF > 1)
      nt_load_tile<T, BN, G>(q, a_blk + a_kin, a_tile * BK, a, b);
    else
      nt_load_tile_direct<T, BN, G>(p, blo, bhi, ldb, m0, a_blk + a_kin, a_tile * BK, a, b);
  };
#pragma unroll
  for (int i = 0; i < NPF; ++i) {
    if (i) a_next();
    load(ra[i], rb[i]);
  }
  nt_store_tile<T, BN, G>(As, Bs, ra[0], rb[0]);
  lds_barrier();
  auto step = [&](auto slot_c, int64_t kt) {
    constexpr int SLOT = decltype(slot_c)::value, NEXT = (SLOT + 1) % NPF;
    const int buf = (int)(kt & 1);
    // With several slots, past the end the last tile is loaded again: every
    // step issues the same loads, so the wait before a slot's store counts
    // exactly the younger slots.
    if (NPF > 1 || kt + 1 < nk) {  // tile min(kt + NPF, nk - 1)
      a_next();
      load(ra[SLOT], rb[SLOT]);
    }
    const T* Ab = As + buf * BM * SK;
    const T* Bb = Bs + buf * BN * SK;
    mma_tile<T, BN, BK / 16>(Ab, Bb, SK, wm, wn, acc);
    if (NPF > 1 || kt + 1 < nk)
      nt_store_tile<T, BN, G>(As + (buf ^ 1) * BM * SK, Bs + (buf ^ 1) * BN * SK, ra[NEXT], rb[NEXT]);
    lds_barrier();
  };
  int64_t kt = 0;
  for (; kt + NPF <= nk; kt += NPF) {
    step(std::integral_constant<int, 0>(), kt);
    if constexpr (NPF > 1) step(std::integral_constant<int, 1>(), kt + 1);
    if constexpr (NPF > 2) step(std::integral_constant<int, 2>(), kt + 2);
  }
  if constexpr (NPF > 1)
    if (kt < nk) step(std::integral_constant<int, 0>(), kt);
  if constexpr (NPF > 2)
    if (kt + 1 < nk) step(std::integral_constant<int, 1>(), kt + 1);
  // Rows of C past M hold copies of row M - 1's products. Every epilogue but
  // the head-wise one skips them; that one writes the padded rows, as zeros.
  if (EPI == EPI_HEADS && p.M - m0 < BM) {
    const int h = lane_id() >> 5;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (m0 + wm * 64 + mt * 32 + 8 * (e / 4) + 4 * h + e % 4 >= p.M) acc[mt][nt][e] = 0.f;
  }

  // Head-wise epilogue: the rotary frequencies theta^(-2i/d) of the tile's
  // columns, once per workgroup (read after the first pass's barrier).
  __shared__ double omega_s[EPI == EPI_HEADS ? BN / 2 : 1];
  if constexpr (EPI == EPI_HEADS)
    if (tid < BN / 2) omega_s[tid] = exp2(-(2.0 * tid / BN) * p.log2_theta);

  // Epilogue in two passes of EPI_ROWS tile rows through Cs[EPI_ROWS][BN + 4].
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int r0 = pass * EPI_ROWS;
    if (pass) lds_barrier();  // the previous pass is done with Cs
    acc_to_lds<BN>(Cs, r0, EPI_ROWS, wm, wn, acc);
    lds_barrier();

    if constexpr (EPI == EPI_STORE || EPI == EPI_GLU || EPI == EPI_GLU_BWD || EPI == EPI_CE || EPI == EPI_CE_BWD) {
      epi_pass<T, BN, EPI, EPI_ROWS, NTHREADS>(p, Cs, m0 + r0, n0, tid);
    } else if constexpr (EPI == EPI_ACCUM) {
      if (pass) load_old(1);
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = tid + i * NTHREADS;
        const int row = c / (BN / VEC), cv = c % (BN / VEC);
        const int64_t m = m0 + r0 + row;
        if (m >= p.M) continue;
        float v[VEC], o[VEC];
        raw16_to_f<T>(old[i], o);
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[e] = Cs[row * SC + cv * VEC + e] + o[e];
        st16_f<T>(p.c + m * p.ldc + n0 + cv * VEC, v);
      }
    } else {
      const HeadOut<T> ho = p.ho[seg];
      const int64_t head = nrow0 / BN;
      const int64_t mr = m0 + r0;  // first token row of the pass
      if (ho.pre) {
        T* dst = ho.pre + head * p.Np * BN + mr * BN;
        for (int c = tid; c < EPI_ROWS * BN / VEC; c += NTHREADS) {
          const int row = c / (BN / VEC), cv = c % (BN / VEC);
          float v[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = Cs[row * SC + cv * VEC + e];
          st16_f<T>(dst + row * BN + cv * VEC, v);
        }
        lds_barrier();
      }
      if (ho.gamma || ho.rope) {
        // four threads per row; quarter q covers pairs [q*BN/8, q*BN/8 + BN/8)
        static_assert(EPI_ROWS * 4 == NTHREADS, "four threads per row");
        const int row = tid >> 2, qq = tid & 3;
        float* cr = Cs + row * SC;
        constexpr int PP = BN / 8;
        if (ho.gamma) {
          float ss = 0.f;
#pragma unroll 4
          for (int i = qq * PP; i < qq * PP + PP; ++i) ss += cr[i] * cr[i] + cr[i + BN / 2] * cr[i + BN / 2];
          ss += __shfl_xor(ss, 1);
          ss += __shfl_xor(ss, 2);
          const float rs = 1.0f / sqrtf(ss / (float)BN + p.eps);
          for (int i = qq * PP; i < qq * PP + PP; ++i) {
            cr[i] = to_f<T>(ho.gamma[i]) * (cr[i] * rs);
            cr[i + BN / 2] = to_f<T>(ho.gamma[i + BN / 2]) * (cr[i + BN / 2] * rs);
          }
        }
        if (ho.rope) {
          // angle p * omega_i in fp64, reduced mod 2 pi in fp64 (|r| <= pi);
          // sin and cos of the reduced angle in fp32
          const double pos = (double)(mr + row);
          for (int i = qq * PP; i < qq * PP + PP; ++i) {
            const double ang = pos * omega_s[i];
            const double red = fma(-rint(ang * 0.15915494309189535), 6.283185307179586, ang);
            float sn, c;
            sincosf((float)red, &sn, &c);
            const float u = cr[i], wv = cr[i + BN / 2];
            cr[i] = u * c - wv * sn;
            cr[i + BN / 2] = wv * c + u * sn;
          }
        }
        lds_barrier();
      }
      if (ho.rm) {
        T* dst = ho.rm + head * p.Np * BN + mr * BN;
        for (int c = tid; c < EPI_ROWS * BN / VEC; c += NTHREADS) {
          const int row = c / (BN / VEC), cv = c % (BN / VEC);
          float v[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) v[e] = Cs[row * SC + cv * VEC + e] * ho.scale;
          st16_f<T>(dst + row * BN + cv * VEC, v);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// gemm_nt on 256 x 256 tiles (bf16, long k: the MLP and LM-head products)
// ------------------------------------------------------------------------
// 8 waves in 2 x 4, each 128 x 64 of 32x32 MFMA tiles: per 16-wide k step a
// wave reads 4 A and 2 B fragments for 8 MFMAs, where the 128 x 128 kernel
// reads 4 for 4, and a k tile of 64 is 32 MFMAs per wave between barriers
// instead of 16. k tiles arrive by direct global -> LDS loads into two
// 64 KB stages of swizzled 128-byte rows (no register staging). Rows of A
// past M load row M - 1. The epilogue runs in two passes of 128 rows
// through an fp32 staging tile, with the epilogue code of the 128 x 128
// kernel.
constexpr int BIG = 256;
constexpr int BIG_THREADS = 512;
constexpr int BIG_BK = 64;
using BigL = Tile<bf16, BIG_BK>;  // [rows][64 k]

constexpr int big_smem_bytes() {
  constexpr int main_bytes = 2 * 2 * BigL::ELEMS(BIG) * 2;  // two stages of A and B
  constexpr int epi_bytes = (BIG / 2) * (BIG + 4) * 4;
  return main_bytes > epi_bytes ? main_bytes : epi_bytes;
}

// Direct loads of rows [row0, row0 + 8) of a [BIG][64] k tile: row `row` of
// the tile comes from src_row(row) (a pointer at the tile's first k).
template <class F>
DEV void big_dma_rows(bf16* tile, int row0, F src_row) {
  constexpr int CPR = BigL::ROW_BYTES / 16;  // 16-byte chunks per row
  const int l = lane_id();
  const int row = row0 + l / CPR;
  const int chunk = (l % CPR) ^ BigL::swz(row);
  const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)(tile + row0 * BigL::STRIDE);
  lds_dma16(src_row(row) + chunk * BigL::E, __builtin_amdgcn_readfirstlane(lds));
}

template <int EPI>
__global__ __launch_bounds__(BIG_THREADS) void gemm_nt_big_kernel(const GemmNT<bf16> p) {
  using T = bf16;
  constexpr int SC = BIG + 4;
  constexpr int TILE = BigL::ELEMS(BIG);
  constexpr int RPI = 1024 / BigL::ROW_BYTES;  // rows per direct-load instruction
  static_assert(BIG / RPI / (BIG_THREADS / 64) == 4, "four direct loads per wave and operand");
  __shared__ __attribute__((aligned(16))) char smem[big_smem_bytes()];
  T* sm = reinterpret_cast<T*>(smem);  // stage s: A at 2 s TILE, B at (2 s + 1) TILE

  // tile order as in gemm_nt_kernel (XCD-aware; the smaller operand's tiles
  // vary fastest)
  const int64_t ntn = p.N / BIG;
  const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  int64_t mtile, ntile;
  if (p.M < p.N) {
    const int64_t mtn = gridDim.x / ntn;
    mtile = bid % mtn;
    ntile = bid / mtn;
  } else {
    mtile = bid / ntn;
    ntile = bid % ntn;
  }
  const int64_t m0 = mtile * BIG, n0 = ntile * BIG;
  const int64_t ldb = p.ldb[0];
  const T* blo;
  const T* bhi;
  if constexpr (EPI == EPI_GLU) {  // 128 gate rows, then the same 128 up rows
    blo = p.b[0] + (n0 / 2) * ldb;
    bhi = p.b[1] + (n0 / 2) * ldb;
  } else {
    blo = p.b[0] + n0 * ldb;
    bhi = blo + (BIG / 2) * ldb;
  }

  const int w = wave_id(), l = lane_id(), r = l & 31, h = l >> 5;
  const int wm = w >> 2, wn = w & 3;  // rows wm*128 .., columns wn*64 ..
  const int tid = threadIdx.x;
  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = zero16();

  const int64_t nk = p.K / BIG_BK;
  // A's offset of a k tile: its k block times the block stride plus k within
  // the block (the blocks hold whole k tiles)
  int64_t a_blk = 0, a_kin = 0;
  auto dma_tile = [&](int64_t kt, int stage) {
    T* As = sm + 2 * stage * TILE;
    T* Bs = As + TILE;
    const T* a = p.a + a_blk + a_kin;
    const int64_t k0 = kt * BIG_BK;
    // load i moves rows 8 (8 i + w) .. +7: B loads 0, 1 are gate/low rows, 2, 3 high rows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row0 = (i * 8 + w) * RPI;
      big_dma_rows(As, row0, [&](int row) { return a + min(m0 + row, p.M - 1) * p.lda; });
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row0 = (i * 8 + w) * RPI;
      if (i < 2)
        big_dma_rows(Bs, row0, [&](int row) { return blo + row * ldb + k0; });
      else
        big_dma_rows(Bs, row0, [&](int row) { return bhi + (row - BIG / 2) * ldb + k0; });
    }
    a_kin += BIG_BK;
    if (a_kin == p.a_kblk) {
      a_kin = 0;
      a_blk += p.a_kblk_stride;
    }
  };

  // fragments of 16-wide k step ks of the stage in LDS
  auto frags = [&](const T* As, const T* Bs, int ks, Frag<T> (&fa)[4], Frag<T> (&fb)[2]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) fa[mt] = ld_frag(As + BigL::idx(wm * 128 + mt * 32 + r, ks * 16 + 8 * h));
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) fb[nt] = ld_frag(Bs + BigL::idx(wn * 64 + nt * 32 + r, ks * 16 + 8 * h));
  };

  dma_tile(0, 0);
  wait_vmem();
  lds_barrier();
  // As in the TN kernel, the last 16-wide step of k tile kt issues its MFMAs
  // after the barrier (from ring slot 1), covering the latency of tile
  // kt + 1's first fragment reads.
  constexpr int NKS = BIG_BK / 16;
  static_assert(NKS % 2 == 0, "the deferred step uses ring slot 1");
  Frag<T> fa[2][4], fb[2][2];
  auto mma_step = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) mma(acc[mt][nt], fa[slot][mt], fb[slot][nt]);
  };
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int stage = (int)(kt & 1);
    const T* As = sm + 2 * stage * TILE;
    const T* Bs = As + TILE;
    // the first fragment reads go out before the next tile's loads are
    // issued, so their latency overlaps that issue
    frags(As, Bs, 0, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) dma_tile(kt + 1, stage ^ 1);
    if (kt > 0) {
      __builtin_amdgcn_sched_barrier(0);
      mma_step(1);  // the deferred last step of tile kt - 1
    }
#pragma unroll
    for (int ks = 0; ks < NKS - 1; ++ks) {
      frags(As, Bs, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of this step's MFMAs
      mma_step(ks & 1);
    }
    if (kt + 1 < nk) wait_vmem();  // this wave's loads of the next stage have landed
    lds_barrier();
  }
  if (nk > 0) mma_step(1);

  // Epilogue in two passes of 128 rows through Cs[128][BIG + 4]: pass q
  // holds the rows of the waves with wm == q.
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (pass) lds_barrier();  // the previous pass is done with Cs
    if (wm == pass) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              Cs[(mt * 32 + 8 * i + 4 * h + j) * SC + wn * 64 + nt * 32 + r] = acc[mt][nt][4 * i + j];
    }
    lds_barrier();
    epi_pass<T, BIG, EPI, BIG / 2, BIG_THREADS>(p, Cs, m0 + pass * (BIG / 2), n0, tid);
  }
}

// ------------------------------------------------------------------------
// split-K GEMM for weight gradients
// ------------------------------------------------------------------------
// A token-major tile [BK tokens][COLS] kept row-major in LDS (Tile layout):
// the global loads are coalesced (consecutive lanes take consecutive 16-byte
// chunks of a row) and the MFMA operands, which need 8 consecutive tokens for
// one column, are column reads (LDS transpose reads for bf16).
template <typename T, int COLS>
struct TnTile {
  using L = Tile<T, COLS>;
  static constexpr int VEC = 16 / (int)sizeof(T), BK = GemmGeo<T, 128>::BK;
  static constexpr int RCH = COLS / VEC;        // 16-byte chunks per row
  static constexpr int PER = BK * RCH / NTHREADS;  // chunks per thread
  static_assert((BK * RCH) % NTHREADS == 0, "tile chunks");
};

// Thread t loads the 16-byte chunk t % RCH of rows t / RCH + i * (NTHREADS / RCH)
// of each k tile: the same column for every i. Its row pointers (relative to
// k = 0) are set up once; a full tile then costs one 64-bit add per load.
// On a tile that runs past K (uniform test) rows at or past K are read from
// row K - 1, and the A operand replaces them with zeros.
template <typename T, int COLS>
struct TnPtrs {
  const T* p[TnTile<T, COLS>::PER];
};

template <typename T, int COLS>
DEV void tn_ptrs(const T* base, int64_t ld, TnPtrs<T, COLS>& q) {
  using G = TnTile<T, COLS>;
#pragma unroll
  for (int i = 0; i < G::PER; ++i)
    q.p[i] = base + (int64_t)(threadIdx.x / G::RCH + i * (NTHREADS / G::RCH)) * ld;
}

template <typename T, int COLS, bool ZERO_TAIL>
DEV void tn_load(const TnPtrs<T, COLS>& q, int64_t ld, int64_t k0, int64_t K, u32x4 (&r)[TnTile<T, COLS>::PER]) {
  using G = TnTile<T, COLS>;
  const int64_t off = k0 * ld;
  if (k0 + G::BK <= K) {
#pragma unroll
    for (int i = 0; i < G::PER; ++i) r[i] = ld_raw16(q.p[i] + off);
  } else {
    // the last tile of a split: clamp the rows, and zero them in one operand
#pragma unroll
    for (int i = 0; i < G::PER; ++i) {
      const int64_t rel = threadIdx.x / G::RCH + i * (NTHREADS / G::RCH);
      const bool in = k0 + rel < K;
      r[i] = ld_raw16(q.p[i] + ((in ? k0 + rel : K - 1) - rel) * ld);
      if (ZERO_TAIL && !in) r[i] = zero_raw16();
    }
  }
}

template <typename T, int COLS>
DEV void tn_store(T* S, const u32x4 (&r)[TnTile<T, COLS>::PER]) {
  using G = TnTile<T, COLS>;
#pragma unroll
  for (int i = 0; i < G::PER; ++i) {
    const int c = threadIdx.x + i * NTHREADS;
    st_raw16(S + G::L::idx(c / G::RCH, (c % G::RCH) * G::VEC), r[i]);
  }
}

template <typename T, int BN>
constexpr int tn_smem_bytes() {
  constexpr int BK = GemmGeo<T, 128>::BK;
  constexpr int main_bytes = 2 * (Tile<T, BM>::ELEMS(BK) + Tile<T, BN>::ELEMS(BK)) * (int)sizeof(T);
  constexpr int epi_bytes = BM * (BN + 4) * 4;
  return main_bytes > epi_bytes ? main_bytes : epi_bytes;
}

template <typename T, int BN>
__global__ __launch_bounds__(NTHREADS) void gemm_tn_kernel(const GemmTN<T> p) {
  constexpr int BK = GemmGeo<T, 128>::BK;
  constexpr int NTW = BN / 64, SC = BN + 4;
  using LA = Tile<T, BM>;
  using LB = Tile<T, BN>;
  constexpr int A_EL = LA::ELEMS(BK), B_EL = LB::ELEMS(BK);
  __shared__ __attribute__((aligned(16))) char smem[tn_smem_bytes<T, BN>()];
  T* As = reinterpret_cast<T*>(smem);  // [2][BK tokens][BM]
  T* Bs = As + 2 * A_EL;               // [2][BK tokens][BN]

  // 1-D grid, consecutive logical blocks on one XCD: the faster tile index
  // runs over the smaller operand, so the blocks that share a tile of the
  // larger one (m tiles of one n tile when M <= N, else n tiles of one m
  // tile) run together and it is streamed from HBM once.
  const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t gm = p.M / BM, gn = p.N / BN;
  const bool mfast = p.M <= p.N;
  const int64_t m0 = (mfast ? bid % gm : (bid / gn) % gm) * BM;
  const int64_t n0 = (mfast ? (bid / gm) % gn : bid % gn) * BN;
  const int64_t kb = (bid / (gm * gn)) * p.ksplit;
  const int64_t ke = (kb + p.ksplit < p.K) ? kb + p.ksplit : p.K;

  // this thread's column of each operand (fixed over k) and its row pointers
  TnPtrs<T, BM> pa;
  TnPtrs<T, BN> pb;
  {
    const int col_a = (threadIdx.x % TnTile<T, BM>::RCH) * TnTile<T, BM>::VEC;
    const int col_b = (threadIdx.x % TnTile<T, BN>::RCH) * TnTile<T, BN>::VEC;
    const int64_t n = n0 + col_b;
    tn_ptrs<T, BM>(p.a + m0 + col_a, p.lda, pa);
    tn_ptrs<T, BN>(p.b + (n / p.b_nblk) * p.b_nblk_stride + (n % p.b_nblk), p.ldb, pb);
  }

  const int w = wave_id();
  const int wm = w >> 1, wn = w & 1;
  const int h = lane_id() >> 5;
  f32x16 acc[2][NTW];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = zero16();

  u32x4 ra[TnTile<T, BM>::PER], rb[TnTile<T, BN>::PER];
  const int64_t nk = (ke - kb + BK - 1) / BK;
  tn_load<T, BM, true>(pa, p.lda, kb, ke, ra);
  tn_load<T, BN, false>(pb, p.ldb, kb, ke, rb);
  tn_store<T, BM>(As, ra);
  tn_store<T, BN>(Bs, rb);
  lds_barrier();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nk) {
      tn_load<T, BM, true>(pa, p.lda, kb + (kt + 1) * BK, ke, ra);
      tn_load<T, BN, false>(pb, p.ldb, kb + (kt + 1) * BK, ke, rb);
    }
    const T* Ab = As + buf * A_EL;
    const T* Bb = Bs + buf * B_EL;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int k0 = ks * 16 + 8 * h;  // tokens 8h..8h+7 of the step
      Frag<T> a[2], b[NTW];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int c0 = wm * 64 + mt * 32;
        a[mt] = frag_from_col4<T>(ld_col4<LA>(Ab, k0, c0), ld_col4<LA>(Ab, k0 + 4, c0));
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int c0 = wn * (BN / 2) + nt * 32;
        b[nt] = frag_from_col4<T>(ld_col4<LB>(Bb, k0, c0), ld_col4<LB>(Bb, k0 + 4, c0));
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) mma(acc[mt][nt], a[mt], b[nt]);
    }
    if (kt + 1 < nk) {
      tn_store<T, BM>(As + (buf ^ 1) * A_EL, ra);
      tn_store<T, BN>(Bs + (buf ^ 1) * B_EL, rb);
    }
    lds_barrier();
  }

  float* Cs = reinterpret_cast<float*>(smem);
  acc_to_lds<BN>(Cs, 0, BM, wm, wn, acc);
  lds_barrier();
  const int tid = threadIdx.x;
  if (p.part && p.ksplit < p.K) {
    // fixed-order reduction: this split's tile goes whole to part[split], and
    // splitk_reduce_kernel adds the splits into out one after another
    float* dst = p.part + (bid / (gm * gn)) * p.M * p.N;
    for (int c = tid; c < BM * BN / 4; c += NTHREADS) {
      const int row = c / (BN / 4), col = (c % (BN / 4)) * 4;
      *reinterpret_cast<f32x4*>(dst + (m0 + row) * p.N + (n0 + col)) =
          *reinterpret_cast<const f32x4*>(Cs + row * SC + col);
    }
    return;
  }
  int seg = 0;
  while (seg + 1 < p.nseg && n0 >= p.seg_end[seg]) ++seg;
  float* out = p.out[seg];
  const int64_t nc0 = n0 - (seg ? p.seg_end[seg - 1] : 0);
  if (p.ldn == 1 && p.ksplit >= p.K && (p.ldm & 3) == 0) {
    // one k split: this workgroup is the only writer of its tile in this
    // launch (launches on a stream run in order), so a plain read-modify-write
    for (int c = tid; c < BM * BN / 4; c += NTHREADS) {
      const int row = c / (BN / 4), col = (c % (BN / 4)) * 4;
      f32x4* o = reinterpret_cast<f32x4*>(out + (m0 + row) * p.ldm + (nc0 + col));
      *o += *reinterpret_cast<const f32x4*>(Cs + row * SC + col);
    }
  } else if (p.ldn == 1) {
    for (int c = tid; c < BM * BN; c += NTHREADS) {
      const int row = c / BN, col = c % BN;
      atomicAdd(out + (m0 + row) * p.ldm + (nc0 + col), Cs[row * SC + col]);
    }
  } else {
    for (int c = tid; c < BM * BN; c += NTHREADS) {
      const int col = c / BM, row = c % BM;
      atomicAdd(out + (m0 + row) * p.ldm + (nc0 + col) * p.ldn, Cs[row * SC + col]);
    }
  }
}

// ------------------------------------------------------------------------
// gemm_tn on 256 x 256 tiles (bf16): the MLP and LM-head weight gradients
// ------------------------------------------------------------------------
// 8 waves in 2 x 4, each 128 x 64 of the output. A k tile is 64 tokens of
// both operands' 256 columns, each operand kept as two [64][128] halves in
// swizzled 256-byte rows and loaded straight into LDS; the MFMA operands
// (8 consecutive tokens of one column) are LDS transpose reads. Two 64 KB
// stages. The output tile goes through an fp32 staging tile in two passes of
// 128 rows and is added as in gemm_tn_kernel.
using TnBigL = Tile<bf16, 128>;  // [tokens][128 columns]

template <int UNUSED = 0>
__global__ __launch_bounds__(BIG_THREADS) void gemm_tn_big_kernel(const GemmTN<bf16> p) {
  using T = bf16;
  constexpr int HALF = TnBigL::ELEMS(BIG_BK);  // [64 tokens][128 columns]
  constexpr int OPER = 2 * HALF;                // one operand's k tile: halves 0 and 1
  constexpr int SC = BIG + 4;
  constexpr int CPR = TnBigL::ROW_BYTES / 16;  // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                // rows per direct-load instruction
  static_assert(2 * 2 * BIG_BK / RPI == 8 * (BIG_THREADS / 64), "eight direct loads per wave");
  __shared__ __attribute__((aligned(16))) char smem[big_smem_bytes()];
  T* sm = reinterpret_cast<T*>(smem);  // stage s: A at 2 s OPER, B at (2 s + 1) OPER

  // tile order as in gemm_tn_kernel
  const int64_t bid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t gm = p.M / BIG, gn = p.N / BIG;
  const bool mfast = p.M <= p.N;
  const int64_t m0 = (mfast ? bid % gm : (bid / gn) % gm) * BIG;
  const int64_t n0 = (mfast ? (bid / gm) % gn : bid % gn) * BIG;
  const int64_t split = bid / (gm * gn);
  const int64_t kb = split * p.ksplit;
  const int64_t ke = (kb + p.ksplit < p.K) ? kb + p.ksplit : p.K;
  // column bases of the operands' halves (a half never straddles a B block);
  // plain values, not an array indexed per wave (that would live in scratch)
  const T* a0 = p.a + m0;
  const T* a1 = a0 + 128;
  const T* b0 = p.b + (n0 / p.b_nblk) * p.b_nblk_stride + (n0 % p.b_nblk);
  const T* b1 = p.b + ((n0 + 128) / p.b_nblk) * p.b_nblk_stride + ((n0 + 128) % p.b_nblk);

  const int w = wave_id(), l = lane_id(), r = l & 31, h = l >> 5;
  const int wm = w >> 2, wn = w & 3;
  const int tid = threadIdx.x;
  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = zero16();

  // Load i of a stage (unrolled: operand i / 4, half (i / 2) % 2 known at
  // compile time) moves token rows 4 rb .. 4 rb + 3 of the k tile, row block
  // rb = (i % 2) * 8 + w; the eight waves cover the 16 row blocks of each half.
  const int64_t lda = p.lda, ldb = p.ldb;
  auto dma_tile = [&](int64_t t0, int stage) {
    T* st = sm + 2 * stage * OPER;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int op = i / 4, hb = (i / 2) % 2;
      const int row0 = ((i % 2) * 8 + w) * RPI;
      const T* src = op ? (hb ? b1 : b0) : (hb ? a1 : a0);
      const int64_t ld = op ? ldb : lda;
      T* tile = st + op * OPER + hb * HALF;
      const int row = row0 + l / CPR;
      const int chunk = (l % CPR) ^ TnBigL::swz(row);
      const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T*)(tile + row0 * TnBigL::STRIDE);
      lds_dma16(src + (t0 + row) * ld + chunk * TnBigL::E, __builtin_amdgcn_readfirstlane(lds));
    }
  };
  // Lane offsets of the column reads, computed once: the swizzle depends only
  // on a row's low four bits, which a 16-token step does not change, so step
  // ks adds 16 ks rows to the base. Output column c of the tile lives in half
  // c / 128: A rows wm*128 + mt*32 are half wm, B columns wn*64 + nt*32 half
  // wn / 2.
  int offa[2][4], offb[2][2];
  {
    const int Ln = l & 15, hi = (l >> 4) & 1;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) offa[x][mt] = TnBigL::idx(4 * x + 8 * h + (Ln >> 2), mt * 32 + 16 * hi + 4 * (Ln & 3));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        offb[x][nt] = TnBigL::idx(4 * x + 8 * h + (Ln >> 2), (wn * 64 + nt * 32) % 128 + 16 * hi + 4 * (Ln & 3));
    }
  }
  auto frags = [&](const T* st, int ks, Frag<T> (&fa)[4], Frag<T> (&fb)[2]) {
    const T* Xa = st + wm * HALF + ks * 16 * TnBigL::STRIDE;
    const T* Xb = st + OPER + (wn >> 1) * HALF + ks * 16 * TnBigL::STRIDE;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) fa[mt] = frag_from_col4<T>(ld_col4_at(Xa, offa[0][mt]), ld_col4_at(Xa, offa[1][mt]));
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) fb[nt] = frag_from_col4<T>(ld_col4_at(Xb, offb[0][nt]), ld_col4_at(Xb, offb[1][nt]));
  };

  const int64_t nk = (ke - kb) / BIG_BK;  // the launcher admits whole k tiles only
  if (nk > 0) {
    dma_tile(kb, 0);
    wait_vmem();
  }
  lds_barrier();
  // The last 16-wide step of k tile kt issues its MFMAs after the barrier,
  // beside the first column reads of tile kt + 1: its fragments are in
  // registers (slot 1 of the ring), so the LDS latency after the barrier is
  // covered by MFMA work instead of stalling every wave at once.
  constexpr int NKS = BIG_BK / 16;
  static_assert(NKS % 2 == 0, "the deferred step uses ring slot 1");
  Frag<T> fa[2][4], fb[2][2];
  auto mma_step = [&](int slot) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) mma(acc[mt][nt], fa[slot][mt], fb[slot][nt]);
  };
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int stage = (int)(kt & 1);
    if (kt + 1 < nk) dma_tile(kb + (kt + 1) * BIG_BK, stage ^ 1);
    const T* st = sm + 2 * stage * OPER;
    frags(st, 0, fa[0], fb[0]);
    if (kt > 0) {
      __builtin_amdgcn_sched_barrier(0);
      mma_step(1);  // the deferred last step of tile kt - 1
    }
#pragma unroll
    for (int ks = 0; ks < NKS - 1; ++ks) {
      frags(st, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);  // keep those reads ahead of this step's MFMAs
      mma_step(ks & 1);
    }
    if (kt + 1 < nk) wait_vmem();  // this wave's loads of the next stage have landed
    lds_barrier();
  }
  if (nk > 0) mma_step(1);

  // output segment of the tile (constant indices: an argument array indexed
  // at run time would be copied to scratch)
  float* out = p.out[0];
  int64_t nc0 = n0;
  if (p.nseg > 1 && n0 >= p.seg_end[0]) {
    out = p.out[1];
    nc0 = n0 - p.seg_end[0];
  }
  if (p.nseg > 2 && n0 >= p.seg_end[1]) {
    out = p.out[2];
    nc0 = n0 - p.seg_end[1];
  }
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (pass) lds_barrier();  // the previous pass is done with Cs
    if (wm == pass) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              Cs[(mt * 32 + 8 * i + 4 * h + j) * SC + wn * 64 + nt * 32 + r] = acc[mt][nt][4 * i + j];
    }
    lds_barrier();
    const int64_t mr0 = m0 + pass * (BIG / 2);  // first output row of the pass
    constexpr int ROWS = BIG / 2;
    if (p.part && p.ksplit < p.K) {
      // fixed-order reduction: this split's tile goes to part[split]
      float* dst = p.part + split * p.M * p.N;
      for (int c = tid; c < ROWS * BIG / 4; c += BIG_THREADS) {
        const int row = c / (BIG / 4), col = (c % (BIG / 4)) * 4;
        *reinterpret_cast<f32x4*>(dst + (mr0 + row) * p.N + (n0 + col)) =
            *reinterpret_cast<const f32x4*>(Cs + row * SC + col);
      }
    } else if (p.ldn == 1 && p.ksplit >= p.K && (p.ldm & 3) == 0) {
      // one k split: the only writer of its tile in this launch
      for (int c = tid; c < ROWS * BIG / 4; c += BIG_THREADS) {
        const int row = c / (BIG / 4), col = (c % (BIG / 4)) * 4;
        f32x4* o = reinterpret_cast<f32x4*>(out + (mr0 + row) * p.ldm + (nc0 + col));
        *o += *reinterpret_cast<const f32x4*>(Cs + row * SC + col);
      }
    } else if (p.ldn == 1) {
      for (int c = tid; c < ROWS * BIG; c += BIG_THREADS) {
        const int row = c / BIG, col = c % BIG;
        atomicAdd(out + (mr0 + row) * p.ldm + (nc0 + col), Cs[row * SC + col]);
      }
    } else {
      for (int c = tid; c < ROWS * BIG; c += BIG_THREADS) {
        const int col = c / ROWS, row = c % ROWS;
        atomicAdd(out + (mr0 + row) * p.ldm + (nc0 + col) * p.ldn, Cs[row * SC + col]);
      }
    }
  }
}

// out (+)= sum over the nsplit partial tiles part[s][M][N], s = 0, 1, ... in
// that order (one thread per output element; the output addressing and
// segments are those of the TN GEMM).
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GemmTN<T> p, int64_t nsplit) {
  const int64_t total = p.M * p.N;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    // n fastest when the output's n stride is 1, else m fastest (coalesced stores)
    const int64_t m = p.ldn == 1 ? idx / p.N : idx % p.M;
    const int64_t n = p.ldn == 1 ? idx % p.N : idx / p.M;
    float acc = 0.f;
    for (int64_t sp = 0; sp < nsplit; ++sp) acc += p.part[sp * total + m * p.N + n];
    int seg = 0;
    while (seg + 1 < p.nseg && n >= p.seg_end[seg]) ++seg;
    const int64_t nc = n - (seg ? p.seg_end[seg - 1] : 0);
    p.out[seg][m * p.ldm + nc * p.ldn] += acc;
  }
}

}  // namespace

template <typename T>
hipError_t launch_gemm_nt(const GemmNT<T>& p, int epi, int bn, hipStream_t s) {
  const int64_t mt = (epi == EPI_HEADS ? p.Np : p.M + BM - 1) / BM;
  const int64_t grid = mt * (p.N / bn);
  if (grid <= 0) return hipSuccess;
  // the k loop reads whole k tiles and clamps rows to M-1
  const int bk = (epi == EPI_ACCUM ? nt_kb<EPI_ACCUM>() : nt_kb<EPI_HEADS>()) / (int)sizeof(T);
  if (p.M <= 0 || p.K <= 0 || p.K % bk) return hipErrorInvalidValue;
  if (p.a_kblk <= 0 || p.a_kblk % bk) return hipErrorInvalidValue;  // A's k blocks hold whole k tiles
  if ((epi == EPI_GLU || epi == EPI_GLU_BWD) && (bn != 128 || p.N % 128 || p.glu.ldf % 64))
    return hipErrorInvalidValue;
  if ((epi == EPI_CE || epi == EPI_CE_BWD) && (bn != 128 || p.N % 128)) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 2) {
    // bf16 products with 256-wide N tiles and one B operand (or the gated
    // pair): 256 x 256 tiles, when there are enough of them to fill the chip
    const bool big_epi = epi == EPI_STORE || epi == EPI_GLU || epi == EPI_GLU_BWD || epi == EPI_CE || epi == EPI_CE_BWD;
    const int64_t big_tiles = ((p.M + BIG - 1) / BIG) * (p.N / BIG);
    if (big_epi && p.N % BIG == 0 && p.nseg == 1 && p.K % BIG_BK == 0 && p.a_kblk % BIG_BK == 0 &&
        (epi != EPI_GLU || p.glu.ldf % (BIG / 2) == 0) && big_tiles >= 256) {
      const dim3 g((unsigned)(((p.M + BIG - 1) / BIG) * (p.N / BIG)));
      if (epi == EPI_STORE)
        hipLaunchKernelGGL((gemm_nt_big_kernel<EPI_STORE>), g, dim3(BIG_THREADS), 0, s, p);
      else if (epi == EPI_GLU)
        hipLaunchKernelGGL((gemm_nt_big_kernel<EPI_GLU>), g, dim3(BIG_THREADS), 0, s, p);
      else if (epi == EPI_GLU_BWD)
        hipLaunchKernelGGL((gemm_nt_big_kernel<EPI_GLU_BWD>), g, dim3(BIG_THREADS), 0, s, p);
      else if (epi == EPI_CE)
        hipLaunchKernelGGL((gemm_nt_big_kernel<EPI_CE>), g, dim3(BIG_THREADS), 0, s, p);
      else
        hipLaunchKernelGGL((gemm_nt_big_kernel<EPI_CE_BWD>), g, dim3(BIG_THREADS), 0, s, p);
      return hipGetLastError();
    }
  }
  if (epi == EPI_CE)
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, EPI_CE>), dim3(grid), dim3(NTHREADS), 0, s, p);
  else if (epi == EPI_CE_BWD)
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, EPI_CE_BWD>), dim3(grid), dim3(NTHREADS), 0, s, p);
  else
  if (epi == EPI_STORE && bn == 128)
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, EPI_STORE>), dim3(grid), dim3(NTHREADS), 0, s, p);
  else if (epi == EPI_GLU)
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, EPI_GLU>), dim3(grid), dim3(NTHREADS), 0, s, p);
  else if (epi == EPI_GLU_BWD)
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, EPI_GLU_BWD>), dim3(grid), dim3(NTHREADS), 0, s, p);
  else if (epi == EPI_ACCUM && bn == 128)
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, EPI_ACCUM>), dim3(grid), dim3(NTHREADS), 0, s, p);
  else if (epi == EPI_ACCUM && bn == 64)
    hipLaunchKernelGGL((gemm_nt_kernel<T, 64, EPI_ACCUM>), dim3(grid), dim3(NTHREADS), 0, s, p);
  else if (epi == EPI_HEADS && bn == 128)
    hipLaunchKernelGGL((gemm_nt_kernel<T, 128, EPI_HEADS>), dim3(grid), dim3(NTHREADS), 0, s, p);
  else if (epi == EPI_HEADS && bn == 64)
    hipLaunchKernelGGL((gemm_nt_kernel<T, 64, EPI_HEADS>), dim3(grid), dim3(NTHREADS), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemm_tn(const GemmTN<T>& p, int bn, hipStream_t s) {
  // whole tiles along M and N; every split holds at least one k row
  if (p.K <= 0 || p.ksplit <= 0 || p.M <= 0 || p.M % BM || bn <= 0 || p.N <= 0 || p.N % bn) return hipErrorInvalidValue;
  const int64_t nsplit = (p.K + p.ksplit - 1) / p.ksplit;
  bool big = false;
  if constexpr (sizeof(T) == 2) {
    // 256 x 256 tiles when the shapes hold whole tiles and k tiles of 64
    // tokens, no 128-column half straddles a B block or an output segment,
    // and there are enough tiles to fill the chip
    big = p.M % BIG == 0 && p.N % BIG == 0 && p.K % BIG_BK == 0 && p.ksplit % BIG_BK == 0 && p.b_nblk % 128 == 0 &&
          (p.M / BIG) * (p.N / BIG) * nsplit >= 256;
    for (int sg = 0; sg < p.nseg; ++sg) big = big && p.seg_end[sg] % BIG == 0;
    if (big) {
      const dim3 g((unsigned)((p.M / BIG) * (p.N / BIG) * nsplit));
      hipLaunchKernelGGL((gemm_tn_big_kernel<0>), g, dim3(BIG_THREADS), 0, s, p);
    }
  }
  if (!big) {
  const dim3 grid((unsigned)((p.M / BM) * (p.N / bn) * nsplit));
  if (bn == 128)
    hipLaunchKernelGGL((gemm_tn_kernel<T, 128>), grid, dim3(NTHREADS), 0, s, p);
  else if (bn == 64)
    hipLaunchKernelGGL((gemm_tn_kernel<T, 64>), grid, dim3(NTHREADS), 0, s, p);
  else
    return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.part || nsplit < 2) return e;
  int64_t blocks = (p.M * p.N + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL((splitk_reduce_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, s, p, nsplit);
  return hipGetLastError();
}

template hipError_t launch_gemm_nt<bf16>(const GemmNT<bf16>&, int, int, hipStream_t);
template hipError_t launch_gemm_nt<float>(const GemmNT<float>&, int, int, hipStream_t);
template hipError_t launch_gemm_tn<bf16>(const GemmTN<bf16>&, int, hipStream_t);
template hipError_t launch_gemm_tn<float>(const GemmTN<float>&, int, hipStream_t);

}  // namespace upipe
