// Causal GQA flash-attention forward for one chunk of heads on gfx950.
//
// The chunk's heads each attend over the whole sequence (one GPU computes
// full-sequence attention for the heads it owns, then the next chunk reuses
// the buffers: "500 万トークンへの道 — Max Ryabinin (Together AI) の Untied
// Ulysses", section "Untied Ulysses (UPipe) — head 単位のチャンク化").
//
// Orientation: each wave computes S^T = K Q^T for its queries, so a lane owns
// one query column and 16 keys of each 32x32 tile. Row statistics of the
// softmax are then an in-lane reduction plus one exchange between the two
// half-waves, and P^T feeds O^T = V^T P^T straight from the accumulators
// (see common.h). q arrives multiplied by log2(e)/sqrt(d), so S is already
// the exponent in log2 units. K and V tiles are row-major copies [key][d] in
// LDS, double buffered: bf16 tiles arrive one tile ahead by direct
// global -> LDS loads, fp32 tiles through registers; V^T operands are column
// reads (LDS transpose reads).
//
// Workgroup: 8 waves x (32*NQT) query rows (two waves per SIMD). `hp` heads
// of the same kv head are packed per workgroup (GQA): the K/V tile in LDS then
// serves hp heads.
// Mode 0 (training forward): online softmax; writes O and LSE.
// Mode 1 (backward recompute): LSE is given; writes O and
//   Delta_i = dO_i . O_i (with the backward's pre-scaled dO), the row term of
//   the softmax backward.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace upipe {

namespace {

constexpr int BC = 64;  // keys per tile

template <typename T, int D>
struct FwdGeo {
  static constexpr int NW = 8;                 // waves per workgroup (2 per SIMD)
  static constexpr int NTHREADS = 64 * NW;
  static constexpr int NQT = 1;                // 32-query tiles per wave
  static constexpr int ROWS_W = 32 * NQT;
  using L = Tile<T, D>;                          // K and V tiles [key][d]
  static constexpr int K_ELEMS = L::ELEMS(BC);
  static constexpr int V_ELEMS = L::ELEMS(BC);
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int KCH = BC * D / VEC / NTHREADS;  // 16-byte chunks per thread (K)
  static_assert((BC * D / VEC) % NTHREADS == 0, "tile chunks");
  static constexpr int VCH = KCH;                      // (V)
};

template <typename T, int D>
DEV void load_kv(const AttnFwd<T>& p, int64_t k0, u32x4 (&rk)[FwdGeo<T, D>::KCH],
                 u32x4 (&rv)[FwdGeo<T, D>::VCH]) {
  using G = FwdGeo<T, D>;
  const int tid = threadIdx.x;
  constexpr int KC_ROW = D / G::VEC;
#pragma unroll
  for (int i = 0; i < G::KCH; ++i) {
    const int c = tid + i * G::NTHREADS;
    rk[i] = ld_raw16(p.k + (k0 + c / KC_ROW) * D + (c % KC_ROW) * G::VEC);
    rv[i] = ld_raw16(p.v + (k0 + c / KC_ROW) * D + (c % KC_ROW) * G::VEC);
  }
}

template <typename T, int D>
DEV void store_kv(T* stage, const u32x4 (&rk)[FwdGeo<T, D>::KCH], const u32x4 (&rv)[FwdGeo<T, D>::VCH]) {
  using G = FwdGeo<T, D>;
  const int tid = threadIdx.x;
  constexpr int KC_ROW = D / G::VEC;
  T* Ks = stage;
  T* Vs = stage + G::K_ELEMS;
#pragma unroll
  for (int i = 0; i < G::KCH; ++i) {
    const int c = tid + i * G::NTHREADS;
    st_raw16(Ks + G::L::idx(c / KC_ROW, (c % KC_ROW) * G::VEC), rk[i]);
    st_raw16(Vs + G::L::idx(c / KC_ROW, (c % KC_ROW) * G::VEC), rv[i]);
  }
}

// Issue the K and V tile starting at key k0 into an LDS stage with direct
// global -> LDS loads (bf16): each wave moves its share of the rows.
template <typename T, int D>
DEV void dma_kv(const AttnFwd<T>& p, int64_t k0, T* stage) {
  using G = FwdGeo<T, D>;
  using L = typename G::L;
  constexpr int ROWS_PER_INST = 1024 / L::ROW_BYTES;
  constexpr int INST = BC / ROWS_PER_INST;  // per tensor
  const int w = wave_id();
  for (int i = w; i < INST; i += G::NW) {
    dma_tile_rows<L>(p.k + k0 * D, D, stage, i * ROWS_PER_INST);
    dma_tile_rows<L>(p.v + k0 * D, D, stage + G::K_ELEMS, i * ROWS_PER_INST);
  }
}

template <typename T, int D, int MODE>
__global__ __launch_bounds__((FwdGeo<T, D>::NTHREADS)) void attn_fwd_kernel(const AttnFwd<T> p, int hp) {
  using G = FwdGeo<T, D>;
  constexpr int NQT = G::NQT, ND = D / 32, NS = D / 16;
  __shared__ __attribute__((aligned(16))) T smem[2 * G::STAGE];

  const int l = lane_id(), r = l & 31, h = l >> 5;
  const int w = wave_id();
  const int qb_rows = G::NW * G::ROWS_W / hp;  // query positions per workgroup
  const int64_t nqb = p.Np / qb_rows;
  const int64_t qb = nqb - 1 - (int64_t)blockIdx.x;  // longest rows first
  const int hh = (int)blockIdx.y * hp + (w % hp);
  const int64_t qs = qb * qb_rows;
  const int64_t q0w = qs + (int64_t)(w / hp) * G::ROWS_W;

  // Q^T as B operands, resident for the whole key loop.
  const T* qh = p.q + (int64_t)hh * p.Np * D;
  Frag<T> qf[NQT][NS];
#pragma unroll
  for (int t = 0; t < NQT; ++t)
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[t][s] = ld_frag(qh + (q0w + t * 32 + r) * D + s * 16 + 8 * h);

  float m_run[NQT], l_run[NQT], base_row[NQT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
    base_row[t] = 0.f;
    if constexpr (MODE == 1) {
      const int64_t q = q0w + t * 32 + r;
      base_row[t] = (q < p.N) ? p.lse[(int64_t)hh * p.lse_stride + q] * 1.4426950408889634f : 0.f;
    }
  }
  f32x16 oacc[NQT][ND];
#pragma unroll
  for (int t = 0; t < NQT; ++t)
#pragma unroll
    for (int j = 0; j < ND; ++j) oacc[t][j] = zero16();

  const int64_t ntiles = (qs + qb_rows) / BC;
  constexpr bool DMA = G::L::SWZ;  // bf16: direct global -> LDS loads
  u32x4 rk[DMA ? 1 : G::KCH], rv[DMA ? 1 : G::VCH];
  if constexpr (DMA) {
    dma_kv<T, D>(p, 0, smem);
    wait_vmem();
  } else {
    load_kv<T, D>(p, 0, rk, rv);
    store_kv<T, D>(smem, rk, rv);
  }
  lds_barrier();

  // bf16: P is packed straight into MFMA operands and its row sum taken with
  // dot2 on the packed pairs (the sum of exactly the values that multiply V).
  // The softmax base moves only when a lane's row sum leaves [0, 2^16] (or is
  // not finite, as on the first tile where the base is -inf): then the row
  // max of the tile becomes the base and O, l are rescaled. Every P stays
  // <= 2^16, and O / l and LSE = base + log2(l) do not depend on the base.
  constexpr float P_LIMIT = 65536.f;
  // bf16: every S^T chain starts from init = splat(-base), base = the LSE in
  // the recompute, the running softmax base in the forward
  float base = 0.f;
  bool have_base = MODE == 1;
  f32x16 init;
#pragma unroll
  for (int e = 0; e < 16; ++e) init[e] = (MODE == 1) ? -base_row[0] : 0.f;
  if constexpr (MODE == 1) base = base_row[0];
  // bf16: lane offsets of the V^T column reads, computed once
  Col4Plan<typename G::L, ND> vplan;
  if constexpr (sizeof(T) == 2) vplan.init();
  auto step = [&](auto bc, int64_t kt_i) {
    constexpr int buf = decltype(bc)::value;  // LDS stage (immediate offsets)
    const int64_t k0 = kt_i * BC;
    if (kt_i + 1 < ntiles) {
      if constexpr (DMA)
        dma_kv<T, D>(p, k0 + BC, smem + (buf ^ 1) * G::STAGE);
      else
        load_kv<T, D>(p, k0 + BC, rk, rv);
    }
    const T* Ks = smem + buf * G::STAGE;
    const T* Vs = Ks + G::K_ELEMS;

    if constexpr (sizeof(T) == 2) {
      if (k0 <= q0w + G::ROWS_W - 1) {  // some key of the tile is visible to this wave
        // S^T of both 32-key halves (two independent chains), each chain
        // started from the splat of -base, so it holds S - base (log2 units);
        // then softmax and P V half by half.
        // The K fragments of step s + 1 are read before the MFMAs of step s
        // issue, so their LDS latency overlaps those MFMAs.
        f32x16 sacc2[2];
        Frag<T> kf[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) kf[0][kt] = ld_frag(Ks + G::L::idx(kt * 32 + r, 8 * h));
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s + 1 < NS)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) kf[(s + 1) & 1][kt] = ld_frag(Ks + G::L::idx(kt * 32 + r, (s + 1) * 16 + 8 * h));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            if (s == 0)
              sacc2[kt] = mma_first(kf[0][kt], qf[0][0], init);
            else
              mma(sacc2[kt], kf[s & 1][kt], qf[0][s]);
          }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          f32x16& sacc = sacc2[kt];
          // V^T fragments of the P V products below. The training forward
          // reads the first two before its softmax, whose VALU work (row sums,
          // base checks) then covers their latency
          auto vfrag = [&](int t) {
            const T* Vr = Vs + (kt * 32 + 16 * (t / ND)) * G::L::STRIDE;
            return frag_from_col4<T>(ld_col4_at(Vr, vplan.off[0][t % ND]), ld_col4_at(Vr, vplan.off[1][t % ND]));
          };
          Frag<T> vf[3];
          if constexpr (MODE == 0) {
            vf[0] = vfrag(0);
            vf[1] = vfrag(1);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (k0 + kt * 32 + 31 > q0w) {  // the half crosses this wave's diagonal
            const int qrel = (int)(q0w - k0) + r - kt * 32;  // query minus the half's first key
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (8 * (e >> 2) + 4 * h + (e & 3) > qrel) sacc[e] = -INFINITY;
          }
          // P = exp2(S - base) packed as MFMA operands; returns the lane's row sum
          Frag<T> pf[2];
          auto make_p = [&](float shift) {
            const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
            float ps[2] = {0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
              for (int e = 0; e < 8; e += 2) {
                const float x0 = fast_exp2(sacc[8 * s2 + e] - shift);
                const float x1 = fast_exp2(sacc[8 * s2 + e + 1] - shift);
                const bf16x2 pr = {(bf16)x0, (bf16)x1};
                pf[s2].v[e] = pr[0];
                pf[s2].v[e + 1] = pr[1];
                if constexpr (MODE == 0) ps[(e >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps[(e >> 1) & 1], false);
              }
            return ps[0] + ps[1];
          };
          auto make_p0 = [&]() {  // shift 0: no subtraction
            const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
            float ps[2] = {0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
              for (int e = 0; e < 8; e += 2) {
                const bf16x2 pr = {(bf16)fast_exp2(sacc[8 * s2 + e]), (bf16)fast_exp2(sacc[8 * s2 + e + 1])};
                pf[s2].v[e] = pr[0];
                pf[s2].v[e + 1] = pr[1];
                if constexpr (MODE == 0) ps[(e >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ps[(e >> 1) & 1], false);
              }
            return ps[0] + ps[1];
          };
          if constexpr (MODE == 0) {
            // The base moves only when a lane's row sum leaves [0, 2^16] (or is not
            // finite), and on the first half: then the row max becomes the base and
            // O and l are rescaled. Every P stays <= 2^16; O / l and
            // LSE = base + log2(l) do not depend on the base.
            float psum = have_base ? make_p0() : 0.f;
            if (!have_base || __builtin_amdgcn_ballot_w64(!(psum <= P_LIMIT))) {
              float mx = -INFINITY;
#pragma unroll
              for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
              // the first half holds key 0, visible to every query: m_new is finite
              const float m_new = fmaxf(m_run[0], wave_max_pair(mx) + base);
              const float alpha = fast_exp2(m_run[0] - m_new);
              l_run[0] *= alpha;
#pragma unroll
              for (int j = 0; j < ND; ++j) oacc[0][j] *= alpha;
              psum = make_p(m_new - base);
              // the other half's chain already ran against the old base
              if (kt == 0) {
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc2[1][e] -= m_new - base;
              }
              m_run[0] = m_new;
              base = m_new;
#pragma unroll
              for (int e = 0; e < 16; ++e) init[e] = -base;
              have_base = true;
            }
            l_run[0] += psum;
          } else {
            make_p0();
          }
          // O^T += V^T P^T over the half's keys (rows kt*32 + 16*s2 + ... of V):
          // 2*ND products t = (s2, j). In the recompute the V^T fragment of
          // product t + 2 is read before product t issues; the training
          // forward, where that ring was slower, reads the rest in the
          // compiler's order.
          if constexpr (MODE == 1) {
            vf[0] = vfrag(0);
            vf[1] = vfrag(1);
#pragma unroll
            for (int t = 0; t < 2 * ND; ++t) {
              if (t + 2 < 2 * ND) vf[(t + 2) % 3] = vfrag(t + 2);
              __builtin_amdgcn_sched_barrier(0);
              mma(oacc[0][t % ND], vf[t % 3], pf[t / ND]);
            }
          } else {
#pragma unroll
            for (int t = 0; t < 2 * ND; ++t) mma(oacc[0][t % ND], t < 2 ? vf[t] : vfrag(t), pf[t / ND]);
          }
        }
      }
    } else {
      if (k0 <= q0w + G::ROWS_W - 1) {  // some key of the tile is visible to this wave
        f32x16 sacc[2][NQT];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int t = 0; t < NQT; ++t) sacc[kt][t] = zero16();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const Frag<T> a = ld_frag(Ks + G::L::idx(kt * 32 + r, s * 16 + 8 * h));
#pragma unroll
            for (int t = 0; t < NQT; ++t) mma(sacc[kt][t], a, qf[t][s]);
          }
        }
        if (k0 + BC - 1 > q0w) {  // the tile crosses this wave's diagonal
#pragma unroll
          for (int t = 0; t < NQT; ++t) {
            const int qrel = (int)(q0w - k0) + t * 32 + r;  // query minus tile start
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int e = 0; e < 16; ++e)
                if (kt * 32 + 8 * (e >> 2) + 4 * h + (e & 3) > qrel) sacc[kt][t][e] = -INFINITY;
          }
        }
        Frag<T> pf[2][2][NQT];  // P^T as B operands [key half][16-key step][query tile]
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          if constexpr (MODE == 0) {
            // fp32: lazily moved base, raised when a score exceeds it by more than 2^8
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kt][t][e]);
            mx = wave_max_pair(mx);
            const bool need = mx > m_run[t] + 8.0f;
            if (__builtin_amdgcn_ballot_w64(need)) {
              const float m_new = need ? mx : m_run[t];
              const float alpha = fast_exp2(m_run[t] - m_new);
              m_run[t] = m_new;
              l_run[t] *= alpha;
#pragma unroll
              for (int j = 0; j < ND; ++j) oacc[t][j] *= alpha;
            }
            base_row[t] = m_run[t];
          }
          float psum = 0.f;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float pe = fast_exp2(sacc[kt][t][e] - base_row[t]);
              sacc[kt][t][e] = pe;
              psum += pe;
            }
          l_run[t] += psum;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) pf[kt][s2][t] = frag_from_acc<T>(sacc[kt][t], s2, 1.0f);
        }
        // O^T += V^T P^T
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int row0 = kt * 32 + 16 * s2 + 4 * h;
#pragma unroll
            for (int j = 0; j < ND; ++j) {
              const Frag<T> a = frag_from_col4<T>(ld_col4<typename G::L>(Vs, row0, j * 32),
                                                  ld_col4<typename G::L>(Vs, row0 + 8, j * 32));
#pragma unroll
              for (int t = 0; t < NQT; ++t) mma(oacc[t][j], a, pf[kt][s2][t]);
            }
          }
      }
    }
    if (kt_i + 1 < ntiles) {
      if constexpr (DMA)
        wait_vmem();
      else
        store_kv<T, D>(smem + (buf ^ 1) * G::STAGE, rk, rv);
    }
    lds_barrier();
  };
  for (int64_t kt_i = 0; kt_i < ntiles; kt_i += 2) {
    step(std::integral_constant<int, 0>(), kt_i);
    if (kt_i + 1 < ntiles) step(std::integral_constant<int, 1>(), kt_i + 1);
  }

  // epilogue
  T* oh = p.o + (int64_t)hh * p.Np * D;
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    const int64_t q = q0w + t * 32 + r;
    const float l_tot = l_run[t] + __shfl_xor(l_run[t], 32);
    float scale = 1.f;
    if constexpr (MODE == 0) {
      scale = 1.0f / l_tot;
      if (h == 0 && q < p.N)
        p.lse[(int64_t)hh * p.lse_stride + q] = (m_run[t] + log2f(l_tot)) * 0.6931471805599453f;
    }
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < ND; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dd = j * 32 + 8 * i + 4 * h;
        float v[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) v[jj] = oacc[t][j][4 * i + jj] * scale;
        T* dst = oh + q * D + dd;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<bf16x4*>(dst) = (bf16x4){(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
        } else {
          *reinterpret_cast<f32x4*>(dst) = (f32x4){v[0], v[1], v[2], v[3]};
        }
        if constexpr (MODE == 1) {
          const T* src = p.dout + (int64_t)hh * p.Np * D + q * D + dd;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) dot += v[jj] * to_f<T>(src[jj]);
        }
      }
    if constexpr (MODE == 1) {
      dot += __shfl_xor(dot, 32);
      if (h == 0) p.delta[(int64_t)hh * p.Np + q] = (q < p.N) ? dot : 0.f;
    }
  }
}

template <typename T, int D>
hipError_t launch_fwd_d(const AttnFwd<T>& p, int mode, hipStream_t s) {
  using G = FwdGeo<T, D>;
  int hp = 1;
  while (hp * 2 <= 4 && p.nh % (hp * 2) == 0) hp *= 2;
  const int qb_rows = G::NW * G::ROWS_W / hp;
  const dim3 grid((unsigned)(p.Np / qb_rows), (unsigned)(p.nh / hp));
  if (mode == 0)
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, 0>), grid, dim3(G::NTHREADS), 0, s, p, hp);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, 1>), grid, dim3(G::NTHREADS), 0, s, p, hp);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_attn_fwd(const AttnFwd<T>& p, int head_dim, int mode, hipStream_t s) {
  if (head_dim == 64) return launch_fwd_d<T, 64>(p, mode, s);
  if (head_dim == 128) return launch_fwd_d<T, 128>(p, mode, s);
  return hipErrorInvalidValue;
}

template hipError_t launch_attn_fwd<bf16>(const AttnFwd<bf16>&, int, int, hipStream_t);
template hipError_t launch_attn_fwd<float>(const AttnFwd<float>&, int, int, hipStream_t);

}  // namespace upipe
