// Causal GQA flash-attention backward for one chunk of heads on gfx950.
//
// Backward recomputes P from Q, K and the saved log-sum-exp instead of
// keeping any per-head activation from the forward (activation
// checkpointing applied inside the op: "Road to 5 Million Tokens",
// transcript, activation-checkpointing part; the chunk's activations are
// "recomputed", memeeeeeex.com article, section "Untied Ulysses (UPipe) —
// head 単位のチャンク化").
//
// One workgroup owns 128 keys of one kv head (4 waves x 32 keys) and walks
// the query tiles at or after its keys for every q head of the chunk that
// reads this kv head, so dK and dV sum over the GQA group in registers:
//   S  = Q K^T,  dP = dO V^T             (rows q, one key per lane)
//   P  = exp(S/sqrt(d) - LSE),  dS = P (dP - Delta) / sqrt(d)
//   dV^T += dO^T P,  dK^T += Q^T dS       (P and dS feed MFMA from registers)
//   dQ  += dS K                           (dS staged through LDS, fp32 atomics)
// Q and dO tiles are staged in LDS both row-major and transposed (written
// transposed on the way in), and K^T for the whole key block is built in LDS
// once. The next query tile is prefetched through registers.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace upipe {

namespace {

constexpr int BKEY = 128;
constexpr int NTHREADS = 256;

template <typename T, int D>
struct BwdGeo {
  static constexpr int BQ = (sizeof(T) == 4 && D == 128) ? 32 : 64;
  static constexpr int NQB = BQ / 32;
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int SQ = lds_stride<T>(D);      // [BQ][D] tiles
  static constexpr int SQT = lds_stride<T>(BQ);    // [D][BQ] tiles
  static constexpr int SDS = lds_stride<T>(BKEY);  // dS [BQ][BKEY]
  static constexpr int SKT = lds_stride<T>(BKEY);  // K^T [D][BKEY]
  static constexpr int Q_OFF = 0;
  static constexpr int QT_OFF = Q_OFF + BQ * SQ;
  static constexpr int DO_OFF = QT_OFF + D * SQT;
  static constexpr int DOT_OFF = DO_OFF + BQ * SQ;
  static constexpr int DS_OFF = DOT_OFF + D * SQT;
  static constexpr int KT_OFF = DS_OFF + BQ * SDS;
  static constexpr int T_ELEMS = KT_OFF + D * SKT;
  // prefetch units: (row pair, 16-byte column chunk)
  static constexpr int UNITS = (BQ / 2) * (D / VEC);
  static constexpr int PER = UNITS / NTHREADS;
  static_assert(UNITS % NTHREADS == 0, "tile units");
};

template <typename T> DEV void st_pair2(T* p, float a, float b);
template <> DEV void st_pair2<bf16>(bf16* p, float a, float b) {
  *reinterpret_cast<bf16x2*>(p) = (bf16x2){(bf16)a, (bf16)b};
}
template <> DEV void st_pair2<float>(float* p, float a, float b) {
  *reinterpret_cast<f32x2*>(p) = (f32x2){a, b};
}

// Raw 16-byte chunks of rows (2*pr, 2*pr+1), column chunk cc, of a [rows][D] tensor.
template <typename T, int D>
DEV void load_rows(const T* base, int64_t row0, u32x4 (&r)[BwdGeo<T, D>::PER][2]) {
  using G = BwdGeo<T, D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < G::PER; ++i) {
    const int u = tid + i * NTHREADS;
    const int pr = u % (G::BQ / 2), cc = u / (G::BQ / 2);
#pragma unroll
    for (int t = 0; t < 2; ++t) r[i][t] = ld_raw16(base + (row0 + 2 * pr + t) * D + cc * G::VEC);
  }
}

template <typename T>
DEV float lane_elem(const u32x4& v, int e) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t wd = v[e >> 1];
    const uint32_t bits = (e & 1) ? (wd & 0xFFFF0000u) : (wd << 16);
    return __uint_as_float(bits);
  } else {
    return __uint_as_float(v[e]);
  }
}

// Store a prefetched tile row-major into S[BQ][SQ] and transposed into ST[D][SQT].
template <typename T, int D>
DEV void store_rows(T* S, T* ST, const u32x4 (&r)[BwdGeo<T, D>::PER][2]) {
  using G = BwdGeo<T, D>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < G::PER; ++i) {
    const int u = tid + i * NTHREADS;
    const int pr = u % (G::BQ / 2), cc = u / (G::BQ / 2);
#pragma unroll
    for (int t = 0; t < 2; ++t) st_raw16(S + (2 * pr + t) * G::SQ + cc * G::VEC, r[i][t]);
#pragma unroll
    for (int e = 0; e < G::VEC; ++e)
      st_pair2<T>(ST + (cc * G::VEC + e) * G::SQT + 2 * pr, lane_elem<T>(r[i][0], e), lane_elem<T>(r[i][1], e));
  }
}

template <typename T, int D>
__global__ __launch_bounds__(NTHREADS) void attn_bwd_kernel(const AttnBwd<T> p) {
  using G = BwdGeo<T, D>;
  constexpr int BQ = G::BQ, NQB = G::NQB, ND = D / 32, NS = D / 16;
  extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
  T* sm = reinterpret_cast<T*>(dyn_smem);
  T* Qs = sm + G::Q_OFF;
  T* QTs = sm + G::QT_OFF;
  T* dOs = sm + G::DO_OFF;
  T* dOTs = sm + G::DOT_OFF;
  T* dSs = sm + G::DS_OFF;
  T* KTs = sm + G::KT_OFF;
  float* lse_s = reinterpret_cast<float*>(sm + G::T_ELEMS);
  float* del_s = lse_s + BQ;

  const int l = lane_id(), r = l & 31, h = l >> 5;
  const int w = wave_id();
  const int tid = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * BKEY;  // block 0 has the most query tiles
  const int64_t kw = k0 + w * 32 + r;             // this lane's key

  // K^T of the whole key block into LDS (transposed on the way in).
  {
    constexpr int KU = (BKEY / 2) * (D / G::VEC);
    for (int u = tid; u < KU; u += NTHREADS) {
      const int pr = u % (BKEY / 2), cc = u / (BKEY / 2);
      const u32x4 a = ld_raw16(p.k + (k0 + 2 * pr) * D + cc * G::VEC);
      const u32x4 b = ld_raw16(p.k + (k0 + 2 * pr + 1) * D + cc * G::VEC);
#pragma unroll
      for (int e = 0; e < G::VEC; ++e)
        st_pair2<T>(KTs + (cc * G::VEC + e) * G::SKT + 2 * pr, lane_elem<T>(a, e), lane_elem<T>(b, e));
    }
  }
  // K and V of this lane's key as B operands (k = head dim).
  Frag<T> kf[NS], vf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kf[s] = ld_frag(p.k + kw * D + s * 16 + 8 * h);
    vf[s] = ld_frag(p.v + kw * D + s * 16 + 8 * h);
  }
  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    dk[j] = zero16();
    dv[j] = zero16();
  }

  const int64_t qend = ((p.N + BQ - 1) / BQ) * BQ;
  const int64_t nqt = (qend - k0) / BQ;  // k0 is a multiple of BQ
  const int64_t total = nqt * p.nh;

  u32x4 rq[G::PER][2], rdo[G::PER][2];
  float rl = 0.f, rd = 0.f;
  auto prefetch = [&](int64_t it) {
    const int hh = (int)(it / nqt);
    const int64_t q0 = k0 + (it % nqt) * BQ;
    load_rows<T, D>(p.q + (int64_t)hh * p.Np * D, q0, rq);
    load_rows<T, D>(p.dout + (int64_t)hh * p.Np * D, q0, rdo);
    if (tid < BQ) {
      const int64_t q = q0 + tid;
      rl = (q < p.N) ? p.lse[(int64_t)hh * p.lse_stride + q] * 1.4426950408889634f : 0.f;
      rd = (q < p.N) ? p.delta[(int64_t)hh * p.Np + q] : 0.f;
    }
  };
  auto commit = [&]() {
    store_rows<T, D>(Qs, QTs, rq);
    store_rows<T, D>(dOs, dOTs, rdo);
    if (tid < BQ) {
      lse_s[tid] = rl;
      del_s[tid] = rd;
    }
  };

  if (total > 0) {
    prefetch(0);
    commit();
  }
  __syncthreads();

  for (int64_t it = 0; it < total; ++it) {
    const int hh = (int)(it / nqt);
    const int64_t q0 = k0 + (it % nqt) * BQ;
    if (it + 1 < total) prefetch(it + 1);

    f32x16 sacc[NQB], dpacc[NQB];
#pragma unroll
    for (int t = 0; t < NQB; ++t) {
      sacc[t] = zero16();
      dpacc[t] = zero16();
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int t = 0; t < NQB; ++t) {
        const Frag<T> aq = ld_frag(Qs + (t * 32 + r) * G::SQ + s * 16 + 8 * h);
        mma(sacc[t], aq, kf[s]);
        const Frag<T> ad = ld_frag(dOs + (t * 32 + r) * G::SQ + s * 16 + 8 * h);
        mma(dpacc[t], ad, vf[s]);
      }
    // P and dS in place (rows q, column = this lane's key)
#pragma unroll
    for (int t = 0; t < NQB; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int qr = t * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        const int64_t q = q0 + qr;
        const bool valid = (kw <= q) && (q < p.N);
        const float pe = valid ? fast_exp2(sacc[t][e] * p.scale_log2 - lse_s[qr]) : 0.f;
        sacc[t][e] = pe;
        dpacc[t][e] = pe * (dpacc[t][e] - del_s[qr]) * p.scale;
      }
    // dV^T += dO^T P ; dK^T += Q^T dS  (contraction over the tile's queries)
#pragma unroll
    for (int t = 0; t < NQB; ++t)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const Frag<T> pb = frag_from_acc<T>(sacc[t], s2, 1.0f);
        const Frag<T> sb = frag_from_acc<T>(dpacc[t], s2, 1.0f);
#pragma unroll
        for (int j = 0; j < ND; ++j) {
          const int off = (j * 32 + r) * G::SQT + t * 32 + 16 * s2 + 4 * h;
          const Frag<T> ado = ld_frag2(dOTs + off, dOTs + off + 8);
          mma(dv[j], ado, pb);
          const Frag<T> aq = ld_frag2(QTs + off, QTs + off + 8);
          mma(dk[j], aq, sb);
        }
      }
    // dS -> LDS [q][key]
#pragma unroll
    for (int t = 0; t < NQB; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        dSs[(t * 32 + 8 * (e >> 2) + 4 * h + (e & 3)) * G::SDS + w * 32 + r] = from_f<T>(dpacc[t][e]);
    __syncthreads();
    if (it + 1 < total) commit();
    // dQ[q][d] += sum over the block's 128 keys of dS[q][key] K[key][d]
    {
      constexpr int TILES = NQB * ND;
      float* dqh = p.dq_acc + (int64_t)hh * p.Np * D;
      for (int ti = w; ti < TILES; ti += 4) {
        const int qt = ti % NQB, jd = ti / NQB;
        f32x16 acc = zero16();
#pragma unroll
        for (int s = 0; s < BKEY / 16; ++s) {
          const Frag<T> a = ld_frag(dSs + (qt * 32 + r) * G::SDS + s * 16 + 8 * h);
          const Frag<T> b = ld_frag(KTs + (jd * 32 + r) * G::SKT + s * 16 + 8 * h);
          mma(acc, a, b);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t q = q0 + qt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
          if (q < p.N) atomicAdd(dqh + q * D + jd * 32 + r, acc[e]);
        }
      }
    }
    __syncthreads();
  }

  // dK, dV rows of this lane's key: C tiles hold rows = head dim.
#pragma unroll
  for (int j = 0; j < ND; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dd = j * 32 + 8 * i + 4 * h;
      f32x4 vk = (f32x4){dk[j][4 * i], dk[j][4 * i + 1], dk[j][4 * i + 2], dk[j][4 * i + 3]};
      f32x4 vv = (f32x4){dv[j][4 * i], dv[j][4 * i + 1], dv[j][4 * i + 2], dv[j][4 * i + 3]};
      f32x4* pk = reinterpret_cast<f32x4*>(p.dk_acc + kw * D + dd);
      f32x4* pv = reinterpret_cast<f32x4*>(p.dv_acc + kw * D + dd);
      if (p.accumulate) {
        vk += *pk;
        vv += *pv;
      }
      *pk = vk;
      *pv = vv;
    }
}

template <typename T, int D>
hipError_t launch_bwd_d(const AttnBwd<T>& p, hipStream_t s) {
  using G = BwdGeo<T, D>;
  const size_t smem = (size_t)G::T_ELEMS * sizeof(T) + 2 * G::BQ * sizeof(float);
  const dim3 grid((unsigned)((p.N + BKEY - 1) / BKEY));
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_kernel<T, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_kernel<T, D>), grid, dim3(NTHREADS), smem, s, p);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_attn_bwd(const AttnBwd<T>& p, int head_dim, hipStream_t s) {
  if (head_dim == 64) return launch_bwd_d<T, 64>(p, s);
  if (head_dim == 128) return launch_bwd_d<T, 128>(p, s);
  return hipErrorInvalidValue;
}

template hipError_t launch_attn_bwd<bf16>(const AttnBwd<bf16>&, int, hipStream_t);
template hipError_t launch_attn_bwd<float>(const AttnBwd<float>&, int, hipStream_t);

}  // namespace upipe
