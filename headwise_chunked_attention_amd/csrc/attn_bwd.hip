// Causal GQA flash-attention backward for one chunk of heads on gfx950.
//
// Backward recomputes P from Q, K and the saved log-sum-exp instead of
// keeping any per-head activation from the forward (activation
// checkpointing applied inside the op: "Road to 5 Million Tokens",
// transcript, activation-checkpointing part; the chunk's activations are
// "recomputed", memeeeeeex.com article, section "Untied Ulysses (UPipe) —
// head 単位のチャンク化").
//
// One workgroup owns a block of keys of one kv head and walks the query tiles
// at or after its keys for every q head of the chunk that reads this kv head,
// so dK and dV sum over the GQA group in registers:
//   S  = Q K^T,  dP = dO V^T             (rows q, one key per lane)
//   P  = exp(S/sqrt(d) - LSE),  dS = P (dP - Delta) / sqrt(d)
//   dV^T += dO^T P,  dK^T += Q^T dS       (P and dS feed MFMA from registers)
//   dQ  += dS K                           (dS staged through LDS, fp32 atomics)
// Every LDS tile is a row-major copy of global memory (K, V of the key block
// once; Q, dO per query tile, prefetched one tile ahead through registers);
// the transposed operands (dO^T, Q^T, K as a column operand) are read with
// gfx950's LDS transpose reads.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace upipe {

namespace {

// Workgroup geometry: KT x QT waves. Wave w owns key tile w % KT (32 keys)
// and query tile w / KT (32 queries) of each step, so a workgroup covers
// BKEY = 32*KT keys and BQ = 32*QT queries per step. With 8 waves two waves
// share each SIMD and hide each other's LDS and MFMA latency.
template <typename T, int D>
struct BwdGeo {
  static constexpr bool BIG = (sizeof(T) == 4 && D == 128);  // fp32, head_dim 128: smaller block (LDS)
  static constexpr int KT = BIG ? 2 : 4;
  static constexpr int QT = BIG ? 1 : 2;
  static constexpr int NW = KT * QT;
  static constexpr int NT = 64 * NW;
  static constexpr int BKEY = 32 * KT;
  static constexpr int BQ = 32 * QT;
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int SK = lds_stride<T>(D);      // K, V, Q, dO tiles [rows][D]
  static constexpr int SDS = lds_stride<T>(BKEY);  // dS [BQ][BKEY]
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = K_OFF + BKEY * SK;
  static constexpr int Q_OFF = V_OFF + BKEY * SK;
  static constexpr int DO_OFF = Q_OFF + BQ * SK;
  static constexpr int DS_OFF = DO_OFF + BQ * SK;
  static constexpr int T_ELEMS = DS_OFF + BQ * SDS;
  static constexpr int RCH = D / VEC;            // 16-byte chunks per row
  static constexpr int PER = BQ * RCH / NT;      // prefetch chunks per thread and tensor
  static constexpr size_t SMEM = (size_t)T_ELEMS * sizeof(T) + 2 * BQ * sizeof(float);
  // end-of-kernel reduction of the QT partial dK/dV sums per key tile
  static constexpr size_t RED = (size_t)KT * 64 * 16 * (D / 32) * sizeof(float);
  static_assert((BQ * RCH) % NT == 0, "tile chunks");
  static_assert(QT == 1 || RED <= SMEM, "reduction buffer fits in LDS");
};

template <typename T, int D>
DEV void load_tile(const T* base, int64_t row0, u32x4 (&r)[BwdGeo<T, D>::PER]) {
  using G = BwdGeo<T, D>;
#pragma unroll
  for (int i = 0; i < G::PER; ++i) {
    const int c = threadIdx.x + i * G::NT;
    r[i] = ld_raw16(base + (row0 + c / G::RCH) * D + (c % G::RCH) * G::VEC);
  }
}

template <typename T, int D>
DEV void store_tile(T* S, const u32x4 (&r)[BwdGeo<T, D>::PER]) {
  using G = BwdGeo<T, D>;
#pragma unroll
  for (int i = 0; i < G::PER; ++i) {
    const int c = threadIdx.x + i * G::NT;
    st_raw16(S + (c / G::RCH) * G::SK + (c % G::RCH) * G::VEC, r[i]);
  }
}

template <typename T, int D>
__global__ __launch_bounds__((BwdGeo<T, D>::NT)) void attn_bwd_kernel(const AttnBwd<T> p) {
  using G = BwdGeo<T, D>;
  constexpr int BQ = G::BQ, BKEY = G::BKEY, ND = D / 32, NS = D / 16, SK = G::SK;
  extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
  T* sm = reinterpret_cast<T*>(dyn_smem);
  T* Ks = sm + G::K_OFF;
  T* Vs = sm + G::V_OFF;
  T* Qs = sm + G::Q_OFF;
  T* dOs = sm + G::DO_OFF;
  T* dSs = sm + G::DS_OFF;
  float* lse_s = reinterpret_cast<float*>(sm + G::T_ELEMS);
  float* del_s = lse_s + BQ;

  const int l = lane_id(), r = l & 31, h = l >> 5;
  const int w = wave_id();
  const int kt = w % G::KT, qt = w / G::KT;
  const int tid = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * BKEY;  // block 0 has the most query tiles
  const int krel = kt * 32 + r;                   // this lane's key within the block
  const int64_t kw = k0 + krel;

  // K and V of the key block, row-major in LDS.
  for (int c = tid; c < BKEY * G::RCH; c += G::NT) {
    const int row = c / G::RCH, cc = c % G::RCH;
    st_raw16(Ks + row * SK + cc * G::VEC, ld_raw16(p.k + (k0 + row) * D + cc * G::VEC));
    st_raw16(Vs + row * SK + cc * G::VEC, ld_raw16(p.v + (k0 + row) * D + cc * G::VEC));
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

  u32x4 rq[G::PER], rdo[G::PER];
  float rl = 0.f, rd = 0.f;
  auto prefetch = [&](int64_t it) {
    const int hh = (int)(it / nqt);
    const int64_t q0 = k0 + (it % nqt) * BQ;
    load_tile<T, D>(p.q + (int64_t)hh * p.Np * D, q0, rq);
    load_tile<T, D>(p.dout + (int64_t)hh * p.Np * D, q0, rdo);
    if (tid < BQ) {
      const int64_t q = q0 + tid;
      rl = (q < p.N) ? p.lse[(int64_t)hh * p.lse_stride + q] * 1.4426950408889634f : 0.f;
      rd = (q < p.N) ? p.delta[(int64_t)hh * p.Np + q] : 0.f;
    }
  };
  auto commit = [&]() {
    store_tile<T, D>(Qs, rq);
    store_tile<T, D>(dOs, rdo);
    if (tid < BQ) {
      lse_s[tid] = rl;
      del_s[tid] = rd;
    }
  };

  prefetch(0);
  commit();
  lds_barrier();

  for (int64_t it = 0; it < total; ++it) {
    const int hh = (int)(it / nqt);
    const int64_t q0 = k0 + (it % nqt) * BQ;
    if (it + 1 < total) prefetch(it + 1);
    // rows of this wave's query tile, relative to the key block start
    const int qrel0 = (int)(q0 - k0) + qt * 32;
    const int qlim = (int)((p.N - q0 < (int64_t)BQ) ? (p.N - q0) : BQ);  // valid rows of the tile

    // S = Q K^T and dP = dO V^T (rows q of tile qt, lane = key of tile kt)
    f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const Frag<T> kb = ld_frag(Ks + krel * SK + s * 16 + 8 * h);
      const Frag<T> vb = ld_frag(Vs + krel * SK + s * 16 + 8 * h);
      mma(sacc, ld_frag(Qs + (qt * 32 + r) * SK + s * 16 + 8 * h), kb);
      mma(dpacc, ld_frag(dOs + (qt * 32 + r) * SK + s * 16 + 8 * h), vb);
    }
    // P = exp(S/sqrt(d) - LSE), dS = P (dP - Delta) / sqrt(d), in place
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = qt * 32 + 8 * i + 4 * h;  // tile row of accumulator element 4*i
      const f32x4 lv = *reinterpret_cast<const f32x4*>(lse_s + rr);
      const f32x4 dv4 = *reinterpret_cast<const f32x4*>(del_s + rr);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 4 * i + j;
        const bool valid = (krel <= qrel0 + 8 * i + 4 * h + j) && (rr + j < qlim);
        const float pe = valid ? fast_exp2(sacc[e] * p.scale_log2 - lv[j]) : 0.f;
        sacc[e] = pe;
        dpacc[e] = pe * (dpacc[e] - dv4[j]) * p.scale;
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS over this wave's 32 queries: P/dS feed
    // MFMA from the accumulators, dO^T/Q^T are column reads of LDS tiles.
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const Frag<T> pb = frag_from_acc<T>(sacc, s2, 1.0f);
      const Frag<T> sb = frag_from_acc<T>(dpacc, s2, 1.0f);
      const int row0 = qt * 32 + 16 * s2 + 4 * h;
#pragma unroll
      for (int j = 0; j < ND; ++j) {
        const Frag<T> ado = frag_from_col4<T>(ld_col4<T>(dOs, SK, row0, j * 32), ld_col4<T>(dOs, SK, row0 + 8, j * 32));
        mma(dv[j], ado, pb);
        const Frag<T> aq = frag_from_col4<T>(ld_col4<T>(Qs, SK, row0, j * 32), ld_col4<T>(Qs, SK, row0 + 8, j * 32));
        mma(dk[j], aq, sb);
      }
    }
    // dS -> LDS [q][key]
#pragma unroll
    for (int e = 0; e < 16; ++e)
      dSs[(qt * 32 + 8 * (e >> 2) + 4 * h + (e & 3)) * G::SDS + krel] = from_f<T>(dpacc[e]);
    lds_barrier();
    if (it + 1 < total) commit();
    // dQ[q][d] += sum over the block's keys of dS[q][key] K[key][d]
    {
      float* dqh = p.dq_acc + (int64_t)hh * p.Np * D;
      for (int ti = w; ti < G::QT * ND; ti += G::NW) {
        const int tq = ti % G::QT, jd = ti / G::QT;
        f32x16 acc = zero16();
#pragma unroll
        for (int s = 0; s < BKEY / 16; ++s) {
          const Frag<T> a = ld_frag(dSs + (tq * 32 + r) * G::SDS + s * 16 + 8 * h);
          const Frag<T> b = frag_from_col4<T>(ld_col4<T>(Ks, SK, s * 16 + 8 * h, jd * 32),
                                              ld_col4<T>(Ks, SK, s * 16 + 8 * h + 4, jd * 32));
          mma(acc, a, b);
        }
        float* dst = dqh + (q0 + tq * 32 + 4 * h) * D + jd * 32 + r;
        if (tq * 32 + 32 <= qlim) {
#pragma unroll
          for (int e = 0; e < 16; ++e) atomicAdd(dst + (8 * (e >> 2) + (e & 3)) * D, acc[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (tq * 32 + 8 * (e >> 2) + 4 * h + (e & 3) < qlim) atomicAdd(dst + (8 * (e >> 2) + (e & 3)) * D, acc[e]);
        }
      }
    }
    lds_barrier();
  }

  // Sum the QT partial dK/dV of each key tile through LDS, then write rows of
  // this lane's key (C tiles hold rows = head dim).
  if constexpr (G::QT > 1) {
    float* red = reinterpret_cast<float*>(dyn_smem);
    for (int pass = 0; pass < 2; ++pass) {
      f32x16(&acc)[ND] = pass == 0 ? dk : dv;
      for (int src = 1; src < G::QT; ++src) {
        if (qt == src) {
#pragma unroll
          for (int j = 0; j < ND; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[((kt * ND + j) * 16 + e) * 64 + l] = acc[j][e];
        }
        lds_barrier();
        if (qt == 0) {
#pragma unroll
          for (int j = 0; j < ND; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] += red[((kt * ND + j) * 16 + e) * 64 + l];
        }
        lds_barrier();
      }
    }
  }
  if (qt == 0) {
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
}

template <typename T, int D>
hipError_t launch_bwd_d(const AttnBwd<T>& p, hipStream_t s) {
  using G = BwdGeo<T, D>;
  const dim3 grid((unsigned)((p.N + G::BKEY - 1) / G::BKEY));
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_kernel<T, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)G::SMEM);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_kernel<T, D>), grid, dim3(G::NT), G::SMEM, s, p);
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
