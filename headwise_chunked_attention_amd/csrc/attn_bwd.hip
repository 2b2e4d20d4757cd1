// Causal GQA flash-attention backward for one chunk of heads on gfx950.
//
// Backward recomputes P from Q, K and the saved log-sum-exp instead of
// keeping any per-head activation from the forward (activation
// checkpointing applied inside the op: "Road to 5 Million Tokens",
// transcript, activation-checkpointing part; the chunk's activations are
// "recomputed", memeeeeeex.com article, section "Untied Ulysses (UPipe) —
// head 単位のチャンク化").
//
// With P = exp(S/sqrt(d) - LSE) and dS = P (dP - Delta) / sqrt(d):
//   dV = P^T dO,  dK = dS^T Q,  dQ = dS K.
// q arrives multiplied by log2(e)/sqrt(d) and dO by 1/sqrt(d), so Q K^T is
// the exponent in log2 units and dO V^T is dP/sqrt(d); the dK/dV kernel
// scales its two results back once at the end. Both kernels form the same
// dS values.
// Two kernels, no dQ atomics:
//  * dK/dV kernel, key-stationary: a workgroup owns a block of keys and walks
//    the query tiles at or after it for every q head of the chunk reading this
//    kv head, so dK and dV sum over the GQA group in registers (short
//    sequences split the heads over several workgroups per key block and add
//    their sums with fp32 atomics; the deterministic entry point does not). Per step it
//    computes S = Q K^T and dP = dO V^T (rows q, one key per lane), then
//    dV^T += dO^T P and dK^T += Q^T dS with P/dS fed from the accumulators.
//  * dQ kernel, query-stationary (the forward's shape): a wave owns 32 queries
//    and walks the key tiles up to them computing S^T = K Q^T, dP^T = V dO^T
//    (one query per lane), then dQ^T += K^T dS^T.
// The dQ kernel recomputes S and dP (4*d more flops per visible pair) but
// writes dQ once instead of accumulating it with fp32 atomics, which on this
// chip cost more than the whole rest of the backward.
// Every LDS tile is a row-major copy of global memory; transposed operands
// (dO^T, Q^T, K^T) are column reads with gfx950's LDS transpose reads.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace upipe {

namespace {

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
// Workgroup geometry: KT x QT waves. Wave w owns key tile w % KT (32 keys) and
// query tile w / KT (32 queries) of each step, so a workgroup covers
// BKEY = 32*KT keys and BQ = 32*QT queries per step; with 8 waves two waves
// share each SIMD. Q/dO tiles are double buffered in LDS.
//
// Every Q/dO tile a workgroup loads serves its BKEY keys, so the direct loads
// (and their LDS writes) per flop fall as BKEY grows. bf16 with head_dim 128
// takes the widest block that fits: 8 x 1 waves, 256 keys, 32 queries per
// step. K and V of 256 keys (128 KB) and two 32-query Q/dO buffers (32 KB)
// fill the 160 KB of LDS, so the per-step LSE/Delta go into bytes of the K
// tile that no step reads (stat_at in the kernel).
template <typename T, int D>
struct DkdvGeo {
  static constexpr bool BIG = (sizeof(T) == 4 && D == 128);  // fp32, head_dim 128: smaller block (LDS)
  static constexpr bool WIDE = (sizeof(T) == 2 && D == 128);
  static constexpr int KT = BIG ? 2 : (WIDE ? 8 : 4);
  static constexpr int QT = (BIG || WIDE) ? 1 : 2;
  static constexpr int NW = KT * QT;
  static constexpr int NT = 64 * NW;
  static constexpr int BKEY = 32 * KT;
  static constexpr int BQ = 32 * QT;
  static constexpr int VEC = 16 / (int)sizeof(T);
  using L = Tile<T, D>;  // every tile is [rows][D]
  // the two [Q | dO] buffers first: every per-step tile address is then a
  // per-lane register plus an immediate offset below 64 KB
  static constexpr int BUF_OFF = 0;
  static constexpr int BUF_ELEMS = 2 * L::ELEMS(BQ);
  static constexpr int K_OFF = BUF_OFF + 2 * BUF_ELEMS;
  static constexpr int V_OFF = K_OFF + L::ELEMS(BKEY);
  static constexpr int T_ELEMS = V_OFF + L::ELEMS(BKEY);
  static constexpr int RCH = D / VEC;         // 16-byte chunks per row
  static constexpr int PER = BQ * RCH / NT;   // prefetch chunks per thread and tensor
  static constexpr size_t SMEM = (size_t)T_ELEMS * sizeof(T) + (WIDE ? 0 : 2 * 2 * BQ * sizeof(float));
  static_assert(!WIDE || (2 * 2 * BQ <= 8 * 16 && BKEY >= 32), "statistics fit the unread K bytes of 16 rows");
  // end-of-kernel reduction of the QT partial dK/dV sums per key tile
  static constexpr size_t RED = (size_t)KT * 64 * 16 * (D / 32) * sizeof(float);
  static_assert((BQ * RCH) % NT == 0, "tile chunks");
  static_assert(QT == 1 || RED <= SMEM, "reduction buffer fits in LDS");
};

template <typename T, int D, class G>
DEV void load_rows(const T* base, int64_t row0, u32x4 (&r)[G::PER]) {
#pragma unroll
  for (int i = 0; i < G::PER; ++i) {
    const int c = threadIdx.x + i * G::NT;
    r[i] = ld_raw16(base + (row0 + c / G::RCH) * D + (c % G::RCH) * G::VEC);
  }
}

template <typename T, int D, class G>
DEV void store_rows(T* S, const u32x4 (&r)[G::PER]) {
#pragma unroll
  for (int i = 0; i < G::PER; ++i) {
    const int c = threadIdx.x + i * G::NT;
    st_raw16(S + G::L::idx(c / G::RCH, (c % G::RCH) * G::VEC), r[i]);
  }
}

template <typename T, int D>
__global__ __launch_bounds__((DkdvGeo<T, D>::NT)) void attn_bwd_dkdv_kernel(const AttnBwd<T> p, int hs) {
  using G = DkdvGeo<T, D>;
  constexpr int BQ = G::BQ, BKEY = G::BKEY, ND = D / 32, NS = D / 16;
  using L = typename G::L;
  extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
  T* sm = reinterpret_cast<T*>(dyn_smem);
  T* Ks = sm + G::K_OFF;
  T* Vs = sm + G::V_OFF;
  float* stat = reinterpret_cast<float*>(sm + G::T_ELEMS);  // [2 buffers][lse | delta][BQ]
  // float f of those statistics. WIDE: every wave holds head-dim columns
  // 0..15 of its keys' K in registers before the walk, and in K row r those
  // columns (logical chunks 0 and 1) sit at physical chunks 2k and 2k + 1,
  // k = swz(r) / 2, where no step reads. Slot s = f / 8 (8 floats) goes to
  // one of wave 0's rows, chosen so that the four slots of one commit store
  // (slots 4j .. 4j + 3) have k = 0, 1, 2, 3: 32-byte runs at byte offsets 0,
  // 32, 64 and 96 of their rows, on different LDS banks.
  auto stat_at = [&](int f) -> float* {
    if constexpr (G::WIDE) {
      const int sl = f / 8;
      const int row = 16 * (sl >> 3) + 4 * ((sl >> 2) & 1) + 8 * (sl & 1) + ((sl >> 1) & 1);
      return reinterpret_cast<float*>(Ks + row * L::STRIDE + (L::swz(row) >> 1) * 16) + f % 8;
    } else {
      return stat + f;
    }
  };

  const int l = lane_id(), r = l & 31, h = l >> 5;
  const int w = wave_id();
  const int kt = w % G::KT, qt = w / G::KT;
  const int tid = threadIdx.x;
  // workgroup -> (key block, head group): the hs head groups of a key block
  // are adjacent, and key block 0 (the most query tiles) comes first
  const int64_t lin = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t k0 = (lin / hs) * BKEY;
  const int krel = kt * 32 + r;                   // this lane's key within the block
  const int64_t kw = k0 + krel;

  for (int c = tid; c < BKEY * G::RCH; c += G::NT) {
    const int row = c / G::RCH, cc = c % G::RCH;
    st_raw16(Ks + L::idx(row, cc * G::VEC), ld_raw16(p.k + (k0 + row) * D + cc * G::VEC));
    st_raw16(Vs + L::idx(row, cc * G::VEC), ld_raw16(p.v + (k0 + row) * D + cc * G::VEC));
  }
  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    dk[j] = zero16();
    dv[j] = zero16();
  }

  const int64_t qend = ((p.N + BQ - 1) / BQ) * BQ;
  const int64_t nqt = (qend - k0) / BQ;  // k0 is a multiple of BQ
  // heads h0 .. h0 + nh_b - 1 of the nh (hs workgroups share a key block)
  const int nh_b = p.nh / hs;
  const int h0 = (int)(lin % hs) * nh_b;
  const int64_t total = nqt * nh_b;

  constexpr bool DMA = L::SWZ;  // bf16: Q/dO tiles by direct global -> LDS loads
  u32x4 rq[DMA ? 1 : G::PER], rdo[DMA ? 1 : G::PER];
  float rl = 0.f, rd = 0.f;
  bool rvalid = false;
  // (head, query tile) of a step, without 64-bit division in the loop
  auto prefetch = [&](int hh, int64_t q0, int dst) {
    if constexpr (DMA) {
      constexpr int ROWS_PER_INST = 1024 / L::ROW_BYTES;
      constexpr int INST = BQ / ROWS_PER_INST;
      T* qd = sm + G::BUF_OFF + dst * G::BUF_ELEMS;
      for (int i = w; i < INST; i += G::NW) {
        dma_tile_rows<L>(p.q + (int64_t)hh * p.Np * D + q0 * D, D, qd, i * ROWS_PER_INST);
        dma_tile_rows<L>(p.dout + (int64_t)hh * p.Np * D + q0 * D, D, qd + L::ELEMS(BQ), i * ROWS_PER_INST);
      }
    } else {
      load_rows<T, D, G>(p.q + (int64_t)hh * p.Np * D, q0, rq);
      load_rows<T, D, G>(p.dout + (int64_t)hh * p.Np * D, q0, rdo);
    }
    if (tid < BQ) {
      // raw values now, used at the commit: nothing here waits for the loads
      const int64_t q = q0 + tid;
      const int64_t qc = q < p.N ? q : p.N - 1;
      rl = p.lse[(int64_t)hh * p.lse_stride + qc];
      rd = p.delta[(int64_t)hh * p.Np + qc];
      rvalid = q < p.N;
    }
  };
  auto commit = [&](int b) {
    if constexpr (DMA) {
      wait_vmem();  // this wave's direct loads into buffer b have landed
    } else {
      store_rows<T, D, G>(sm + G::BUF_OFF + b * G::BUF_ELEMS, rq);
      store_rows<T, D, G>(sm + G::BUF_OFF + b * G::BUF_ELEMS + L::ELEMS(BQ), rdo);
    }
    if (tid < BQ) {
      // negated: they start the S and dP accumulators; rows past the end get P = 0
      *stat_at(b * 2 * BQ + tid) = rvalid ? -rl * 1.4426950408889634f : -INFINITY;
      *stat_at(b * 2 * BQ + BQ + tid) = rvalid ? -rd : 0.f;
    }
  };

  Frag<T> kb0, vb0;
  if constexpr (G::WIDE) {
    // the first d step of this lane's K and V leave LDS before the statistics
    // are written over them
    lds_barrier();
    kb0 = ld_frag(Ks + L::idx(krel, 8 * h));
    vb0 = ld_frag(Vs + L::idx(krel, 8 * h));
    lds_barrier();
  }
  prefetch(h0, k0, 0);
  commit(0);
  lds_barrier();

  int hh = h0;
  int64_t q0 = k0;
  // One step on LDS buffer B (a compile-time constant, so the step's LDS
  // addresses need no per-step arithmetic).
  // bf16: lane offsets of the dO^T / Q^T column reads, computed once
  Col4Plan<L, ND> cplan;
  if constexpr (sizeof(T) == 2) cplan.init();
  // the K and V fragments of the first d step stay in registers: the first
  // MFMAs of a step then wait only for the Q and dO reads
  if constexpr (!G::WIDE) {
    kb0 = ld_frag(Ks + L::idx(krel, 8 * h));
    vb0 = ld_frag(Vs + L::idx(krel, 8 * h));
  }
  auto step = [&](auto bc, int64_t it) {
    constexpr int B = decltype(bc)::value;
    int nh_next = hh;
    int64_t q_next = q0 + BQ;
    if (q_next >= qend) {
      q_next = k0;
      ++nh_next;
    }
    if (it + 1 < total) prefetch(nh_next, q_next, B ^ 1);
    const T* Qs = sm + G::BUF_OFF + B * G::BUF_ELEMS;
    const T* dOs = Qs + L::ELEMS(BQ);
    const int qrel0 = (int)(q0 - k0) + qt * 32;  // wave's first row - block start
    // wave-uniform: only tiles that cross the diagonal need the causal mask
    const bool diag = qrel0 < kt * 32 + 32;

    // S - LSE and dP - Delta (log2 units and 1/sqrt(d) scale come with the
    // pre-scaled q and dout): the accumulators start at -LSE and -Delta of
    // their query rows (element 4i+j is row 8i + 4h + j of the wave's 32),
    // so the MFMAs do the subtraction. Rows past the end of the sequence
    // carry LSE = +inf, so their P is 0 without a mask. fp32 starts the S
    // chain at 0 and subtracts LSE once at the end instead: a chain started
    // at -LSE rounds every partial sum at the LSE's magnitude, which for
    // sharp scores (|LSE| in the hundreds of log2 units) costs fp32 several
    // times the rounding of the plain S - LSE.
    constexpr bool SUB_AFTER = sizeof(T) == 4;
    f32x16 sacc, dpacc, lse_neg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 lv = *reinterpret_cast<const f32x4*>(stat_at(B * 2 * BQ + qt * 32 + 8 * i + 4 * h));
      const f32x4 dv4 = *reinterpret_cast<const f32x4*>(stat_at(B * 2 * BQ + BQ + qt * 32 + 8 * i + 4 * h));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lse_neg[4 * i + j] = lv[j];
        sacc[4 * i + j] = SUB_AFTER ? 0.f : lv[j];
        dpacc[4 * i + j] = dv4[j];
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const Frag<T> kb = s == 0 ? kb0 : ld_frag(Ks + L::idx(krel, s * 16 + 8 * h));
      const Frag<T> vb = s == 0 ? vb0 : ld_frag(Vs + L::idx(krel, s * 16 + 8 * h));
      mma(sacc, ld_frag(Qs + L::idx(qt * 32 + r, s * 16 + 8 * h)), kb);
      mma(dpacc, ld_frag(dOs + L::idx(qt * 32 + r, s * 16 + 8 * h)), vb);
    }
    if constexpr (SUB_AFTER) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[e] += lse_neg[e];
    }
    // bf16: the dO^T / Q^T fragment pairs of the first two dV/dK products are
    // read before the softmax, whose VALU work then covers their latency
    Frag<T> ado[2], aq[2];
    auto frags = [&](auto t, int i) {
      // rows qt*32 + 16*s2 + ... of dO and Q at the precomputed lane offsets
      const T* dOr = dOs + (qt * 32 + 16 * (t / ND)) * L::STRIDE;
      const T* Qr = Qs + (qt * 32 + 16 * (t / ND)) * L::STRIDE;
      ado[i] = frag_from_col4<T>(ld_col4_at(dOr, cplan.off[0][t % ND]), ld_col4_at(dOr, cplan.off[1][t % ND]));
      aq[i] = frag_from_col4<T>(ld_col4_at(Qr, cplan.off[0][t % ND]), ld_col4_at(Qr, cplan.off[1][t % ND]));
    };
    if constexpr (sizeof(T) == 2) {
      frags(0, 0);
      frags(1, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P = exp2(S - LSE); dS = P (dP - Delta) / sqrt(d), the same values the dQ
    // kernel forms
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = fast_exp2(sacc[e]);
    if (diag) {
      // element e is query row qrel0 + 8(e/4) + 4h + e%4; keep keys at or before it
      const int dk0 = krel - qrel0 - 4 * h;
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[e] = (dk0 <= 8 * (e / 4) + e % 4) ? sacc[e] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) dpacc[e] = sacc[e] * dpacc[e];
    // dV^T += dO^T P and dK^T += Q^T dS over this wave's 32 queries.
    if constexpr (sizeof(T) == 2) {
      // 2*ND product pairs t = (s2, j); pairs 0 and 1 have their fragments
      // already, and from pair 1 on the fragments of pair t + 1 are read
      // before pair t issues
      const Frag<T> pbf[2] = {frag_from_acc<T>(sacc, 0, 1.0f), frag_from_acc<T>(sacc, 1, 1.0f)};
      const Frag<T> sbf[2] = {frag_from_acc<T>(dpacc, 0, 1.0f), frag_from_acc<T>(dpacc, 1, 1.0f)};
#pragma unroll
      for (int t = 0; t < 2 * ND; ++t) {
        if (t >= 1 && t + 1 < 2 * ND) frags(t + 1, (t + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        mma(dv[t % ND], ado[t & 1], pbf[t / ND]);
        mma(dk[t % ND], aq[t & 1], sbf[t / ND]);
      }
    } else {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const Frag<T> pb = frag_from_acc<T>(sacc, s2, 1.0f);
        const Frag<T> sb = frag_from_acc<T>(dpacc, s2, 1.0f);
        const int row0 = qt * 32 + 16 * s2 + 4 * h;
#pragma unroll
        for (int j = 0; j < ND; ++j) {
          const Frag<T> ado = frag_from_col4<T>(ld_col4<L>(dOs, row0, j * 32), ld_col4<L>(dOs, row0 + 8, j * 32));
          const Frag<T> aq = frag_from_col4<T>(ld_col4<L>(Qs, row0, j * 32), ld_col4<L>(Qs, row0 + 8, j * 32));
          mma(dv[j], ado, pb);
          mma(dk[j], aq, sb);
        }
      }
    }
    if (it + 1 < total) commit(B ^ 1);
    lds_barrier();
    hh = nh_next;
    q0 = q_next;
  };
  for (int64_t it = 0; it < total; it += 2) {
    step(std::integral_constant<int, 0>(), it);
    if (it + 1 < total) step(std::integral_constant<int, 1>(), it + 1);
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
        f32x4 vk = (f32x4){dk[j][4 * i], dk[j][4 * i + 1], dk[j][4 * i + 2], dk[j][4 * i + 3]} * p.dk_mul;
        f32x4 vv = (f32x4){dv[j][4 * i], dv[j][4 * i + 1], dv[j][4 * i + 2], dv[j][4 * i + 3]} * p.dv_mul;
        if (hs > 1) {  // several workgroups per key block: add (the launcher zeroed)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            atomicAdd(p.dk_acc + kw * D + dd + e, vk[e]);
            atomicAdd(p.dv_acc + kw * D + dd + e, vv[e]);
          }
          continue;
        }
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

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
constexpr int BC = 64;  // keys per tile

template <typename T, int D>
struct DqGeo {
  static constexpr int NW = 8;  // waves per workgroup, 32 queries each
  static constexpr int NT = 64 * NW;
  using L = Tile<T, D>;
  static constexpr int STAGE = 2 * L::ELEMS(BC);  // K tile then V tile
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int RCH = D / VEC;
  static constexpr int KCH = BC * RCH / NT;  // 16-byte chunks per thread and tensor
  static_assert((BC * RCH) % NT == 0, "tile chunks");
};

template <typename T, int D>
__global__ __launch_bounds__((DqGeo<T, D>::NT)) void attn_bwd_dq_kernel(const AttnBwd<T> p, int hp) {
  using G = DqGeo<T, D>;
  constexpr int ND = D / 32, NS = D / 16;
  using L = typename G::L;
  extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
  T* smem = reinterpret_cast<T*>(dyn_smem);

  const int l = lane_id(), r = l & 31, h = l >> 5;
  const int w = wave_id();
  const int qb_rows = G::NW * 32 / hp;  // query positions per workgroup
  const int64_t nqb = p.Np / qb_rows;
  const int64_t qb = nqb - 1 - (int64_t)blockIdx.x;  // longest rows first
  const int hh = (int)blockIdx.y * hp + (w % hp);
  const int64_t qs = qb * qb_rows;
  const int64_t q0w = qs + (int64_t)(w / hp) * 32;
  const int64_t q = q0w + r;  // this lane's query

  // Q and dO of this lane's query as B operands (k = head dim), resident.
  const int64_t hoff = (int64_t)hh * p.Np * D;
  Frag<T> qf[NS], df[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    qf[s] = ld_frag(p.q + hoff + q * D + s * 16 + 8 * h);
    df[s] = ld_frag(p.dout + hoff + q * D + s * 16 + 8 * h);
  }
  // past the end of the sequence LSE = +inf makes P = 0
  const float lse2 = (q < p.N) ? p.lse[(int64_t)hh * p.lse_stride + q] * 1.4426950408889634f : INFINITY;
  const float dlt = (q < p.N) ? p.delta[(int64_t)hh * p.Np + q] : 0.f;
  // accumulator starts: -LSE and -Delta of this lane's query; fp32 starts the
  // S chain at 0 and subtracts LSE after it (the rounding of the plain S - LSE,
  // as in the dK/dV kernel)
  constexpr bool SUB_AFTER = sizeof(T) == 4;
  f32x16 init_s, init_dp;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    init_s[e] = SUB_AFTER ? 0.f : -lse2;
    init_dp[e] = -dlt;
  }
  f32x16 dq[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) dq[j] = zero16();

  auto load = [&](int64_t k0, u32x4(&rk)[G::KCH], u32x4(&rv)[G::KCH]) {
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
      const int c = threadIdx.x + i * G::NT;
      rk[i] = ld_raw16(p.k + (k0 + c / G::RCH) * D + (c % G::RCH) * G::VEC);
      rv[i] = ld_raw16(p.v + (k0 + c / G::RCH) * D + (c % G::RCH) * G::VEC);
    }
  };
  auto store = [&](T* st, const u32x4(&rk)[G::KCH], const u32x4(&rv)[G::KCH]) {
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
      const int c = threadIdx.x + i * G::NT;
      st_raw16(st + L::idx(c / G::RCH, (c % G::RCH) * G::VEC), rk[i]);
      st_raw16(st + L::ELEMS(BC) + L::idx(c / G::RCH, (c % G::RCH) * G::VEC), rv[i]);
    }
  };

  constexpr bool DMA = L::SWZ;  // bf16: K/V tiles by direct global -> LDS loads
  auto dma = [&](int64_t k0, T* st) {
    if constexpr (DMA) {
      constexpr int ROWS_PER_INST = 1024 / L::ROW_BYTES;
      constexpr int INST = BC / ROWS_PER_INST;
      for (int i = w; i < INST; i += G::NW) {
        dma_tile_rows<L>(p.k + k0 * D, D, st, i * ROWS_PER_INST);
        dma_tile_rows<L>(p.v + k0 * D, D, st + L::ELEMS(BC), i * ROWS_PER_INST);
      }
    }
  };
  const int64_t ntiles = (qs + qb_rows) / BC;
  u32x4 rk[DMA ? 1 : G::KCH], rv[DMA ? 1 : G::KCH];
  if constexpr (DMA) {
    dma(0, smem);
    wait_vmem();
  } else {
    load(0, rk, rv);
    store(smem, rk, rv);
  }
  lds_barrier();
  // one key tile on LDS stage BUF (a compile-time constant: immediate LDS offsets)
  // bf16: lane offsets of the K^T column reads, computed once
  Col4Plan<L, ND> kplan;
  if constexpr (sizeof(T) == 2) kplan.init();
  auto step = [&](auto bc, int64_t kt_i) {
    constexpr int buf = decltype(bc)::value;
    const int64_t k0 = kt_i * BC;
    if (kt_i + 1 < ntiles) {
      if constexpr (DMA)
        dma(k0 + BC, smem + (buf ^ 1) * G::STAGE);
      else
        load(k0 + BC, rk, rv);
    }
    const T* Ks = smem + buf * G::STAGE;
    const T* Vs = Ks + L::ELEMS(BC);
    if (k0 <= q0w + 31) {  // some key of the tile is visible to this wave
      // The two 32-key halves one after the other. S^T - LSE and dP^T - Delta:
      // every accumulator chain starts from the loop-invariant splat of -LSE
      // (or -Delta) of this lane's query, so the MFMAs do the subtraction.
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        // the K and V fragments of step s + 1 are read before the MFMAs of step s
        f32x16 sacc, dpacc;
        Frag<T> kf[2], vf[2];
        kf[0] = ld_frag(Ks + L::idx(kt * 32 + r, 8 * h));
        vf[0] = ld_frag(Vs + L::idx(kt * 32 + r, 8 * h));
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s + 1 < NS) {
            kf[(s + 1) & 1] = ld_frag(Ks + L::idx(kt * 32 + r, (s + 1) * 16 + 8 * h));
            vf[(s + 1) & 1] = ld_frag(Vs + L::idx(kt * 32 + r, (s + 1) * 16 + 8 * h));
          }
          __builtin_amdgcn_sched_barrier(0);
          if (s == 0) {
            sacc = mma_first(kf[0], qf[0], init_s);
            dpacc = mma_first(vf[0], df[0], init_dp);
          } else {
            mma(sacc, kf[s & 1], qf[s]);
            mma(dpacc, vf[s & 1], df[s]);
          }
        }
        // bf16: the K^T fragments of the first three dQ products are read
        // before the softmax, whose VALU work then covers their latency
        auto kfrag = [&](auto t) {
          // rows kt*32 + 16*s2 + ... of K at the precomputed lane offsets
          const T* Kr = Ks + (kt * 32 + 16 * (t / ND)) * L::STRIDE;
          return frag_from_col4<T>(ld_col4_at(Kr, kplan.off[0][t % ND]), ld_col4_at(Kr, kplan.off[1][t % ND]));
        };
        Frag<T> kf3[3];
        if constexpr (sizeof(T) == 2) {
          kf3[0] = kfrag(0);
          kf3[1] = kfrag(1);
          kf3[2] = kfrag(2);
          __builtin_amdgcn_sched_barrier(0);
        }
        // P = exp2(S - LSE); dS = P (dP - Delta) / sqrt(d) (log2 units and the
        // 1/sqrt(d) come with the pre-scaled q and dout)
        if constexpr (SUB_AFTER) {
#pragma unroll
          for (int e = 0; e < 16; ++e) sacc[e] -= lse2;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = fast_exp2(sacc[e]);
        if (k0 + kt * 32 + 31 > q0w) {  // wave-uniform: the half crosses this wave's diagonal
          // element e is key kt*32 + 8(e/4) + 4h + e%4 of the tile
          const int qrel = (int)(q - k0) - 4 * h - kt * 32;
#pragma unroll
          for (int e = 0; e < 16; ++e) sacc[e] = (8 * (e >> 2) + (e & 3) <= qrel) ? sacc[e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) dpacc[e] = sacc[e] * dpacc[e];
        // dQ^T += K^T dS^T (contraction over the half's keys = accumulator
        // rows): 2*ND products t = (s2, j); bf16 has the fragments of products
        // 0-2 already and from product 1 on reads the K^T fragment of product
        // t + 2 before product t issues
        const Frag<T> sbf[2] = {frag_from_acc<T>(dpacc, 0, 1.0f), frag_from_acc<T>(dpacc, 1, 1.0f)};
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int t = 0; t < 2 * ND; ++t) {
            if (t >= 1 && t + 2 < 2 * ND) kf3[(t + 2) % 3] = kfrag(t + 2);
            __builtin_amdgcn_sched_barrier(0);
            mma(dq[t % ND], kf3[t % 3], sbf[t / ND]);
          }
        } else {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int j = 0; j < ND; ++j) {
              const int row0 = kt * 32 + 16 * s2 + 4 * h;
              mma(dq[j], frag_from_col4<T>(ld_col4<L>(Ks, row0, j * 32), ld_col4<L>(Ks, row0 + 8, j * 32)), sbf[s2]);
            }
        }
      }
    }
    if (kt_i + 1 < ntiles) {
      if constexpr (DMA)
        wait_vmem();
      else
        store(smem + (buf ^ 1) * G::STAGE, rk, rv);
    }
    lds_barrier();
  };
  for (int64_t kt_i = 0; kt_i < ntiles; kt_i += 2) {
    step(std::integral_constant<int, 0>(), kt_i);
    if (kt_i + 1 < ntiles) step(std::integral_constant<int, 1>(), kt_i + 1);
  }
  // dQ rows of this lane's query: C tiles hold rows = head dim.
  float* dst = p.dq + hoff + q * D;
#pragma unroll
  for (int j = 0; j < ND; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f32x4*>(dst + j * 32 + 8 * i + 4 * h) =
          (f32x4){dq[j][4 * i], dq[j][4 * i + 1], dq[j][4 * i + 2], dq[j][4 * i + 3]};
}

template <typename T, int D>
hipError_t launch_dkdv_d(const AttnBwd<T>& p, hipStream_t s) {
  using G = DkdvGeo<T, D>;
  const int64_t nkb = (p.N + G::BKEY - 1) / G::BKEY;
  // Key block b holds (N - b BKEY) / BQ query tiles per head: the work falls
  // off linearly with b, so the grid balances over the CUs only with several
  // workgroups per CU. With fewer key blocks than that and several heads, the
  // heads are split over hs workgroups and their partial sums added atomically.
  int hs = 1;
  while (!p.no_head_split && nkb * hs < 4 * 256 && p.nh % (hs * 2) == 0) hs *= 2;
  hipError_t e;
  if (hs > 1 && !p.accumulate) {
    if ((e = launch_fill_f32(p.dk_acc, nkb * G::BKEY * D, 0.f, s)) != hipSuccess) return e;
    if ((e = launch_fill_f32(p.dv_acc, nkb * G::BKEY * D, 0.f, s)) != hipSuccess) return e;
  }
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<T, D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)G::SMEM);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D>), dim3((unsigned)(nkb * hs)), dim3(G::NT), G::SMEM, s, p, hs);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dq_d(const AttnBwd<T>& p, hipStream_t s) {
  using G = DqGeo<T, D>;
  int hp = 1;
  while (hp * 2 <= 4 && p.nh % (hp * 2) == 0) hp *= 2;
  const int qb_rows = G::NW * 32 / hp;
  const dim3 grid((unsigned)(p.Np / qb_rows), (unsigned)(p.nh / hp));
  const size_t smem = (size_t)2 * G::STAGE * sizeof(T);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<T, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D>), grid, dim3(G::NT), smem, s, p, hp);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_attn_bwd_dkdv(const AttnBwd<T>& p, int head_dim, hipStream_t s) {
  if (head_dim == 64) return launch_dkdv_d<T, 64>(p, s);
  if (head_dim == 128) return launch_dkdv_d<T, 128>(p, s);
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_attn_bwd_dq(const AttnBwd<T>& p, int head_dim, hipStream_t s) {
  if (head_dim == 64) return launch_dq_d<T, 64>(p, s);
  if (head_dim == 128) return launch_dq_d<T, 128>(p, s);
  return hipErrorInvalidValue;
}

template hipError_t launch_attn_bwd_dkdv<bf16>(const AttnBwd<bf16>&, int, hipStream_t);
template hipError_t launch_attn_bwd_dkdv<float>(const AttnBwd<float>&, int, hipStream_t);
template hipError_t launch_attn_bwd_dq<bf16>(const AttnBwd<bf16>&, int, hipStream_t);
template hipError_t launch_attn_bwd_dq<float>(const AttnBwd<float>&, int, hipStream_t);

}  // namespace upipe
