// GDPA backward for bf16 on gfx950: one workgroup (4 waves) per (sequence, head) work item.
//
//   dp_ij = <dO_i, V_j>;   ds_ij = dp_ij phi'(s_ij)   or   p_ij (dp_ij - D_i), D_i = <dO_i, O_i>
//   dQ = scale dS K;   dK = scale dS^T Q;   dV = P^T dO;   dG_j = sigmoid(-G_j) sum_i ds_ij
//
// (FlashAttention-style backward that recomputes the scores tile by tile and never writes the
// score matrix to HBM: Kunlun review, section 2.3 and Figure 2. Gate: reproduction README "Core
// equations"; window: review section 2.5.)
//
// Work split inside an item: each wave owns one block of KB keys (K and V rows in registers, dK^T
// and dV^T accumulators in registers) and the four waves sweep the query tiles (64 rows) of the
// sequence together. Per query tile:
//   1. stage Q and dO into LDS, both row-major (A operand of S = Q K^T and dP = dO V^T) and
//      transposed in MFMA slot order (A operand of dK^T = Q^T dS and dV^T = dO^T P); for the
//      softmax form also the forward's row log-sum-exp, and then D_i = sum_j p_ij dp_ij from a
//      first pass in the transposed orientation (query on the lane);
//   2. each wave: S, dP on MFMA, P and dS in registers; their accumulator layout is directly the
//      B operand of the dK^T / dV^T products; dS also goes to an LDS exchange tile;
//   3. the waves split the dQ tile: dQ^T = K^T dS^T over all resident keys, with K^T staged in LDS
//      when a key block is taken.
// Personalized-FFN form: all (<= 4 KB) keys are resident for the whole sweep. Sliding window: key
// blocks rotate through the four wave slots as the sweep advances; a block's dK / dV / dG are
// written when it leaves the window. Every output element is written exactly once (no atomics).
#include "gdpa_device.hpp"
#include "gdpa_launch.hpp"

namespace gdpa {

template <int D>
struct BwdGeo {
  static constexpr int KB = D == 128 ? 32 : 64;  // keys per wave
  static constexpr int KS = KB / 32;             // 32-key subtiles per wave
  static constexpr int CAP = 4 * KB;             // resident keys per item
  static constexpr int QT = 64;                  // query rows per tile
  static constexpr int KK = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int NROW = D * 2 + 16;        // row-major Q / dO tile row (bytes)
  static constexpr int TROW = QT * 2 + 16;       // transposed tile row: 64 queries
  static constexpr int KTROW = CAP * 2 + 16;     // K^T row: CAP keys
  static constexpr int SXROW = CAP * 2 + 16;     // dS exchange row: CAP keys
  static constexpr int OFF_QN = 0;
  static constexpr int OFF_DON = OFF_QN + QT * NROW;
  static constexpr int OFF_QT = OFF_DON + QT * NROW;
  static constexpr int OFF_DOT = OFF_QT + D * TROW;
  static constexpr int OFF_KT = OFF_DOT + D * TROW;
  static constexpr int OFF_SX = OFF_KT + D * KTROW;       // dS (bf16; softmax: high part)
  static constexpr int OFF_SXL = OFF_SX + QT * SXROW;      // softmax: dS - high part, in bf16
  static constexpr int OFF_ROW = OFF_SXL + QT * SXROW;     // lse2[QT]
  static constexpr int OFF_DPART = OFF_ROW + QT * 4;       // softmax: partial D_i per wave [4][QT]
  static constexpr int OFF_GATE = OFF_DPART + 4 * QT * 4;  // gate term per resident key [CAP]
  static constexpr int BYTES = OFF_GATE + CAP * 4;
};

constexpr int max3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }
constexpr int kBwdLdsBytes = max3(BwdGeo<32>::BYTES, BwdGeo<64>::BYTES, BwdGeo<128>::BYTES);

__device__ inline int slot_pos(int i) { return (i & ~15) + slot_row(i & 15); }
__device__ inline int pmod4(int x) { return ((x % 4) + 4) % 4; }

template <int D, int ACT>
struct BwdWave {
  using G = BwdGeo<D>;
  bf16x8 kreg[G::KS][G::KK];
  bf16x8 vreg[G::KS][G::KK];
  f32x16 dk[G::DT][G::KS];
  f32x16 dv[G::DT][G::KS];
  float dgs[G::KS];
  float gate[G::KS];   // per-lane gate term of its key (natural units; log2 units for softmax)
  float graw[G::KS];   // raw G of its key (for dG)
};

// Block of keys [kbase, kbase + KB) of the sequence: registers + K^T into the wave's LDS slot.
template <int D, int ACT>
__device__ void take_block(BwdWave<D, ACT>& st, char* lds, const GroupDesc& gd, const bf16* kseq,
                           const bf16* vseq, const float* gseq, int kbase, int n, int slot) {
  using G = BwdGeo<D>;
  const int lane = lane_id(), kc = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)gd.num_heads * D;
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    const int key = kbase + ks * 32 + kc;
    const bool ok = key < n;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) {
      u32x4 ku = {0u, 0u, 0u, 0u}, vu = {0u, 0u, 0u, 0u};
      if (ok) {
        ku = *reinterpret_cast<const u32x4*>(kseq + key * rs + g * (D / 2) + kk * 8);
        vu = *reinterpret_cast<const u32x4*>(vseq + key * rs + g * (D / 2) + kk * 8);
      }
      st.kreg[ks][kk] = as_bf16x8(ku);
      st.vreg[ks][kk] = as_bf16x8(vu);
      // K^T into LDS: this lane's 8 d values of key `key` (d = g*D/2 + kk*8 + e)
      const int pos = slot * G::KB + slot_pos(ks * 32 + kc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d0 = g * (D / 2) + kk * 8 + 2 * e;
        *reinterpret_cast<uint16_t*>(lds + G::OFF_KT + d0 * G::KTROW + pos * 2) = (uint16_t)(ku[e] & 0xFFFF);
        *reinterpret_cast<uint16_t*>(lds + G::OFF_KT + (d0 + 1) * G::KTROW + pos * 2) = (uint16_t)(ku[e] >> 16);
      }
    }
    float t = 0.0f, gr = 0.0f;
    if (gseq != nullptr && ok) {
      gr = gseq[(size_t)key * gd.num_heads];
      t = log_sigmoid_f(gr);
      if (ACT == GDPA_ACT_SOFTMAX) t *= kLog2e;
    }
    st.gate[ks] = t;
    st.graw[ks] = gr;
    if (g == 0) reinterpret_cast<float*>(lds + G::OFF_GATE)[slot * G::KB + ks * 32 + kc] = t;
    st.dgs[ks] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt) {
      st.dk[dt][ks] = f32x16{};
      st.dv[dt][ks] = f32x16{};
    }
  }
}

// Write dK, dV (and dG) of the wave's block.
template <int D, int ACT>
__device__ void flush_block(BwdWave<D, ACT>& st, const GroupDesc& gd, bf16* dkseq, bf16* dvseq, float* dgseq,
                            int kbase, int n) {
  using G = BwdGeo<D>;
  const int lane = lane_id(), kc = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)gd.num_heads * D;
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    const int key = kbase + ks * 32 + kc;
    const float dgsum = st.dgs[ks] + __shfl_xor(st.dgs[ks], 32);
    if (key < n) {
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt) {
        u32x4 a0, a1, b0, b1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a0[e] = pack_bf16x2(st.dk[dt][ks][2 * e] * gd.scale, st.dk[dt][ks][2 * e + 1] * gd.scale);
          a1[e] = pack_bf16x2(st.dk[dt][ks][8 + 2 * e] * gd.scale, st.dk[dt][ks][9 + 2 * e] * gd.scale);
          b0[e] = pack_bf16x2(st.dv[dt][ks][2 * e], st.dv[dt][ks][2 * e + 1]);
          b1[e] = pack_bf16x2(st.dv[dt][ks][8 + 2 * e], st.dv[dt][ks][9 + 2 * e]);
        }
        bf16* pk = dkseq + key * rs + dt * 32 + g * 16;
        bf16* pv = dvseq + key * rs + dt * 32 + g * 16;
        *reinterpret_cast<u32x4*>(pk) = a0;
        *reinterpret_cast<u32x4*>(pk + 8) = a1;
        *reinterpret_cast<u32x4*>(pv) = b0;
        *reinterpret_cast<u32x4*>(pv + 8) = b1;
      }
      if (dgseq != nullptr && g == 0) {
        const float sg = 1.0f / (1.0f + __expf(st.graw[ks]));  // sigmoid(-G)
        dgseq[(size_t)key * gd.num_heads] = sg * dgsum;
      }
    }
  }
}

// Stage query tile rows [r0, r0 + QT) (sequence-relative) into LDS.
template <int D, int ACT>
__device__ void stage_qtile(char* lds, const GroupDesc& gd, const bf16* qseq, const bf16* doseq,
                            const float* lseseq, int r0, int L) {
  using G = BwdGeo<D>;
  constexpr int CPR = D / 8;
  const size_t rs = (size_t)gd.num_heads * D;
  float* lse2 = reinterpret_cast<float*>(lds + G::OFF_ROW);
  for (int idx = threadIdx.x; idx < G::QT * CPR; idx += kThreads) {
    const int r = idx / CPR, c = idx % CPR;
    const int row = r0 + r;
    u32x4 qu = {0u, 0u, 0u, 0u}, du = {0u, 0u, 0u, 0u};
    if (row < L) {
      qu = *reinterpret_cast<const u32x4*>(qseq + row * rs + c * 8);
      du = *reinterpret_cast<const u32x4*>(doseq + row * rs + c * 8);
    }
    *reinterpret_cast<u32x4*>(lds + G::OFF_QN + r * G::NROW + c * 16) = qu;
    *reinterpret_cast<u32x4*>(lds + G::OFF_DON + r * G::NROW + c * 16) = du;
    const int pos = slot_pos(r);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d0 = c * 8 + 2 * e;
      *reinterpret_cast<uint16_t*>(lds + G::OFF_QT + d0 * G::TROW + pos * 2) = (uint16_t)(qu[e] & 0xFFFF);
      *reinterpret_cast<uint16_t*>(lds + G::OFF_QT + (d0 + 1) * G::TROW + pos * 2) = (uint16_t)(qu[e] >> 16);
      *reinterpret_cast<uint16_t*>(lds + G::OFF_DOT + d0 * G::TROW + pos * 2) = (uint16_t)(du[e] & 0xFFFF);
      *reinterpret_cast<uint16_t*>(lds + G::OFF_DOT + (d0 + 1) * G::TROW + pos * 2) = (uint16_t)(du[e] >> 16);
    }
  }
  if (ACT == GDPA_ACT_SOFTMAX) {
    for (int r = threadIdx.x; r < G::QT; r += kThreads) {
      const int row = r0 + r;
      lse2[r] = row < L ? lseseq[(size_t)row * gd.num_heads] * kLog2e : __builtin_inff();
    }
  }
}

template <int D, int ACT>
__device__ void bwd_item(char* lds, const GroupDesc& gd, int b, int h) {
  using G = BwdGeo<D>;
  const int q0 = gd.q_off[b], L = gd.q_off[b + 1] - q0;
  const int k0 = gd.kv_off[b], n = gd.kv_off[b + 1] - k0;
  const int H = gd.num_heads;
  const size_t rs = (size_t)H * D;
  const bf16* qseq = reinterpret_cast<const bf16*>(gd.q) + ((size_t)q0 * H + h) * D;
  const bf16* doseq = reinterpret_cast<const bf16*>(gd.dout) + ((size_t)q0 * H + h) * D;
  const float* lseseq = gd.lse ? gd.lse + (size_t)q0 * H + h : nullptr;
  bf16* dqseq = reinterpret_cast<bf16*>(gd.dq) + ((size_t)q0 * H + h) * D;
  const bf16* kseq = reinterpret_cast<const bf16*>(gd.k) + ((size_t)k0 * H + h) * D;
  const bf16* vseq = reinterpret_cast<const bf16*>(gd.v) + ((size_t)k0 * H + h) * D;
  const float* gseq = gd.g ? gd.g + (size_t)k0 * H + h : nullptr;
  bf16* dkseq = reinterpret_cast<bf16*>(gd.dk) + ((size_t)k0 * H + h) * D;
  bf16* dvseq = reinterpret_cast<bf16*>(gd.dv) + ((size_t)k0 * H + h) * D;
  float* dgseq = gd.dg ? gd.dg + (size_t)k0 * H + h : nullptr;
  const int w = wave_id(), lane = lane_id(), lc = lane & 31, g = lane >> 5;
  constexpr bool softmax = ACT == GDPA_ACT_SOFTMAX;
  const int wl = gd.wl, wr = gd.wr;

  if (n <= 0) {
    // no keys: dQ = 0
    for (int idx = threadIdx.x; idx < L * (D / 8); idx += kThreads) {
      const int r = idx / (D / 8), c = idx % (D / 8);
      *reinterpret_cast<u32x4*>(dqseq + r * rs + c * 8) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  if (L <= 0) {
    // no queries: dK = dV = dG = 0
    for (int idx = threadIdx.x; idx < n * (D / 8); idx += kThreads) {
      const int r = idx / (D / 8), c = idx % (D / 8);
      *reinterpret_cast<u32x4*>(dkseq + r * rs + c * 8) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(dvseq + r * rs + c * 8) = u32x4{0u, 0u, 0u, 0u};
    }
    if (dgseq)
      for (int r = threadIdx.x; r < n; r += kThreads) dgseq[(size_t)r * H] = 0.0f;
    return;
  }

  const int nkb = (n + G::KB - 1) / G::KB;
  const int ntiles = (L + G::QT - 1) / G::QT;
  BwdWave<D, ACT> st;
  int cur = -1;  // key block held by this wave
  const float sc = softmax ? gd.scale * kLog2e : gd.scale;

  for (int j = 0; j < ntiles; ++j) {
    const int r0 = j * G::QT;
    // active key blocks for this query tile
    int kmin = 0, kmax = nkb - 1;
    if (wl >= 0) kmin = (r0 - wl > 0 ? r0 - wl : 0) / G::KB;
    if (wr >= 0) {
      const int hi = r0 + G::QT - 1 + wr < n - 1 ? r0 + G::QT - 1 + wr : n - 1;
      kmax = hi / G::KB;
    }
    const int mine = kmax - pmod4(kmax - w);
    const bool active = mine >= kmin && mine >= 0 && kmin <= kmax;
    __syncthreads();  // previous tile fully consumed (LDS tiles, dS exchange, K^T slots)
    if (active && mine != cur) {
      if (cur >= 0) flush_block<D, ACT>(st, gd, dkseq, dvseq, dgseq, cur * G::KB, n);
      take_block<D, ACT>(st, lds, gd, kseq, vseq, gseq, mine * G::KB, n, w);
      cur = mine;
    }
    stage_qtile<D, ACT>(lds, gd, qseq, doseq, lseseq, r0, L);
    __syncthreads();

    const float* lse2 = reinterpret_cast<const float*>(lds + G::OFF_ROW);
    float* dpart = reinterpret_cast<float*>(lds + G::OFF_DPART);
    if constexpr (softmax) {
      // D_i = sum_j p_ij dp_ij over all keys of row i, exactly as defined (not <dO_i, O_i> of the
      // rounded forward output). S^T = K Q^T and dP^T = V dO^T put the query on the lane, so the
      // sum over this wave's keys is a sum over registers plus one cross-half exchange; the four
      // waves' partial sums are then combined in a fixed order (deterministic).
      const float* gl = reinterpret_cast<const float*>(lds + G::OFF_GATE);
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        float part = 0.0f;
        const int rf = r0 + qs * 32, rl = rf + 31;
        const int row = rf + lc;
        if (active) {
#pragma unroll
          for (int ks = 0; ks < G::KS; ++ks) {
            const int kf = mine * G::KB + ks * 32, kl = kf + 31;
            bool empty = kf >= n || rf >= L;
            if (wl >= 0 && kl < rf - wl) empty = true;
            if (wr >= 0 && kf > rl + wr) empty = true;
            if (empty) continue;
            f32x16 st_ = f32x16{}, dpt = f32x16{};
#pragma unroll
            for (int kk = 0; kk < G::KK; ++kk) {
              const bf16x8 qb = as_bf16x8(*reinterpret_cast<const u32x4*>(
                  lds + G::OFF_QN + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
              const bf16x8 db = as_bf16x8(*reinterpret_cast<const u32x4*>(
                  lds + G::OFF_DON + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
              st_ = mfma32(st.kreg[ks][kk], qb, st_);
              dpt = mfma32(st.vreg[ks][kk], db, dpt);
            }
            const float l2 = lse2[qs * 32 + lc];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kloc = ks * 32 + c_row(r, g);
              const int key = mine * G::KB + kloc;
              const float x = __builtin_fmaf(st_[r], sc, gl[w * G::KB + kloc]);
              const bool ok = key < n && row < L && (wl < 0 || key >= row - wl) && (wr < 0 || key <= row + wr);
              part += ok ? fast_exp2(x - l2) * dpt[r] : 0.0f;
            }
          }
        }
        part += __shfl_xor(part, 32);
        if (g == 0) dpart[w * G::QT + qs * 32 + lc] = part;
      }
      __syncthreads();
    }
    if (active) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
          const int key = mine * G::KB + ks * 32 + lc;  // this lane's key (sequence position)
          // window / tail test for the whole 32x32 subtile
          const int rf = r0 + qs * 32, rl = rf + 31;
          const int kf = mine * G::KB + ks * 32, kl = kf + 31;
          bool empty = kf >= n || rf >= L;
          if (wl >= 0 && kl < rf - wl) empty = true;
          if (wr >= 0 && kf > rl + wr) empty = true;
          bool full = kl < n && rl < L;
          if (wl >= 0 && kf < rl - wl) full = false;
          if (wr >= 0 && kl > rf + wr) full = false;
          uint16_t* sx = reinterpret_cast<uint16_t*>(lds + G::OFF_SX);
          uint16_t* sxl = reinterpret_cast<uint16_t*>(lds + G::OFF_SXL);
          const int spos = w * G::KB + slot_pos(ks * 32 + lc);
          if (empty) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              sx[(qs * 32 + c_row(r, g)) * (G::SXROW / 2) + spos] = 0;
              if constexpr (softmax) sxl[(qs * 32 + c_row(r, g)) * (G::SXROW / 2) + spos] = 0;
            }
            continue;
          }
          f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
          for (int kk = 0; kk < G::KK; ++kk) {
            const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(
                lds + G::OFF_QN + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
            const bf16x8 da = as_bf16x8(*reinterpret_cast<const u32x4*>(
                lds + G::OFF_DON + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
            s = mfma32(qa, st.kreg[ks][kk], s);
            dp = mfma32(da, st.vreg[ks][kk], dp);
          }
          // element-wise: register r is query row r0 + qs*32 + c_row(r, g), key `key`
          float p[16], ds[16];
          float dsum = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = qs * 32 + c_row(r, g);
            const float x = __builtin_fmaf(s[r], sc, st.gate[ks]);
            float pv, dsv;
            if constexpr (softmax) {
              const float Di = ((dpart[rr] + dpart[G::QT + rr]) + dpart[2 * G::QT + rr]) + dpart[3 * G::QT + rr];
              pv = fast_exp2(x - lse2[rr]);
              dsv = pv * (dp[r] - Di);
            } else {
              float dphi;
              Act<ACT>::fg(x, pv, dphi);
              dsv = dp[r] * dphi;
            }
            if (!full) {
              const int row = r0 + rr;
              const bool ok = key < n && row < L && (wl < 0 || key >= row - wl) && (wr < 0 || key <= row + wr);
              pv = ok ? pv : 0.0f;
              dsv = ok ? dsv : 0.0f;
            }
            p[r] = pv;
            ds[r] = dsv;
            dsum += dsv;
          }
          st.dgs[ks] += dsum;
          // P and dS as bf16 B operands (k-tile t = registers 8t..8t+7). The softmax form also
          // carries the rounding remainder as a second bf16 term (x ~ hi + lo): its products mix
          // a few large probabilities, whose bf16 rounding alone would exceed the tolerance.
          bf16x8 pb[2], db[2], pl[2], dl[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            u32x4 pu, du, plu = {0u, 0u, 0u, 0u}, dlu = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              pu[e] = pack_bf16x2(p[8 * t + 2 * e], p[8 * t + 2 * e + 1]);
              du[e] = pack_bf16x2(ds[8 * t + 2 * e], ds[8 * t + 2 * e + 1]);
              if constexpr (softmax) {
                plu[e] = pack_bf16x2(p[8 * t + 2 * e] - bf16_lo(pu[e]), p[8 * t + 2 * e + 1] - bf16_hi(pu[e]));
                dlu[e] = pack_bf16x2(ds[8 * t + 2 * e] - bf16_lo(du[e]), ds[8 * t + 2 * e + 1] - bf16_hi(du[e]));
              }
            }
            pb[t] = as_bf16x8(pu);
            db[t] = as_bf16x8(du);
            pl[t] = as_bf16x8(plu);
            dl[t] = as_bf16x8(dlu);
            // dS to the exchange tile (row = query, column = key slot) for the dQ product
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int ra = (qs * 32 + c_row(8 * t + 2 * e, g)) * (G::SXROW / 2) + spos;
              const int rb = (qs * 32 + c_row(8 * t + 2 * e + 1, g)) * (G::SXROW / 2) + spos;
              sx[ra] = (uint16_t)(du[e] & 0xFFFF);
              sx[rb] = (uint16_t)(du[e] >> 16);
              if constexpr (softmax) {
                sxl[ra] = (uint16_t)(dlu[e] & 0xFFFF);
                sxl[rb] = (uint16_t)(dlu[e] >> 16);
              }
            }
          }
#pragma unroll
          for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int drow = dt * 32 + out_perm(lc);
              const int qpos = (qs * 32 + t * 16 + g * 8) * 2;
              const bf16x8 dota = as_bf16x8(*reinterpret_cast<const u32x4*>(lds + G::OFF_DOT + drow * G::TROW + qpos));
              const bf16x8 qta = as_bf16x8(*reinterpret_cast<const u32x4*>(lds + G::OFF_QT + drow * G::TROW + qpos));
              st.dv[dt][ks] = mfma32(dota, pb[t], st.dv[dt][ks]);
              st.dk[dt][ks] = mfma32(qta, db[t], st.dk[dt][ks]);
              if constexpr (softmax) {
                st.dv[dt][ks] = mfma32(dota, pl[t], st.dv[dt][ks]);
                st.dk[dt][ks] = mfma32(qta, dl[t], st.dk[dt][ks]);
              }
            }
        }
      }
    }
    __syncthreads();  // dS exchange tile complete

    // dQ^T tiles (qs, dt) split over the waves; contraction over the active slots' keys
    for (int tile = w; tile < 2 * G::DT; tile += 4) {
      const int qs = tile % 2, dt = tile / 2;
      f32x16 acc = f32x16{};
      for (int sl = 0; sl < 4; ++sl) {
        const int blk = kmax - pmod4(kmax - sl);
        if (!(blk >= kmin && blk >= 0 && kmin <= kmax)) continue;
#pragma unroll
        for (int u = 0; u < G::KB / 16; ++u) {
          const int kpos = (sl * G::KB + u * 16 + g * 8) * 2;
          const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(
              lds + G::OFF_KT + (dt * 32 + out_perm(lc)) * G::KTROW + kpos));
          const bf16x8 sb = as_bf16x8(*reinterpret_cast<const u32x4*>(
              lds + G::OFF_SX + (qs * 32 + lc) * G::SXROW + kpos));
          acc = mfma32(ka, sb, acc);
          if constexpr (softmax) {
            const bf16x8 sl_ = as_bf16x8(*reinterpret_cast<const u32x4*>(
                lds + G::OFF_SXL + (qs * 32 + lc) * G::SXROW + kpos));
            acc = mfma32(ka, sl_, acc);
          }
        }
      }
      const int row = r0 + qs * 32 + lc;
      if (row < L) {
        u32x4 u0, u1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u0[e] = pack_bf16x2(acc[2 * e] * gd.scale, acc[2 * e + 1] * gd.scale);
          u1[e] = pack_bf16x2(acc[8 + 2 * e] * gd.scale, acc[9 + 2 * e] * gd.scale);
        }
        bf16* dst = dqseq + row * rs + dt * 32 + g * 16;
        *reinterpret_cast<u32x4*>(dst) = u0;
        *reinterpret_cast<u32x4*>(dst + 8) = u1;
      }
    }
  }
  if (cur >= 0) flush_block<D, ACT>(st, gd, dkseq, dvseq, dgseq, cur * G::KB, n);
}

template <int D, int ASET>
__device__ void bwd_dispatch_act(char* lds, const GroupDesc& gd, int b, int h) {
  if constexpr ((ASET & (1 << GDPA_ACT_GELU)) != 0)
    if (gd.act == GDPA_ACT_GELU) { bwd_item<D, GDPA_ACT_GELU>(lds, gd, b, h); return; }
  if constexpr ((ASET & (1 << GDPA_ACT_SILU)) != 0)
    if (gd.act == GDPA_ACT_SILU) { bwd_item<D, GDPA_ACT_SILU>(lds, gd, b, h); return; }
  if constexpr ((ASET & (1 << GDPA_ACT_SOFTMAX)) != 0)
    if (gd.act == GDPA_ACT_SOFTMAX) bwd_item<D, GDPA_ACT_SOFTMAX>(lds, gd, b, h);
}

template <int DSET, int ASET>
__global__ void __launch_bounds__(kThreads, 1) bwd_bf16_kernel(LaunchDesc d) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  if ((int)blockIdx.x >= d.n_items) return;
  int g, h, b;
  unpack_item(d.items[blockIdx.x], g, h, b);
  const GroupDesc gd = select_group(d, g);
  if constexpr ((DSET & kDim32) != 0)
    if (gd.head_dim == 32) { bwd_dispatch_act<32, ASET>(lds, gd, b, h); return; }
  if constexpr ((DSET & kDim64) != 0)
    if (gd.head_dim == 64) { bwd_dispatch_act<64, ASET>(lds, gd, b, h); return; }
  if constexpr ((DSET & kDim128) != 0)
    if (gd.head_dim == 128) { bwd_dispatch_act<128, ASET>(lds, gd, b, h); return; }
}

hipError_t launch_bwd_bf16(const LaunchDesc& d, int dim_set, int act_set, hipStream_t stream) {
  if (d.n_items == 0) return hipSuccess;
  const dim3 grid(d.n_items), block(kThreads);
  constexpr int kAll = (1 << GDPA_ACT_GELU) | (1 << GDPA_ACT_SILU) | (1 << GDPA_ACT_SOFTMAX);
#define GDPA_LAUNCH(DS, AS) hipLaunchKernelGGL((bwd_bf16_kernel<DS, AS>), grid, block, kBwdLdsBytes, stream, d)
#define GDPA_LAUNCH_ACTS(DS)                                          \
  switch (act_set) {                                                  \
    case 1 << GDPA_ACT_GELU: GDPA_LAUNCH(DS, 1 << GDPA_ACT_GELU); break;  \
    case 1 << GDPA_ACT_SILU: GDPA_LAUNCH(DS, 1 << GDPA_ACT_SILU); break;  \
    case 1 << GDPA_ACT_SOFTMAX: GDPA_LAUNCH(DS, 1 << GDPA_ACT_SOFTMAX); break; \
    default: GDPA_LAUNCH(DS, kAll); break;                            \
  }
  switch (dim_set) {
    case kDim32: GDPA_LAUNCH_ACTS(kDim32); break;
    case kDim64: GDPA_LAUNCH_ACTS(kDim64); break;
    case kDim128: GDPA_LAUNCH_ACTS(kDim128); break;
    case kDim32 | kDim128: GDPA_LAUNCH(kDim32 | kDim128, kAll); break;
    default: GDPA_LAUNCH(kDim32 | kDim64 | kDim128, kAll); break;
  }
#undef GDPA_LAUNCH_ACTS
#undef GDPA_LAUNCH
  return hipGetLastError();
}

}  // namespace gdpa
