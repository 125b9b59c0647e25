// GDPA backward for bf16 on gfx950: one workgroup per (sequence, head) work item.
//
//   dp_ij = <dO_i, V_j>;   ds_ij = dp_ij phi'(s_ij)   or   p_ij (dp_ij - D_i), D_i = sum_j p_ij dp_ij
//   dQ = scale dS K;   dK = scale dS^T Q;   dV = P^T dO;   dG_j = sigmoid(-G_j) sum_i ds_ij
//
// (FlashAttention-style backward that recomputes the scores tile by tile and never writes the
// score matrix to HBM: Kunlun review, section 2.3 and Figure 2. Gate: reproduction README "Core
// equations"; window: review section 2.5.)
//
// Work split inside an item: NW waves (8 when the launch holds only d <= 64 problems, giving two
// waves per SIMD; 4 when it holds d = 128), each owning one block of 32 keys: its K and V rows
// live in registers (B operands of S = Q K^T and dP = dO V^T) and its dK^T, dV^T accumulate in
// registers. The waves sweep the 64-row query tiles of the sequence together. Per query tile:
//   1. Q and dO (prefetched into registers during the previous tile) are written row-major to
//      LDS; the softmax form also stages the forward's row log-sum-exp and then computes
//      D_i = sum_j p_ij dp_ij exactly, from a pass with the query on the lane (S^T = K Q^T);
//   2. each wave: S, dP on 32x32x16 MFMA, P and dS in registers; their accumulator layout is the
//      B operand of dK^T = Q^T dS and dV^T = dO^T P, whose Q^T / dO^T operands are read straight
//      from the row-major tiles with the transposing LDS read; dS also goes to an LDS tile laid
//      out [key][query];
//   3. dQ^T = K^T dS^T over all resident keys, on 16x16x32 MFMA tiles split over the waves (K^T
//      is staged in LDS when a key block is taken; dS^T is read with the transposing read).
// Personalized-FFN form: all (<= NW * 32) keys are resident for the whole sweep. Sliding window:
// key blocks rotate through the NW wave slots as the sweep advances; a block's dK / dV / dG are
// written when it leaves the window. Every output element is written exactly once (no atomics).
#include "gdpa_device.hpp"
#include "gdpa_launch.hpp"

namespace gdpa {

template <int D, int NW_>
struct BwdGeo {
  static constexpr int NW = NW_;                // waves per workgroup
  static constexpr int THREADS = NW * kWave;
  static constexpr int KB = 32;                 // keys per wave
  static constexpr int CAP = NW * KB;           // resident keys per item
  static constexpr int QT = 64;                 // query rows per tile
  static constexpr int KK = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int CPR = D / 8;             // 16-byte chunks per row
  static constexpr int NPF = (QT * CPR + THREADS - 1) / THREADS;  // prefetch chunks per thread
  static constexpr int NROW = D * 2 + 16;       // row-major Q / dO tile row (bytes)
  static constexpr int KTROW = CAP * 2 + 16;    // K^T row: CAP keys
  static constexpr int SXROW = QT * 2 + 16;     // dS^T row (one key): 64 queries
  static constexpr int OFF_QN = 0;
  static constexpr int OFF_DON = OFF_QN + QT * NROW;
  static constexpr int OFF_KT = OFF_DON + QT * NROW;
  static constexpr int OFF_SX = OFF_KT + D * KTROW;        // dS^T (bf16; softmax: high part)
  static constexpr int OFF_SXL = OFF_SX + CAP * SXROW;     // softmax: dS - high part, in bf16
  static constexpr int OFF_ROW = OFF_SXL + CAP * SXROW;    // lse2[QT]
  static constexpr int OFF_DPART = OFF_ROW + QT * 4;       // softmax: partial D_i per wave [NW][QT]
  static constexpr int OFF_GATE = OFF_DPART + NW * QT * 4; // gate term per resident key [CAP]
  static constexpr int BYTES = OFF_GATE + CAP * 4;
};

// Waves per workgroup of a launch: 4 if it holds d = 128 problems (their register footprint
// allows one wave per SIMD), else 8.
template <int DSET>
constexpr int bwd_waves() { return (DSET & kDim128) ? 4 : 8; }

constexpr int max3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }
constexpr int kBwdLdsBytes = max3(max3(BwdGeo<32, 8>::BYTES, BwdGeo<64, 8>::BYTES, BwdGeo<32, 4>::BYTES),
                                  BwdGeo<64, 4>::BYTES, BwdGeo<128, 4>::BYTES);

template <int N>
__device__ inline int pmod(int x) { return ((x % N) + N) % N; }

template <int D, int NW>
struct BwdWave {
  using G = BwdGeo<D, NW>;
  bf16x8 kreg[G::KK];
  bf16x8 vreg[G::KK];
  f32x16 dk[G::DT];
  f32x16 dv[G::DT];
  float dgs;
  float gate;   // this lane's key: gate term (natural units; log2 units for softmax)
  float graw;   // raw G of this lane's key (for dG)
};

// Block of keys [kbase, kbase + 32): registers, K^T into the wave's LDS slot, gate terms.
template <int D, int NW, int ACT>
__device__ void take_block(BwdWave<D, NW>& st, char* lds, const GroupDesc& gd, const bf16* kseq,
                           const bf16* vseq, const float* gseq, int kbase, int n, int slot) {
  using G = BwdGeo<D, NW>;
  const int lane = lane_id(), kc = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)gd.num_heads * D;
  const int key = kbase + kc;
  const bool ok = key < n;
  const int pos = slot * G::KB + kc;
#pragma unroll
  for (int kk = 0; kk < G::KK; ++kk) {
    u32x4 ku = {0u, 0u, 0u, 0u}, vu = {0u, 0u, 0u, 0u};
    if (ok) {
      ku = *reinterpret_cast<const u32x4*>(kseq + key * rs + g * (D / 2) + kk * 8);
      vu = *reinterpret_cast<const u32x4*>(vseq + key * rs + g * (D / 2) + kk * 8);
    }
    st.kreg[kk] = as_bf16x8(ku);
    st.vreg[kk] = as_bf16x8(vu);
    // K^T: this lane's 8 d values of `key` (d = g*D/2 + kk*8 + e), keys in natural order
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
  st.gate = t;
  st.graw = gr;
  st.dgs = 0.0f;
  if (g == 0) reinterpret_cast<float*>(lds + G::OFF_GATE)[pos] = t;
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) {
    st.dk[dt] = f32x16{};
    st.dv[dt] = f32x16{};
  }
}

// Write dK, dV (and dG) of the wave's block. Accumulator register r of lane (key, g) in d-tile
// dt is d = dt*32 + c_row(r, g): four runs of 4 consecutive d per lane.
template <int D, int NW>
__device__ void flush_block(BwdWave<D, NW>& st, const GroupDesc& gd, bf16* dkseq, bf16* dvseq, float* dgseq,
                            int kbase, int n, float dv_scale) {
  using G = BwdGeo<D, NW>;
  const int lane = lane_id(), kc = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)gd.num_heads * D;
  const int key = kbase + kc;
  const float dgsum = st.dgs + __shfl_xor(st.dgs, 32);
  if (key < n) {
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = dt * 32 + a * 8 + g * 4;
        u32x2 uk, uv;
        uk[0] = pack_bf16x2(st.dk[dt][4 * a] * gd.scale, st.dk[dt][4 * a + 1] * gd.scale);
        uk[1] = pack_bf16x2(st.dk[dt][4 * a + 2] * gd.scale, st.dk[dt][4 * a + 3] * gd.scale);
        uv[0] = pack_bf16x2(st.dv[dt][4 * a] * dv_scale, st.dv[dt][4 * a + 1] * dv_scale);
        uv[1] = pack_bf16x2(st.dv[dt][4 * a + 2] * dv_scale, st.dv[dt][4 * a + 3] * dv_scale);
        *reinterpret_cast<u32x2*>(dkseq + key * rs + d) = uk;
        *reinterpret_cast<u32x2*>(dvseq + key * rs + d) = uv;
      }
    if (dgseq != nullptr && g == 0) {
      const float sg = 1.0f / (1.0f + __expf(st.graw));  // sigmoid(-G)
      dgseq[(size_t)key * gd.num_heads] = sg * dgsum;
    }
  }
}

// Registers holding the next query tile of Q and dO between its global load and its LDS store.
template <int D, int NW>
struct QTileRegs {
  u32x4 q[BwdGeo<D, NW>::NPF];
  u32x4 d[BwdGeo<D, NW>::NPF];
};

// Global loads of query tile rows [r0, r0 + QT) of Q and dO into registers (zeros past L).
template <int D, int NW>
__device__ void prefetch_qtile(QTileRegs<D, NW>& pf, const bf16* qseq, const bf16* doseq, size_t rs, int r0,
                               int L) {
  using G = BwdGeo<D, NW>;
#pragma unroll
  for (int i = 0; i < G::NPF; ++i) {
    const int idx = threadIdx.x + i * G::THREADS;
    const int r = idx / G::CPR, c = idx % G::CPR;
    const int row = r0 + r;
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (idx < G::QT * G::CPR && row < L) {
      a = *reinterpret_cast<const u32x4*>(qseq + row * rs + c * 8);
      b = *reinterpret_cast<const u32x4*>(doseq + row * rs + c * 8);
    }
    pf.q[i] = a;
    pf.d[i] = b;
  }
}

template <int D, int NW>
__device__ void store_qtile(char* lds, const QTileRegs<D, NW>& pf) {
  using G = BwdGeo<D, NW>;
#pragma unroll
  for (int i = 0; i < G::NPF; ++i) {
    const int idx = threadIdx.x + i * G::THREADS;
    if (idx < G::QT * G::CPR) {
      const int r = idx / G::CPR, c = idx % G::CPR;
      *reinterpret_cast<u32x4*>(lds + G::OFF_QN + r * G::NROW + c * 16) = pf.q[i];
      *reinterpret_cast<u32x4*>(lds + G::OFF_DON + r * G::NROW + c * 16) = pf.d[i];
    }
  }
}

// A operand (M = d, K = query) of a 32x32x16 product, read from a row-major [query][d] LDS tile
// with two transposing reads: lane (m, g) gets column d = dt*32 + m of the 8 query rows that
// B k-tile t of a C tile (rows = queries qs*32 + c_row(.)) carries in its slots (g, e), i.e.
// rows qs*32 + 16t + 8h + 4g + (0..3) for h = 0, 1.
template <int ROWBYTES>
__device__ inline bf16x8 tr_operand(const char* lds, int off, int qs, int t, int dt) {
  const int lane = lane_id(), i = lane & 15, hh = (lane >> 4) & 1, g = lane >> 5;
  const int col = dt * 32 + hh * 16 + 4 * (i & 3);
  const int row0 = qs * 32 + 16 * t + g * 4 + (i >> 2);
  const u32x2 lo = lds_read_tr16(lds, off + row0 * ROWBYTES + col * 2);
  const u32x2 hi = lds_read_tr16(lds, off + (row0 + 8) * ROWBYTES + col * 2);
  const u32x4 u = {lo[0], lo[1], hi[0], hi[1]};
  return as_bf16x8(u);
}

// GATED: the problem has a gate G (then dG may also be requested); a template parameter so that
// the ungated element-wise code is straight-line.
template <int D, int NW, int ACT, bool GATED>
__device__ void bwd_item(char* lds, const GroupDesc& gd, int b, int h) {
  using G = BwdGeo<D, NW>;
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

  if (n <= 0) {  // no keys: dQ = 0
    for (int idx = threadIdx.x; idx < L * G::CPR; idx += G::THREADS) {
      const int r = idx / G::CPR, c = idx % G::CPR;
      *reinterpret_cast<u32x4*>(dqseq + r * rs + c * 8) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  if (L <= 0) {  // no queries: dK = dV = dG = 0
    for (int idx = threadIdx.x; idx < n * G::CPR; idx += G::THREADS) {
      const int r = idx / G::CPR, c = idx % G::CPR;
      *reinterpret_cast<u32x4*>(dkseq + r * rs + c * 8) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(dvseq + r * rs + c * 8) = u32x4{0u, 0u, 0u, 0u};
    }
    if (dgseq)
      for (int r = threadIdx.x; r < n; r += G::THREADS) dgseq[(size_t)r * H] = 0.0f;
    return;
  }

  const int nkb = (n + G::KB - 1) / G::KB;
  const int ntiles = (L + G::QT - 1) / G::QT;
  BwdWave<D, NW> st;
  int cur = -1;  // key block held by this wave
  const float sc = softmax ? gd.scale * kLog2e : gd.scale;
  constexpr bool has_gate = GATED;
  const bool want_dg = GATED && dgseq != nullptr;
  // element-wise forms without a gate carry p' = phi(scale s) / scale; dV is scaled at the end
  float c1 = 0.0f, c3 = 0.0f;
  if constexpr (!softmax) PointAct<ACT>::coeffs(has_gate ? 1.0f : gd.scale, c1, c3);
  const float dv_scale = (!softmax && !has_gate) ? gd.scale : 1.0f;
  float* lse2 = reinterpret_cast<float*>(lds + G::OFF_ROW);
  float* dpart = reinterpret_cast<float*>(lds + G::OFF_DPART);
  const float* gl = reinterpret_cast<const float*>(lds + G::OFF_GATE);

  QTileRegs<D, NW> pf;
  prefetch_qtile<D, NW>(pf, qseq, doseq, rs, 0, L);

  for (int j = 0; j < ntiles; ++j) {
    const int r0 = j * G::QT;
    // active key blocks for this query tile
    int kmin = 0, kmax = nkb - 1;
    if (wl >= 0) kmin = (r0 - wl > 0 ? r0 - wl : 0) / G::KB;
    if (wr >= 0) {
      const int hi = r0 + G::QT - 1 + wr < n - 1 ? r0 + G::QT - 1 + wr : n - 1;
      kmax = hi / G::KB;
    }
    const int mine = kmax - pmod<NW>(kmax - w);
    const bool active = mine >= kmin && mine >= 0 && kmin <= kmax;
    __syncthreads();  // previous tile fully consumed (LDS tiles, dS exchange, K^T slots)
    if (active && mine != cur) {
      if (cur >= 0) flush_block<D, NW>(st, gd, dkseq, dvseq, dgseq, cur * G::KB, n, dv_scale);
      take_block<D, NW, ACT>(st, lds, gd, kseq, vseq, gseq, mine * G::KB, n, w);
      cur = mine;
    }
    store_qtile<D, NW>(lds, pf);
    if constexpr (softmax) {
      for (int r = threadIdx.x; r < G::QT; r += G::THREADS)
        lse2[r] = r0 + r < L ? lseseq[(size_t)(r0 + r) * H] * kLog2e : __builtin_inff();
    }
    if (j + 1 < ntiles) prefetch_qtile<D, NW>(pf, qseq, doseq, rs, r0 + G::QT, L);
    __syncthreads();

    if constexpr (softmax) {
      // D_i = sum_j p_ij dp_ij over all keys of row i, exactly as defined (not <dO_i, O_i> of the
      // rounded forward output). S^T = K Q^T and dP^T = V dO^T put the query on the lane, so the
      // sum over this wave's keys is a sum over registers plus one cross-half exchange; the
      // waves' partial sums are then combined in a fixed order (deterministic).
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        float part = 0.0f;
        const int rf = r0 + qs * 32, rl = rf + 31;
        const int row = rf + lc;
        if (active) {
          const int kf = mine * G::KB, kl = kf + 31;
          bool empty = kf >= n || rf >= L;
          if (wl >= 0 && kl < rf - wl) empty = true;
          if (wr >= 0 && kf > rl + wr) empty = true;
          if (!empty) {
            f32x16 st_ = f32x16{}, dpt = f32x16{};
#pragma unroll
            for (int kk = 0; kk < G::KK; ++kk) {
              const bf16x8 qb = as_bf16x8(*reinterpret_cast<const u32x4*>(
                  lds + G::OFF_QN + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
              const bf16x8 db = as_bf16x8(*reinterpret_cast<const u32x4*>(
                  lds + G::OFF_DON + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
              st_ = mfma32(st.kreg[kk], qb, st_);
              dpt = mfma32(st.vreg[kk], db, dpt);
            }
            const float l2 = lse2[qs * 32 + lc];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kloc = c_row(r, g);
              const int key = kf + kloc;
              const float x = __builtin_fmaf(st_[r], sc, gl[w * G::KB + kloc]);
              const bool ok = (key < n) & (row < L) & ((wl < 0) | (key >= row - wl)) & ((wr < 0) | (key <= row + wr));
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
      const int key = mine * G::KB + lc;             // this lane's key (sequence position)
      const int spos = (w * G::KB + lc) * G::SXROW;  // this key's dS^T row
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const int rf = r0 + qs * 32, rl = rf + 31;
        const int kf = mine * G::KB, kl = kf + 31;
        bool empty = kf >= n || rf >= L;
        if (wl >= 0 && kl < rf - wl) empty = true;
        if (wr >= 0 && kf > rl + wr) empty = true;
        bool full = kl < n && rl < L;
        if (wl >= 0 && kf < rl - wl) full = false;
        if (wr >= 0 && kl > rf + wr) full = false;
        if (empty) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int qo = (qs * 32 + a * 8 + g * 4) * 2;
            *reinterpret_cast<u32x2*>(lds + G::OFF_SX + spos + qo) = u32x2{0u, 0u};
            if constexpr (softmax) *reinterpret_cast<u32x2*>(lds + G::OFF_SXL + spos + qo) = u32x2{0u, 0u};
          }
          continue;
        }
        float lrow[16], drow[16];  // softmax: lse (log2 units) and D of the rows of register r
        if constexpr (softmax) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = qs * 32 + c_row(r, g);
            lrow[r] = lse2[rr];
            float dsum = 0.0f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) dsum += dpart[ww * G::QT + rr];
            drow[r] = dsum;
          }
        }
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < G::KK; ++kk) {
          const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(
              lds + G::OFF_QN + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
          const bf16x8 da = as_bf16x8(*reinterpret_cast<const u32x4*>(
              lds + G::OFF_DON + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
          s = mfma32(qa, st.kreg[kk], s);
          dp = mfma32(da, st.vreg[kk], dp);
        }
        // element-wise: register r is query row r0 + qs*32 + c_row(r, g), key `key`
        float p[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (softmax) {
            float x;
            if constexpr (has_gate) x = __builtin_fmaf(s[r], sc, st.gate);
            else x = s[r] * sc;
            p[r] = fast_exp2(x - lrow[r]);
            ds[r] = p[r] * (dp[r] - drow[r]);
          } else {
            float dphi;
            if constexpr (has_gate) {
              PointAct<ACT>::value_grad(__builtin_fmaf(s[r], sc, st.gate), 1.0f, c1, c3, p[r], dphi);
            } else {
              PointAct<ACT>::value_grad(s[r], sc, c1, c3, p[r], dphi);
            }
            ds[r] = dp[r] * dphi;
          }
        }
        if (!full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rf + c_row(r, g);
            const bool ok = (key < n) & (row < L) & ((wl < 0) | (key >= row - wl)) & ((wr < 0) | (key <= row + wr));
            p[r] = ok ? p[r] : 0.0f;
            ds[r] = ok ? ds[r] : 0.0f;
          }
        }
        if constexpr (GATED) if (want_dg) {
          float dsum = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) dsum += ds[r];
          st.dgs += dsum;
        }
        // P and dS as bf16 B operands (k-tile t = registers 8t..8t+7). The softmax form also
        // carries the rounding remainder as a second bf16 term (x ~ hi + lo): its products mix a
        // few large probabilities, whose bf16 rounding alone would exceed the tolerance.
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
          // dS^T to the exchange tile: registers 4a..4a+3 are 4 consecutive query rows
#pragma unroll
          for (int a2 = 0; a2 < 2; ++a2) {
            const int a = 2 * t + a2;
            const int qo = (qs * 32 + a * 8 + g * 4) * 2;
            *reinterpret_cast<u32x2*>(lds + G::OFF_SX + spos + qo) = u32x2{du[2 * a2], du[2 * a2 + 1]};
            if constexpr (softmax)
              *reinterpret_cast<u32x2*>(lds + G::OFF_SXL + spos + qo) = u32x2{dlu[2 * a2], dlu[2 * a2 + 1]};
          }
        }
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const bf16x8 dota = tr_operand<G::NROW>(lds, G::OFF_DON, qs, t, dt);
            const bf16x8 qta = tr_operand<G::NROW>(lds, G::OFF_QN, qs, t, dt);
            st.dv[dt] = mfma32(dota, pb[t], st.dv[dt]);
            st.dk[dt] = mfma32(qta, db[t], st.dk[dt]);
            if constexpr (softmax) {
              st.dv[dt] = mfma32(dota, pl[t], st.dv[dt]);
              st.dk[dt] = mfma32(qta, dl[t], st.dk[dt]);
            }
          }
      }
    }
    __syncthreads();  // dS^T tile complete

    // dQ^T = K^T dS^T on 16x16 tiles (16 d x 16 queries), split over the waves; the contraction
    // runs over the 32-key slots of the active blocks.
    {
      constexpr int DTI = D / 16;
      const int i16 = lane & 15, grp = lane >> 4;
      for (int tile = w; tile < 4 * DTI; tile += NW) {
        const int dti = tile % DTI, qti = tile / DTI;
        f32x4 acc = f32x4{};
        for (int sl = 0; sl < NW; ++sl) {
          const int blk = kmax - pmod<NW>(kmax - sl);
          if (!(blk >= kmin && blk >= 0 && kmin <= kmax)) continue;
          const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(
              lds + G::OFF_KT + (dti * 16 + i16) * G::KTROW + (sl * G::KB + grp * 8) * 2));
          // dS^T column (query qti*16 + i16) over keys sl*32 + grp*8 + 0..7
          const int krow = sl * G::KB + grp * 8 + (i16 >> 2);
          const int qcol = (qti * 16 + 4 * (i16 & 3)) * 2;
          {
            const u32x2 lo = lds_read_tr16(lds, G::OFF_SX + krow * G::SXROW + qcol);
            const u32x2 hi = lds_read_tr16(lds, G::OFF_SX + (krow + 4) * G::SXROW + qcol);
            acc = mfma16(ka, as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), acc);
          }
          if constexpr (softmax) {
            const u32x2 lo = lds_read_tr16(lds, G::OFF_SXL + krow * G::SXROW + qcol);
            const u32x2 hi = lds_read_tr16(lds, G::OFF_SXL + (krow + 4) * G::SXROW + qcol);
            acc = mfma16(ka, as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), acc);
          }
        }
        const int row = r0 + qti * 16 + i16;
        if (row < L) {
          u32x2 u;
          u[0] = pack_bf16x2(acc[0] * gd.scale, acc[1] * gd.scale);
          u[1] = pack_bf16x2(acc[2] * gd.scale, acc[3] * gd.scale);
          *reinterpret_cast<u32x2*>(dqseq + row * rs + dti * 16 + grp * 4) = u;
        }
      }
    }
  }
  if (cur >= 0) flush_block<D, NW>(st, gd, dkseq, dvseq, dgseq, cur * G::KB, n, dv_scale);
}

template <int D, int NW, int ACT>
__device__ void bwd_dispatch_gate(char* lds, const GroupDesc& gd, int b, int h) {
  if (gd.g != nullptr) bwd_item<D, NW, ACT, true>(lds, gd, b, h);
  else bwd_item<D, NW, ACT, false>(lds, gd, b, h);
}

template <int D, int NW, int ASET>
__device__ void bwd_dispatch_act(char* lds, const GroupDesc& gd, int b, int h) {
  if constexpr ((ASET & (1 << GDPA_ACT_GELU)) != 0)
    if (gd.act == GDPA_ACT_GELU) { bwd_dispatch_gate<D, NW, GDPA_ACT_GELU>(lds, gd, b, h); return; }
  if constexpr ((ASET & (1 << GDPA_ACT_SILU)) != 0)
    if (gd.act == GDPA_ACT_SILU) { bwd_dispatch_gate<D, NW, GDPA_ACT_SILU>(lds, gd, b, h); return; }
  if constexpr ((ASET & (1 << GDPA_ACT_SOFTMAX)) != 0)
    if (gd.act == GDPA_ACT_SOFTMAX) bwd_dispatch_gate<D, NW, GDPA_ACT_SOFTMAX>(lds, gd, b, h);
}

template <int DSET, int ASET>
__global__ void __launch_bounds__(bwd_waves<DSET>() * kWave, 1) bwd_bf16_kernel(LaunchDesc d) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int NW = bwd_waves<DSET>();
  if ((int)blockIdx.x >= d.n_items) return;
  int g, h, b;
  unpack_item(d.items[blockIdx.x], g, h, b);
  if (g >= d.n_groups) return;
  const GroupDesc gd = select_group(d, g);
  if (b >= gd.num_seqs || h >= gd.num_heads) return;  // list built for another shape
  if constexpr ((DSET & kDim32) != 0)
    if (gd.head_dim == 32) { bwd_dispatch_act<32, NW, ASET>(lds, gd, b, h); return; }
  if constexpr ((DSET & kDim64) != 0)
    if (gd.head_dim == 64) { bwd_dispatch_act<64, NW, ASET>(lds, gd, b, h); return; }
  if constexpr ((DSET & kDim128) != 0)
    if (gd.head_dim == 128) { bwd_dispatch_act<128, NW, ASET>(lds, gd, b, h); return; }
}

hipError_t launch_bwd_bf16(const LaunchDesc& d, int dim_set, int act_set, hipStream_t stream) {
  if (d.n_items == 0) return hipSuccess;
  const dim3 grid(d.n_items);
  constexpr int kAll = (1 << GDPA_ACT_GELU) | (1 << GDPA_ACT_SILU) | (1 << GDPA_ACT_SOFTMAX);
#define GDPA_LAUNCH(DS, AS) \
  hipLaunchKernelGGL((bwd_bf16_kernel<DS, AS>), grid, dim3(bwd_waves<DS>() * kWave), kBwdLdsBytes, stream, d)
#define GDPA_LAUNCH_ACTS(DS)                                                   \
  switch (act_set) {                                                           \
    case 1 << GDPA_ACT_GELU: GDPA_LAUNCH(DS, 1 << GDPA_ACT_GELU); break;       \
    case 1 << GDPA_ACT_SILU: GDPA_LAUNCH(DS, 1 << GDPA_ACT_SILU); break;       \
    case 1 << GDPA_ACT_SOFTMAX: GDPA_LAUNCH(DS, 1 << GDPA_ACT_SOFTMAX); break; \
    default: GDPA_LAUNCH(DS, kAll); break;                                     \
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
