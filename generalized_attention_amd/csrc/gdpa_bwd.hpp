// GDPA backward for bf16 on gfx950: one workgroup per (sequence, head): 8 waves (two per SIMD) for
// the element-wise forms at d <= 64, else 4 (one per SIMD).
//
//   dp_ij = <dO_i, V_j>;   ds_ij = dp_ij phi'(s_ij)   or   p_ij (dp_ij - D_i), D_i = sum_j p_ij dp_ij
//   dQ = scale dS K;   dK = scale dS^T Q;   dV = P^T dO;   dG_j = sigmoid(-G_j) sum_i ds_ij
//
// (Block-wise backward that recomputes the scores tile by tile and never writes the score matrix
// to HBM: Kunlun review, section 2.3 and Figure 2. Gate: reproduction README "Core equations";
// window: review section 2.5.)
//
// Work split inside an item. The keys are cut into blocks of 32; block b lives in ring slot
// b mod NB, slot s belongs to wave s mod 4. A wave therefore owns KB = 2 blocks (1 at d = 128):
// their K and V rows stay in registers (B operands of S = Q K^T and dP = dO V^T) and their
// dK^T, dV^T accumulate in registers for the whole sweep over the 64-row query tiles. Per tile:
//   1. Blocks entering the window are taken (K^T of a new block goes to an LDS staging area).
//      Q and dO of a tile are loaded from HBM two tiles ahead and stored row-major into LDS
//      while the previous tile's dQ runs.
//   2. Softmax only: D_i = sum_j p_ij dp_ij exactly, from a pass with the query on the lane
//      (S^T = K Q^T, dP^T = V dO^T); the waves' partial sums meet in LDS.
//   3. Each wave, per 32-row half and owned block: S, dP on 32x32x16 MFMA; P and dS in fp32
//      registers; their accumulator layout is the B operand of dV^T = dO^T P and dK^T = Q^T dS,
//      whose dO^T / Q^T operands come from the row-major tiles by the transposing LDS read
//      (loaded once per half and reused for both owned blocks). dS also goes to LDS as
//      [key][query].
//   4. dQ^T = K^T dS^T on 32x32x16 MFMA: each wave owns a 32(d) x 32(query) output tile (two at
//      d = 128); K^T comes from the staging area, dS^T by the transposing LDS read.
// Every wave runs on its own SIMD, so the wave's own instruction stream overlaps MFMA with the
// element-wise VALU work. Every output element is written exactly once (no atomics).
#pragma once

#include <type_traits>

#include "gdpa_device.hpp"
#include "gdpa_launch.hpp"

namespace gdpa {

// NWAVES waves per workgroup: 4 (one per SIMD; 64 keys per wave, 32 at d = 128) or 8 (two per
// SIMD, 32 keys each; element-wise forms at d <= 64). Either way the workgroup holds
// bwd_capacity(D) keys.
template <int D, int NWAVES>
struct BwdGeo {
  static constexpr int NW = NWAVES;
  static constexpr int THREADS = NW * kWave;
  static constexpr int KPW = NW == 8 ? kBwdKeyBlock : bwd_keys_per_wave(D);
  static constexpr int KB = KPW / kBwdKeyBlock;    // blocks per wave
  static constexpr int NB = NW * KB;               // ring slots
  static constexpr int CAP = NB * kBwdKeyBlock;    // resident keys
  static constexpr int QT = kBwdQueryTile;
  static constexpr int KK = D / 16;                // MFMA k-steps over d
  static constexpr int DT = D / 32;                // 32-wide d tiles
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int NPF = (QT * CPR + THREADS - 1) / THREADS;  // prefetch chunks per thread
  // dQ^T output tiles (32 d x 32 queries): DT x 2; wave w takes d-tile w % DT and QH query halves
  static constexpr int QH = (2 * DT >= NW) ? 2 * DT / NW : 1;
  static constexpr int NROW = D * 2 + 16;          // row-major Q / dO tile row (bytes)
  static constexpr int KTROW = CAP * 2 + 16;       // K^T staging row: CAP keys
  static constexpr int SXROW = QT * 2 + 16;        // dS^T row (one key): QT queries
  static constexpr int OFF_QN = 0;
  static constexpr int OFF_DON = OFF_QN + QT * NROW;
  static constexpr int OFF_KT = OFF_DON + QT * NROW;
  static constexpr int OFF_SX = OFF_KT + D * KTROW;         // dS^T (bf16; softmax: high part)
  static constexpr int OFF_SXL = OFF_SX + CAP * SXROW;      // softmax: dS - high part, in bf16
  static constexpr int OFF_ROW = OFF_SXL + CAP * SXROW;     // lse2[QT] (log2 units)
  static constexpr int OFF_DPART = OFF_ROW + QT * 4;        // softmax: partial D_i per wave [NW][QT]
  static constexpr int OFF_GATE = OFF_DPART + NW * QT * 4;  // gate term per ring position [CAP]
  // 8 waves: a second Q / dO tile buffer (the next tile is stored during the current one)
  static constexpr int QBUFS = NW == 8 ? 2 : 1;
  static constexpr int OFF_QN1 = OFF_GATE + CAP * 4;
  static constexpr int OFF_DON1 = OFF_QN1 + QT * NROW;
  // [2][NW][4] max ||q||^2 of the tile rows each row of 16 lanes of a staging wave stored
  static constexpr int OFF_QNRM = QBUFS == 2 ? OFF_DON1 + QT * NROW : OFF_GATE + CAP * 4;
  static constexpr int BYTES = OFF_QNRM + 2 * NW * 4 * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
  static_assert(CAP == bwd_capacity(D), "resident keys per workgroup");
  static_assert(NW == 4 || D <= 64, "8 waves only for d <= 64");
};

constexpr int max3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }
template <int DSET, int ASET>
constexpr int bwd_lds_bytes() {
  constexpr int NW = bwd_waves<DSET, ASET>();
  return max3((DSET & kDim32) ? BwdGeo<32, NW>::BYTES : 0, (DSET & kDim64) ? BwdGeo<64, NW>::BYTES : 0,
              (DSET & kDim128) ? BwdGeo<128, 4>::BYTES : 0);
}

template <int N>
__device__ inline int pmod(int x) { return ((x % N) + N) % N; }

__device__ inline u32x4 as_u32x4(const bf16x8& b) { return __builtin_bit_cast(u32x4, b); }

// Per-wave state of its owned blocks.
template <int D, int NW>
struct BwdWave {
  using G = BwdGeo<D, NW>;
  bf16x8 kreg[G::KB][G::KK];
  bf16x8 vreg[G::KB][G::KK];
  f32x16 dk[G::KB][G::DT];
  f32x16 dv[G::KB][G::DT];
  float dgs[G::KB];
  float gate[G::KB];   // this lane's key: gate term (natural units; log2 units for softmax)
  float graw[G::KB];   // raw G of this lane's key (for dG)
  float kn2[G::KB];    // largest ||k||^2 of each owned block's keys (uniform)
  int cur[G::KB];      // block held in each owned slot (-1: none); uniform
};

// A block's K and V rows (this lane's 8-value pieces) and raw gate between the global loads and
// their commit into an owned slot.
template <int D, int NW>
struct TakeRegs {
  u32x4 k[BwdGeo<D, NW>::KK];
  u32x4 v[BwdGeo<D, NW>::KK];
  float graw;
};

template <int D, int NW>
__device__ __forceinline__ void take_load(TakeRegs<D, NW>& tr, const GroupDesc& gd, const bf16* kseq, const bf16* vseq,
                                          const float* gseq, int blk, int n) {
  using G = BwdGeo<D, NW>;
  const int lane = lane_id(), kc = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)gd.num_heads * D;
  const int key = blk * kBwdKeyBlock + kc;
  const bool ok = key < n;
#pragma unroll
  for (int kk = 0; kk < G::KK; ++kk) {
    tr.k[kk] = u32x4{0u, 0u, 0u, 0u};
    tr.v[kk] = u32x4{0u, 0u, 0u, 0u};
    if (ok) {
      tr.k[kk] = *reinterpret_cast<const u32x4*>(kseq + key * rs + g * (D / 2) + kk * 8);
      tr.v[kk] = *reinterpret_cast<const u32x4*>(vseq + key * rs + g * (D / 2) + kk * 8);
    }
  }
  tr.graw = (gseq != nullptr && ok) ? gseq[(size_t)key * gd.num_heads] : 0.0f;
}

// Commit loaded rows into owned slot kb (ring slot s): K/V rows into registers, K^T into the LDS
// staging area, gate terms; zero the block's accumulators.
template <int D, int NW, int ACT>
__device__ __forceinline__ void take_commit(BwdWave<D, NW>& st, int kb, char* lds, const TakeRegs<D, NW>& tr, bool gated,
                                            int s) {
  using G = BwdGeo<D, NW>;
  const int lane = lane_id(), kc = lane & 31, g = lane >> 5;
  const int pos = s * kBwdKeyBlock + kc;
#pragma unroll
  for (int kk = 0; kk < G::KK; ++kk) {
    const u32x4 ku = tr.k[kk];
    st.kreg[kb][kk] = as_bf16x8(ku);
    st.vreg[kb][kk] = as_bf16x8(tr.v[kk]);
    // K^T staging: this lane's 8 d values of its key (d = g*D/2 + kk*8 + e), keys in ring order
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d0 = g * (D / 2) + kk * 8 + 2 * e;
      *reinterpret_cast<uint16_t*>(lds + G::OFF_KT + d0 * G::KTROW + pos * 2) = (uint16_t)(ku[e] & 0xFFFF);
      *reinterpret_cast<uint16_t*>(lds + G::OFF_KT + (d0 + 1) * G::KTROW + pos * 2) = (uint16_t)(ku[e] >> 16);
    }
  }
  float t = 0.0f;
  if (gated) {
    t = log_sigmoid_f(tr.graw);
    if (ACT == GDPA_ACT_SOFTMAX) t *= kLog2e;
  }
  st.gate[kb] = t;
  st.graw[kb] = tr.graw;
  st.dgs[kb] = 0.0f;
  if constexpr (ACT != GDPA_ACT_SOFTMAX) {
    // the block's largest ||k||^2 (the series bound of ungated element-wise tiles); the lane holds
    // half of its key's row, the other half sits 32 lanes away
    float n2 = 0.0f;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) n2 += sumsq_bf16x8(tr.k[kk]);
    // (8 waves: without LDS round trips; the 4-wave kernels keep the shuffles, since this compiler
    // crashes on them with DPP)
    st.kn2[kb] = NW == 8 ? wave_max_lanes(half32_sum(n2)) : wave_max(n2 + __shfl_xor(n2, 32, 64));
  }
  if (g == 0) reinterpret_cast<float*>(lds + G::OFF_GATE)[pos] = t;
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) {
    st.dk[kb][dt] = f32x16{};
    st.dv[kb][dt] = f32x16{};
  }
}

// Load block `blk`'s K and V rows straight into owned slot kb's registers (the slot's previous
// block must no longer be read) and its raw gate into graw_next; take_commit_regs completes it.
template <int D, int NW>
__device__ __forceinline__ void take_load_regs(BwdWave<D, NW>& st, int kb, float& graw_next, const GroupDesc& gd,
                                               const bf16* kseq, const bf16* vseq, const float* gseq, int blk,
                                               int n) {
  using G = BwdGeo<D, NW>;
  const int lane = lane_id(), kc = lane & 31, g = lane >> 5;
  const size_t rs = (size_t)gd.num_heads * D;
  const int key = blk * kBwdKeyBlock + kc;
  const bool ok = key < n;
#pragma unroll
  for (int kk = 0; kk < G::KK; ++kk) {
    u32x4 ku = {0u, 0u, 0u, 0u}, vu = {0u, 0u, 0u, 0u};
    if (ok) {
      ku = *reinterpret_cast<const u32x4*>(kseq + key * rs + g * (D / 2) + kk * 8);
      vu = *reinterpret_cast<const u32x4*>(vseq + key * rs + g * (D / 2) + kk * 8);
    }
    st.kreg[kb][kk] = as_bf16x8(ku);
    st.vreg[kb][kk] = as_bf16x8(vu);
  }
  graw_next = (gseq != nullptr && ok) ? gseq[(size_t)key * gd.num_heads] : 0.0f;
}

template <int D, int NW, int ACT>
__device__ __forceinline__ void take_commit_regs(BwdWave<D, NW>& st, int kb, char* lds, float graw, bool gated, int s) {
  TakeRegs<D, NW> tr;
#pragma unroll
  for (int kk = 0; kk < BwdGeo<D, NW>::KK; ++kk) {
    tr.k[kk] = as_u32x4(st.kreg[kb][kk]);
    tr.v[kk] = as_u32x4(st.vreg[kb][kk]);
  }
  tr.graw = graw;
  take_commit<D, NW, ACT>(st, kb, lds, tr, gated, s);
}

// Take block `blk` into owned slot kb (ring slot s).
template <int D, int NW, int ACT>
__device__ __forceinline__ void take_block(BwdWave<D, NW>& st, int kb, char* lds, const GroupDesc& gd, const bf16* kseq,
                           const bf16* vseq, const float* gseq, int blk, int n, int s) {
  TakeRegs<D, NW> tr;
  take_load<D, NW>(tr, gd, kseq, vseq, gseq, blk, n);
  take_commit<D, NW, ACT>(st, kb, lds, tr, gseq != nullptr, s);
}

// Write dK, dV (and dG) of owned slot kb. Accumulator register r of lane (key, g) in d-tile dt is
// d = dt*32 + c_row(r, g): four runs of 4 consecutive d per lane.
template <int D, int NW>
__device__ __forceinline__ void flush_block(BwdWave<D, NW>& st, int kb, const GroupDesc& gd, OutPtr dkseq, OutPtr dvseq,
                                            float* dgseq, int n, float dv_scale) {
  using G = BwdGeo<D, NW>;
  const int lane = lane_id(), kc = lane & 31, g = lane >> 5;
  const int key = st.cur[kb] * kBwdKeyBlock + kc;  // sequence-local key of this lane
  const float dgsum = st.dgs[kb] + __shfl_xor(st.dgs[kb], 32);
  const size_t rs = (size_t)gd.num_heads * D;
  if (key < n) {
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const size_t e = key * rs + dt * 32 + a * 8 + g * 4;
        const f32x16& k = st.dk[kb][dt];
        const f32x16& v = st.dv[kb][dt];
        out_store4(dkseq + e, f32x4{k[4 * a], k[4 * a + 1], k[4 * a + 2], k[4 * a + 3]} * gd.scale);
        out_store4(dvseq + e, f32x4{v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]} * dv_scale);
      }
    // sigmoid(-G) * sum_i ds_ij
    if (dgseq != nullptr && g == 0) dgseq[(size_t)key * gd.num_heads] = (1.0f / (1.0f + __expf(st.graw[kb]))) * dgsum;
  }
}

// Registers holding the next query tile of Q and dO (and its lse) between the global load and
// the LDS store.
template <int D, int NW>
struct QTileRegs {
  u32x4 q[BwdGeo<D, NW>::NPF];
  u32x4 d[BwdGeo<D, NW>::NPF];
  float lse;
  float dsum;  // key-chunked softmax: the row term D_i from the workspace
};

// DSUM: also load the row term D_i (key-chunked softmax main pass).
template <int D, int NW, bool SOFTMAX, bool DSUM = false>
__device__ void prefetch_qtile(QTileRegs<D, NW>& pf, const bf16* qseq, const bf16* doseq, const float* lseseq,
                               size_t rs, int H, int r0, int L, const float* dsumseq = nullptr) {
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
  if constexpr (SOFTMAX) {
    const int row = r0 + (int)threadIdx.x;
    pf.lse = (threadIdx.x < G::QT && row < L) ? lseseq[(size_t)row * H] * kLog2e : __builtin_inff();
    if constexpr (DSUM) pf.dsum = (threadIdx.x < G::QT && row < L) ? dsumseq[(size_t)row * H] : 0.0f;
  }
}

// buf: which Q / dO tile buffer (the second exists with 8 waves).
// QNORM: each row of 16 lanes also writes the largest ||q||^2 of the tile rows it stored to
// G::OFF_QNRM + 4 (4 (buf * NW + w) + lane / 16) (the series bound of ungated element-wise tiles).
// With 8 waves the row sums and maxima stay inside rows of 16 lanes (DPP, no LDS round trip on
// the tile's critical path); the 4-wave kernels take the wave's maximum by shuffles and write it
// from four lanes.
template <int D, int NW, bool SOFTMAX, bool DSUM = false, bool QNORM = false>
__device__ void store_qtile(char* lds, const QTileRegs<D, NW>& pf, int buf = 0) {
  using G = BwdGeo<D, NW>;
  const int qoff = buf ? G::OFF_QN1 : G::OFF_QN, doff = buf ? G::OFF_DON1 : G::OFF_DON;
  if constexpr (QNORM) {
    // a row's CPR chunks sit in CPR consecutive lanes (rows past the end hold zeros)
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < G::NPF; ++i) {
      float n2 = sumsq_bf16x8(pf.q[i]);
      if constexpr (NW == 8) {
        n2 = group_sum<G::CPR>(n2);
      } else {
#pragma unroll
        for (int off = 1; off < G::CPR; off <<= 1) n2 += __shfl_xor(n2, off, 64);
      }
      m = fmaxf(m, n2);
    }
    m = NW == 8 ? row16_max(m) : wave_max(m);
    if ((lane_id() & 15) == 0)
      reinterpret_cast<float*>(lds + G::OFF_QNRM)[(buf * NW + (threadIdx.x >> 6)) * 4 + (lane_id() >> 4)] = m;
  }
#pragma unroll
  for (int i = 0; i < G::NPF; ++i) {
    const int idx = threadIdx.x + i * G::THREADS;
    if (idx < G::QT * G::CPR) {
      const int r = idx / G::CPR, c = idx % G::CPR;
      *reinterpret_cast<u32x4*>(lds + qoff + r * G::NROW + c * 16) = pf.q[i];
      *reinterpret_cast<u32x4*>(lds + doff + r * G::NROW + c * 16) = pf.d[i];
    }
  }
  if constexpr (SOFTMAX)
    if (threadIdx.x < G::QT) {
      reinterpret_cast<float*>(lds + G::OFF_ROW)[threadIdx.x] = pf.lse;
      if constexpr (DSUM) reinterpret_cast<float*>(lds + G::OFF_DPART)[threadIdx.x] = pf.dsum;
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

// B operand (K = 16 keys, N = 32 queries) of dQ^T = K^T dS^T, read from the [key][query] dS^T
// tile with two transposing reads: lane (n, g) gets query qh*32 + n, keys kbase + 8g + (0..7).
template <int SXROW>
__device__ inline bf16x8 sx_operand(const char* lds, int off, int kbase, int qh) {
  const int lane = lane_id(), i = lane & 15, hh = (lane >> 4) & 1, g = lane >> 5;
  const int row = kbase + g * 8 + (i >> 2);
  const int col = qh * 32 + hh * 16 + 4 * (i & 3);
  const u32x2 lo = lds_read_tr16(lds, off + row * SXROW + col * 2);
  const u32x2 hi = lds_read_tr16(lds, off + (row + 4) * SXROW + col * 2);
  const u32x4 u = {lo[0], lo[1], hi[0], hi[1]};
  return as_bf16x8(u);
}

// Which rows / keys of the (query half, key block) pair are allowed.
struct BlockMask {
  bool empty;  // no allowed entry (skip)
  bool full;   // every entry allowed (no mask needed)
};
__device__ inline BlockMask block_mask(int kf, int rf, int n, int L, int wl, int wr) {
  const int kl = kf + 31, rl = rf + 31;
  BlockMask m;
  m.empty = kf >= n || rf >= L;
  if (wl >= 0 && kl < rf - wl) m.empty = true;
  if (wr >= 0 && kf > rl + wr) m.empty = true;
  m.full = kl < n && rl < L;
  if (wl >= 0 && kf < rl - wl) m.full = false;
  if (wr >= 0 && kl > rf + wr) m.full = false;
  return m;
}

// Pointers and scalars of one (sequence, head) item.
struct BwdItem {
  const bf16* qseq;
  const bf16* doseq;
  const float* lseseq;
  OutPtr dqseq;
  const bf16* kseq;
  const bf16* vseq;
  const float* gseq;
  OutPtr dkseq;
  OutPtr dvseq;
  float* dgseq;
  float* dq32seq;      // key chunks: fp32 dQ rows of this item (row stride rs)
  float* dsumseq;      // key chunks, softmax: D_i of this item's rows (row stride H)
  size_t rs;
  int H, L, n, wl, wr;
  int kofs;            // sequence position of the item's first key (key chunk start)
  int ntot;            // keys of the whole sequence
  int t0, t1;          // query tiles [t0, t1) swept
  bool shared_q;       // dQ rows are per-sequence partials of a shared query matrix
};

// Key chunks of kchunk keys: which chunks a query row's keys fall in (first, last), under the
// window; a row sees no key when first > last.
__device__ inline void row_chunks(int row, int ntot, int wl, int wr, int kchunk, int& first, int& last) {
  const int lo = (wl >= 0 && row - wl > 0) ? row - wl : 0;
  const int hi = (wr >= 0 && row + wr < ntot - 1) ? row + wr : ntot - 1;
  first = lo / kchunk;
  last = hi >= lo ? hi / kchunk : first - 1;
}

// The sweep over the query tiles of one item. KACT: owned blocks processed per wave (KB, or 1
// when every key of the item fits in one block per wave). The per-block work runs without
// branches around the MFMA accumulations (a skipped block contributes zero operands), which keeps
// the dK / dV accumulators in place in the register file; only the element-wise work is skipped.
// GATED: the problem has a gate G (then dG may also be requested).
// WINDOWED: bounded window whose keys stream through the ring slots as the tiles advance.
// CHUNK: 0 = the item's keys are all resident; 1 = one chunk of CAP keys starting at it.kofs, dQ
// accumulated over the chunks in fp32 workspace rows (softmax: D_i read from the workspace);
// 2 = softmax row-term pass over one chunk: only D_i, accumulated into the workspace.
// SPLIT: an element-wise item whose keys are all resident, with at most kSplitTerms rows or keys:
// P and dS enter the dV, dK and dQ products as a high + low bf16 pair like the softmax form's.
// Masks are applied, so a windowed item whose keys are all resident runs here too. (Key chunks of
// an element-wise item with that few rows take the pair in dV and dK by a uniform branch: their
// dQ sums run over more keys than a chunk holds.)
template <int D, int NW, int ACT, bool GATED, int KACT, bool WINDOWED, int CHUNK = 0, bool SPLIT = false>
__device__ __forceinline__ void bwd_sweep(char* lds, const GroupDesc& gd, const BwdItem& it) {
  using G = BwdGeo<D, NW>;
  constexpr int NS = G::NW * KACT;  // ring slots in use
  const int L = it.L, n = it.n, wl = it.wl, wr = it.wr, H = it.H;
  const size_t rs = it.rs;
  const int w = wave_id(), lane = lane_id(), lc = lane & 31, g = lane >> 5;
  constexpr bool softmax = ACT == GDPA_ACT_SOFTMAX;
  static_assert(CHUNK != 2 || softmax, "row-term pass is softmax only");
  static_assert(CHUNK == 0 || (!WINDOWED && KACT == G::KB), "key chunks hold every block");
  // entries need explicit masks in the softmax form, inside a window or in a key chunk; without
  // a window every block is resident for the whole sweep (taken once, before it)
  constexpr bool MASKED = softmax || WINDOWED || CHUNK != 0 || SPLIT;
  // P and dS as a high + low bf16 pair in dV / dK, and dS in dQ (the softmax form always;
  // element-wise items with few rows / few keys)
  constexpr bool split = softmax || SPLIT;
  constexpr bool split_dq = split;
  // element-wise key chunks of an item with few rows (or split operands asked for): the pair in
  // dV / dK only (uniform)
  const bool chunk_rows_split = !split && CHUNK == 1 && (it.L <= kSplitTerms || gd.split_all);
  constexpr bool DSUM = CHUNK == 1 && softmax;  // D_i comes from the workspace
  // keys are chunk-local below; masks compare sequence positions kofs + key with the rows
  const int kofs = CHUNK ? it.kofs : 0;
  const int nkb = (n + kBwdKeyBlock - 1) / kBwdKeyBlock;
  const int t0 = it.t0, t1 = it.t1;

  BwdWave<D, NW> st;
#pragma unroll
  for (int kb = 0; kb < G::KB; ++kb) {
    st.cur[kb] = -1;
    st.gate[kb] = 0.0f;
    st.graw[kb] = 0.0f;
    st.dgs[kb] = 0.0f;
    st.kn2[kb] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) {
      st.kreg[kb][kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      st.vreg[kb][kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt) {
      st.dk[kb][dt] = f32x16{};
      st.dv[kb][dt] = f32x16{};
    }
  }
  const int dtile = w % G::DT;
  const int qh_first = (G::QH == 2) ? 0 : w / G::DT;  // query half of this wave's dQ tile
  const bool dq_role = qh_first < 2;

  const float sc = softmax ? gd.scale * kLog2e : gd.scale;
  constexpr bool has_gate = GATED;
  const bool want_dg = GATED && it.dgseq != nullptr;
  // element-wise forms without a gate carry p' = phi(scale s) / scale; dV is scaled at the end
  float c1 = 0.0f, c3 = 0.0f;
  if constexpr (!softmax) PointAct<ACT>::coeffs(has_gate ? 1.0f : gd.scale, c1, c3);
  // ungated element-wise tiles whose arguments are all proven within the series range (tile rows'
  // largest ||q||^2 from the staging waves, the wave's keys' largest ||k||^2) take SeriesAct
  constexpr bool kSeries = !softmax && !GATED;
  float a1 = 0.0f, a3 = 0.0f, d1 = 0.0f, d3 = 0.0f;
  if constexpr (kSeries) SeriesAct<ACT>::coeffs(gd.scale, a1, a3, d1, d3);
  const float dv_scale = (!softmax && !has_gate) ? gd.scale : 1.0f;
  const float* lse2 = reinterpret_cast<const float*>(lds + G::OFF_ROW);
  float* dpart = reinterpret_cast<float*>(lds + G::OFF_DPART);
  const float* gl = reinterpret_cast<const float*>(lds + G::OFF_GATE);

  // K^T staging of slots never taken must hold finite values (they meet zero dS in dQ); without a
  // window, an item (or chunk) with a block for every slot takes them all
  if (WINDOWED || nkb < NS)
    for (int idx = threadIdx.x; idx < D * (G::KTROW / 16); idx += G::THREADS)
      reinterpret_cast<u32x4*>(lds + G::OFF_KT)[idx] = u32x4{0u, 0u, 0u, 0u};
  QTileRegs<D, NW> pf;
  prefetch_qtile<D, NW, softmax, DSUM>(pf, it.qseq, it.doseq, it.lseseq, rs, H, t0 * G::QT, L, it.dsumseq);
  // without a window every block of the sequence is resident for the whole sweep: its K / V rows
  // are loaded here, in flight together with the first tile (one memory latency, not two)
  TakeRegs<D, NW> kv[KACT];
  if constexpr (!WINDOWED) {
#pragma unroll
    for (int kb = 0; kb < KACT; ++kb) {
      const int s = kb * G::NW + w;
      if (s < nkb) take_load<D, NW>(kv[kb], gd, it.kseq, it.vseq, it.gseq, s, n);
    }
  }
  __syncthreads();  // K^T staging zeroed
  store_qtile<D, NW, softmax, DSUM, kSeries>(lds, pf);  // first tile
  if (t0 + 1 < t1)
    prefetch_qtile<D, NW, softmax, DSUM>(pf, it.qseq, it.doseq, it.lseseq, rs, H, (t0 + 1) * G::QT, L, it.dsumseq);
  if constexpr (!WINDOWED) {
#pragma unroll
    for (int kb = 0; kb < KACT; ++kb) {
      const int s = kb * G::NW + w;
      if (s < nkb) {
        take_commit<D, NW, ACT>(st, kb, lds, kv[kb], it.gseq != nullptr, s);
        st.cur[kb] = s;
      }
    }
  }

  // windowed sweep: the rows of a block entering at the next tile are loaded into its slot's
  // registers at the end of this tile's main pass (before this tile's dQ and dK / dV stores, so
  // waiting for them never waits for a store); the next tile commits them
  int pend[KACT];
  float gnext[KACT];
#pragma unroll
  for (int kb = 0; kb < KACT; ++kb) {
    pend[kb] = -1;
    gnext[kb] = 0.0f;
  }
  // blocks of tile jj: block held by owned slot kb, and whether the tile touches it
  auto tile_blocks = [&](int jj, int (&bl)[KACT], bool (&ac)[KACT]) {
    const int rr = jj * G::QT;
    int klo = 0, khi = n - 1;
    if (wl >= 0 && rr - wl - kofs > 0) klo = rr - wl - kofs;
    if (wr >= 0 && rr + G::QT - 1 + wr - kofs < n - 1) khi = rr + G::QT - 1 + wr - kofs;
    const bool any = klo <= khi;
    const int kmn = klo / kBwdKeyBlock, kmx = any ? khi / kBwdKeyBlock : -1;
#pragma unroll
    for (int kb = 0; kb < KACT; ++kb) {
      const int s = kb * G::NW + w;
      bl[kb] = kmx - pmod<NS>(kmx - s);
      ac[kb] = any && bl[kb] >= kmn && bl[kb] >= 0;
    }
  };

  // Eight waves, element-wise forms over resident keys: the waves with a dQ tile compute the
  // previous tile's dQ right after their main pass, in the time the other wave of their SIMD still
  // needs for its own main pass, instead of after the barrier; dS^T alternates between the two
  // exchange areas (the second is free without softmax).
  constexpr bool FQ = G::NW == 8 && !split && !WINDOWED && CHUNK == 0 && G::QH == 1;
  constexpr int NK = 2 * NS;                       // 16-key steps of one dQ tile
  const int drow = dtile * 32 + out_perm(lc);      // K^T row carried by this lane's A-operand row
  auto dq_tile = [&](int sxoff) {
    f32x16 a2[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(lds + G::OFF_KT + drow * G::KTROW + (k * 16 + g * 8) * 2));
      a2[k & 1] = mfma32(ka, sx_operand<G::SXROW>(lds, sxoff, k * 16, qh_first), a2[k & 1]);
    }
    return a2[0] + a2[1];
  };
  auto dq_store = [&](const f32x16& acc, int rbase) {
    const int row = rbase + qh_first * 32 + lc;
    if (row < L) out_store16(it.dqseq + (row * rs + dtile * 32 + g * 16), acc, gd.scale);
  };

  for (int j = t0; j < t1; ++j) {
    const int r0 = j * G::QT;
    f32x16 fq;  // FQ: the previous tile's dQ tile
    // ---- 1. take the blocks entering the window (all LDS readers of the previous tile are done)
    int blk[KACT];
    bool act[KACT];
    tile_blocks(j, blk, act);
    if constexpr (WINDOWED) {
#pragma unroll
      for (int kb = 0; kb < KACT; ++kb) {
        if (pend[kb] >= 0) {
          // rows loaded during the previous tile: K^T staging, gate, fresh accumulators
          take_commit_regs<D, NW, ACT>(st, kb, lds, gnext[kb], it.gseq != nullptr, kb * G::NW + w);
          st.cur[kb] = pend[kb];
          pend[kb] = -1;
        } else if (act[kb] && blk[kb] != st.cur[kb]) {  // first tile of the sweep
          take_block<D, NW, ACT>(st, kb, lds, gd, it.kseq, it.vseq, it.gseq, blk[kb], n, kb * G::NW + w);
          st.cur[kb] = blk[kb];
        }
      }
    }
    if (WINDOWED || j == t0) __syncthreads();  // tile, lse, K^T staging and gate terms visible

    // ---- 2. softmax: D_i = sum_j p_ij dp_ij, exactly as defined (not <dO_i, O_i> of the rounded
    // forward output). S^T = K Q^T and dP^T = V dO^T put the query on the lane; the waves' partial
    // sums are combined in a fixed order (deterministic).
    if constexpr (softmax && !DSUM) {
      // iteration it = (query half qs, owned block kb); the products of it+1 are issued before the
      // element-wise work of it (the main pass's registers are free here)
      constexpr int NIT = 2 * KACT;
      bf16x8 qb[G::KK], db[G::KK];
      f32x16 st2[2], dp2[2];
      auto load_b = [&](int qs) {
#pragma unroll
        for (int kk = 0; kk < G::KK; ++kk) {
          qb[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(lds + G::OFF_QN + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
          db[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(lds + G::OFF_DON + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
        }
      };
      auto issue = [&](int kb, int slot) {
        st2[slot] = f32x16{};
        dp2[slot] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < G::KK; ++kk) {
          st2[slot] = mfma32(st.kreg[kb][kk], qb[kk], st2[slot]);
          dp2[slot] = mfma32(st.vreg[kb][kk], db[kk], dp2[slot]);
        }
      };
      load_b(0);
      issue(0, 0);
      float part = 0.0f, l2 = lse2[lc];
#pragma unroll
      for (int it2 = 0; it2 < NIT; ++it2) {
        const int qs = it2 / KACT, kb = it2 % KACT, cs = it2 & 1;
        if (it2 + 1 < NIT) {
          if ((it2 + 1) / KACT != qs) load_b((it2 + 1) / KACT);
          issue((it2 + 1) % KACT, cs ^ 1);
        }
        const int rf = r0 + qs * 32;
        const int row = rf + lc;
        const int kf = blk[kb] * kBwdKeyBlock;
        const BlockMask bm = block_mask(kofs + kf, rf, kofs + n, L, wl, wr);
        if (act[kb] && !bm.empty) {
          const int s = kb * G::NW + w;
          // register r holds key c_row(r, g): its gate term is read for every entry, masked or
          // not (a read under the mask would turn each entry into a branch of its own)
          float e[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = st2[cs][r] * sc;
            if constexpr (has_gate) x += gl[s * kBwdKeyBlock + c_row(r, g)];
            e[r] = fast_exp2(x - l2) * dp2[cs][r];
          }
          if (bm.full) {
#pragma unroll
            for (int r = 0; r < 16; ++r) part += e[r];
          } else {
            // this lane's row sees keys [klo, khi] (sequence positions)
            int klo = kofs, khi = row < L ? kofs + n - 1 : kofs - 1;
            if (wl >= 0) klo = max(klo, row - wl);
            if (wr >= 0) khi = min(khi, row + wr);
            const LaneRange m = lane_range(kofs + kf, klo, khi);
#pragma unroll
            for (int r = 0; r < 16; ++r) part += lane_ok(m, r, g) ? e[r] : 0.0f;
          }
        }
        if (kb == KACT - 1) {
          part = half32_sum(part);
          if (g == 0) dpart[w * G::QT + qs * 32 + lc] = part;
          part = 0.0f;
          if (qs == 0) l2 = lse2[32 + lc];
        }
      }
      __syncthreads();
      if constexpr (CHUNK == 2) {
        // this chunk's share of D_i into the workspace row (the first chunk a row sees writes it)
        const int row = r0 + (int)threadIdx.x;
        if (threadIdx.x < G::QT && row < L) {
          int cf, cl;
          row_chunks(row, it.ntot, wl, wr, G::CAP, cf, cl);
          const int c = kofs / G::CAP;
          if (c >= cf && c <= cl) {
            float v = dpart[threadIdx.x];
#pragma unroll
            for (int ww = 1; ww < G::NW; ++ww) v += dpart[ww * G::QT + threadIdx.x];
            float* dst = it.dsumseq + (size_t)row * H;
            *dst = c == cf ? v : *dst + v;
          }
        }
      } else {
        // D_i of each tile row, once: NW consecutive lanes take a row's NW wave partials and add
        // them in a fixed tree order; the sum replaces the first wave's partial
        constexpr int RPW = kWave / G::NW;  // rows per wave (G::QT = NW * RPW)
        static_assert(G::QT == G::NW * RPW, "one row per group of NW lanes");
        const int drw = w * RPW + lane / G::NW;
        float v = dpart[(lane % G::NW) * G::QT + drw];
        v = group_sum<G::NW>(v);
        if (lane % G::NW == 0) dpart[drw] = v;
        __syncthreads();
      }
    }

    // ---- 3. S, dP, P, dS; dV, dK; dS^T to LDS. Iteration it = (query half qs, owned block kb);
    // the S / dP products of iteration it+1 are issued before the element-wise work of it, so the
    // MFMA pipe runs while the VALU works.
    if constexpr (CHUNK != 2) {
      int series = 0;  // 2: within the shorter series' range, 1: within kSeriesBound, 0: exact
      if constexpr (kSeries) {
        const float* qnrm = reinterpret_cast<const float*>(lds + G::OFF_QNRM) + ((FQ && (j & 1)) ? 4 * NW : 0);
        float qn2 = 0.0f, kn2 = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4 * NW; ++ww) qn2 = fmaxf(qn2, qnrm[ww]);
#pragma unroll
        for (int kb = 0; kb < KACT; ++kb) kn2 = fmaxf(kn2, act[kb] ? st.kn2[kb] : 0.0f);
        series = seq_series_within(gd.scale, qn2, kn2, series_short_bound_bwd<ACT>()) ? 2
                 : seq_series_ok(gd.scale, qn2, kn2)                              ? 1
                                                                                  : 0;
      }
      // the main pass of the tile, instantiated for the two series and the exact activation
      auto main_pass = [&](auto series_tag) {
        constexpr int SER = decltype(series_tag)::value;
        constexpr int NIT = 2 * KACT;
        const int sx_cur = (FQ && (j & 1)) ? G::OFF_SXL : G::OFF_SX;  // this tile's dS^T area
        const int q_cur = (FQ && (j & 1)) ? G::OFF_QN1 : G::OFF_QN;    // this tile's Q / dO buffer
        const int do_cur = (FQ && (j & 1)) ? G::OFF_DON1 : G::OFF_DON;
        f32x16 sacc[2], dpacc[2];
        bf16x8 qa[G::KK], da[G::KK];
        bf16x8 dota[G::DT][2], qta[G::DT][2];
        float lrow[16], drow[16];
        auto load_a = [&](int qs) {
  #pragma unroll
          for (int kk = 0; kk < G::KK; ++kk) {
            qa[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(lds + q_cur + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
            da[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(lds + do_cur + (qs * 32 + lc) * G::NROW + g * D + kk * 16));
          }
        };
        auto issue_sdp = [&](int kb, int slot) {
          sacc[slot] = f32x16{};
          dpacc[slot] = f32x16{};
  #pragma unroll
          for (int kk = 0; kk < G::KK; ++kk) {
            sacc[slot] = mfma32(qa[kk], st.kreg[kb][kk], sacc[slot]);
            dpacc[slot] = mfma32(da[kk], st.vreg[kb][kk], dpacc[slot]);
          }
        };
        // the products of iteration it+1 are issued before the element-wise work of it (the dO^T / Q^T
        // operands of dV / dK are read only after it, which keeps their registers free meanwhile).
        // Key-chunk passes, whose fp32 dQ rows already hold registers, run without it (measured
        // faster there: shared seed queries 540 -> 523 us), and so does the softmax form with 8
        // waves (no registers to spare).
        // (ungated element-wise forms: only the series tiles keep it; the exact tiles of such items
      // would otherwise need more registers than the wave has)
      constexpr bool PIPE = CHUNK == 0 && !(split && NW == 8) && (!kSeries || SER != 0);
        if constexpr (PIPE) {
          load_a(0);
          issue_sdp(0, 0);
        }
  #pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int qs = it / KACT, kb = it % KACT, cs = PIPE ? (it & 1) : 0;
          if constexpr (PIPE) {
            if (it + 1 < NIT) {
              if ((it + 1) / KACT != qs) load_a((it + 1) / KACT);
              issue_sdp((it + 1) % KACT, cs ^ 1);
            }
          } else {
            if (kb == 0) load_a(qs);
            issue_sdp(kb, 0);
          }
          const int rf = r0 + qs * 32;
          if (kb == 0) {
            if constexpr (softmax) {
  #pragma unroll
              for (int a = 0; a < 4; ++a) {
                const int rr = qs * 32 + a * 8 + g * 4;
                const f32x4 lv = *reinterpret_cast<const f32x4*>(lse2 + rr);
                const f32x4 dsum = *reinterpret_cast<const f32x4*>(dpart + rr);  // D_i of the rows
  #pragma unroll
                for (int e = 0; e < 4; ++e) {
                  lrow[4 * a + e] = lv[e];
                  drow[4 * a + e] = dsum[e];
                }
              }
            }
          }
          const int s = kb * G::NW + w;
          const int kf = kofs + blk[kb] * kBwdKeyBlock;  // sequence position of the block
          const int key = kf + lc;                       // this lane's key (sequence position)
          const int spos = (s * kBwdKeyBlock + lc) * G::SXROW;
          // P and dS as bf16 B operands (k-tile t = registers 8t..8t+7); zero for a block outside
          // the tile. The softmax form (and a few-term element-wise item) also carries the rounding
          // remainder as a second bf16 term (x ~ hi + lo): its products mix a few large terms, whose
          // bf16 rounding alone would exceed the tolerance.
          u32x4 pu[2], du[2], plu[2], dlu[2];
          auto elementwise = [&]() {
            // register r is query row rf + c_row(r, g), key `key`
            float p[16], ds[16];
            if constexpr (kSeries && SER == 2) {
  #pragma unroll
              for (int r = 0; r < 16; ++r) {
                float dphi;
                SeriesAct<ACT>::value_grad_short(sacc[cs][r], a1, d1, p[r], dphi);
                ds[r] = dpacc[cs][r] * dphi;
              }
            } else if constexpr (kSeries && SER == 1) {
  #pragma unroll
              for (int r = 0; r < 16; ++r) {
                float dphi;
                SeriesAct<ACT>::value_grad(sacc[cs][r], a1, a3, d1, d3, p[r], dphi);
                ds[r] = dpacc[cs][r] * dphi;
              }
            } else {
  #pragma unroll
              for (int r = 0; r < 16; ++r) {
                if constexpr (softmax) {
                  float x;
                  if constexpr (has_gate) x = __builtin_fmaf(sacc[cs][r], sc, st.gate[kb]);
                  else x = sacc[cs][r] * sc;
                  p[r] = fast_exp2(x - lrow[r]);
                  ds[r] = p[r] * (dpacc[cs][r] - drow[r]);
                } else {
                  float dphi;
                  if constexpr (has_gate) {
                    PointAct<ACT>::value_grad(__builtin_fmaf(sacc[cs][r], sc, st.gate[kb]), 1.0f, c1, c3, p[r], dphi);
                  } else {
                    PointAct<ACT>::value_grad(sacc[cs][r], sc, c1, c3, p[r], dphi);
                  }
                  ds[r] = dpacc[cs][r] * dphi;
                }
              }
            }
            if constexpr (MASKED) {
              if (!block_mask(kf, rf, kofs + n, L, wl, wr).full) {
                // this lane's key is seen by rows [rlo, rhi]
                int rlo = 0, rhi = key < kofs + n ? L - 1 : -1;
                if (wr >= 0) rlo = max(rlo, key - wr);
                if (wl >= 0) rhi = min(rhi, key + wl);
                const LaneRange m = lane_range(rf, rlo, rhi);
  #pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const bool ok = lane_ok(m, r, g);
                  p[r] = ok ? p[r] : 0.0f;
                  ds[r] = ok ? ds[r] : 0.0f;
                }
              }
            }
            if constexpr (GATED) if (want_dg) {
              float dsum = 0.0f;
  #pragma unroll
              for (int r = 0; r < 16; ++r) dsum += ds[r];
              st.dgs[kb] += dsum;
            }
  #pragma unroll
            for (int t = 0; t < 2; ++t)
  #pragma unroll
              for (int e = 0; e < 4; ++e) {
                pu[t][e] = pack_bf16x2(p[8 * t + 2 * e], p[8 * t + 2 * e + 1]);
                du[t][e] = pack_bf16x2(ds[8 * t + 2 * e], ds[8 * t + 2 * e + 1]);
                if (split || chunk_rows_split) {
                  plu[t][e] = pack_bf16x2(p[8 * t + 2 * e] - bf16_lo(pu[t][e]), p[8 * t + 2 * e + 1] - bf16_hi(pu[t][e]));
                  dlu[t][e] = pack_bf16x2(ds[8 * t + 2 * e] - bf16_lo(du[t][e]), ds[8 * t + 2 * e + 1] - bf16_hi(du[t][e]));
                }
              }
          };
          if constexpr (MASKED) {
  #pragma unroll
            for (int t = 0; t < 2; ++t) pu[t] = du[t] = plu[t] = dlu[t] = u32x4{0u, 0u, 0u, 0u};
            if (act[kb] && !block_mask(kf, rf, kofs + n, L, wl, wr).empty) elementwise();
          } else {
            // no mask: keys and rows past the ends meet zero operands, and phi(0) = 0
            elementwise();
          }
          // dS^T to the exchange tile: registers 4a..4a+3 are 4 consecutive query rows
  #pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int qo = (qs * 32 + a * 8 + g * 4) * 2;
            const int t = a >> 1, hlf = (a & 1) * 2;
            *reinterpret_cast<u32x2*>(lds + sx_cur + spos + qo) = u32x2{du[t][hlf], du[t][hlf + 1]};
            if constexpr (split_dq)
              *reinterpret_cast<u32x2*>(lds + G::OFF_SXL + spos + qo) = u32x2{dlu[t][hlf], dlu[t][hlf + 1]};
          }
          if (kb == 0) {
  #pragma unroll
            for (int dt = 0; dt < G::DT; ++dt)
  #pragma unroll
              for (int t = 0; t < 2; ++t) {
                dota[dt][t] = tr_operand<G::NROW>(lds, do_cur, qs, t, dt);
                qta[dt][t] = tr_operand<G::NROW>(lds, q_cur, qs, t, dt);
              }
          }
  #pragma unroll
          for (int dt = 0; dt < G::DT; ++dt)
  #pragma unroll
            for (int t = 0; t < 2; ++t) {
              st.dv[kb][dt] = mfma32(dota[dt][t], as_bf16x8(pu[t]), st.dv[kb][dt]);
              st.dk[kb][dt] = mfma32(qta[dt][t], as_bf16x8(du[t]), st.dk[kb][dt]);
              if (split || chunk_rows_split) {
                st.dv[kb][dt] = mfma32(dota[dt][t], as_bf16x8(plu[t]), st.dv[kb][dt]);
                st.dk[kb][dt] = mfma32(qta[dt][t], as_bf16x8(dlu[t]), st.dk[kb][dt]);
              }
            }
        }
      };
      if constexpr (kSeries) {
        if (series == 2) main_pass(std::integral_constant<int, 2>{});
        else if (series == 1) main_pass(std::integral_constant<int, 1>{});
        else main_pass(std::integral_constant<int, 0>{});
      } else {
        main_pass(std::integral_constant<int, 0>{});
      }
    }
    if constexpr (FQ) {
      // one barrier per tile: the next tile goes into the other Q / dO buffer (last read by the
      // previous tile's main pass) before the barrier, then the previous tile's dQ
      if (j + 1 < t1) {
        store_qtile<D, NW, softmax, DSUM, kSeries>(lds, pf, (j + 1) & 1);
        if (j + 2 < t1)
          prefetch_qtile<D, NW, softmax, DSUM>(pf, it.qseq, it.doseq, it.lseseq, rs, H, r0 + 2 * G::QT, L, it.dsumseq);
      }
      if (j > t0 && dq_role) fq = dq_tile((j & 1) ? G::OFF_SX : G::OFF_SXL);  // previous tile's area
      __syncthreads();  // this tile's dS^T and the next tile's Q / dO complete
      if (j > t0 && dq_role) dq_store(fq, r0 - G::QT);
      continue;
    }
    __syncthreads();  // dS^T tile complete; this tile's Q / dO / lse no longer read
    if (j + 1 < t1) {
      // next tile into LDS (while dQ runs), then the loads of the one after it: issued before this
      // tile's dQ stores, so waiting for them never waits for those stores
      store_qtile<D, NW, softmax, DSUM, kSeries>(lds, pf);
      if (j + 2 < t1)
        prefetch_qtile<D, NW, softmax, DSUM>(pf, it.qseq, it.doseq, it.lseseq, rs, H, r0 + 2 * G::QT, L, it.dsumseq);
      if constexpr (WINDOWED) {
        // blocks entering at the next tile: their rows into the slot registers (the leaving
        // block's K and V are no longer read), then the leaving blocks' dK, dV, dG go out
        int bn[KACT];
        bool an[KACT];
        tile_blocks(j + 1, bn, an);
#pragma unroll
        for (int kb = 0; kb < KACT; ++kb)
          if (an[kb] && bn[kb] != st.cur[kb]) {
            take_load_regs<D, NW>(st, kb, gnext[kb], gd, it.kseq, it.vseq, it.gseq, bn[kb], n);
            pend[kb] = bn[kb];
          }
#pragma unroll
        for (int kb = 0; kb < KACT; ++kb)
          if (pend[kb] >= 0 && st.cur[kb] >= 0) {
            flush_block<D, NW>(st, kb, gd, it.dkseq, it.dvseq, it.dgseq, n, dv_scale);
            st.cur[kb] = -1;
          }
      }
    }

    // ---- 4. dQ^T = K^T dS^T over the ring slots (a slot outside the tile holds zero dS);
    // register r of lane (query, g) is d = dtile*32 + g*16 + r (out_perm order of the K^T rows)
    if (CHUNK != 2 && !FQ && dq_role) {
#pragma unroll
      for (int qi = 0; qi < G::QH; ++qi) {
        const int qh = qh_first + qi;
        f32x16 acc2[2] = {f32x16{}, f32x16{}};
        if constexpr (WINDOWED) {
          // 16-key steps over every ring slot (a slot outside the tile holds zero dS); the operands
          // of step k+1 are read while step k multiplies, and two accumulators keep consecutive
          // MFMAs independent
          bf16x8 ka[2], sb[2], sl[2];
          auto load_step = [&](int k, int buf) {
            const int kbase = k * 16;
            ka[buf] = as_bf16x8(*reinterpret_cast<const u32x4*>(lds + G::OFF_KT + drow * G::KTROW + (kbase + g * 8) * 2));
            sb[buf] = sx_operand<G::SXROW>(lds, G::OFF_SX, kbase, qh);
            if constexpr (split_dq) sl[buf] = sx_operand<G::SXROW>(lds, G::OFF_SXL, kbase, qh);
          };
          load_step(0, 0);
#pragma unroll
          for (int k = 0; k < NK; ++k) {
            if (k + 1 < NK) load_step(k + 1, (k + 1) & 1);
            acc2[k & 1] = mfma32(ka[k & 1], sb[k & 1], acc2[k & 1]);
            if constexpr (split_dq) acc2[k & 1] = mfma32(ka[k & 1], sl[k & 1], acc2[k & 1]);
          }
        } else {
          // only the slots of the item's (or chunk's) nkb blocks: a ragged last chunk leaves the
          // others empty. Two 16-key steps per slot, one accumulator each.
          const int n_act = nkb < NS ? nkb : NS;
          for (int a = 0; a < n_act; ++a) {
#pragma unroll
            for (int hk = 0; hk < 2; ++hk) {
              const int kbase = a * kBwdKeyBlock + hk * 16;
              const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(lds + G::OFF_KT + drow * G::KTROW + (kbase + g * 8) * 2));
              acc2[hk] = mfma32(ka, sx_operand<G::SXROW>(lds, G::OFF_SX, kbase, qh), acc2[hk]);
              if constexpr (split_dq) acc2[hk] = mfma32(ka, sx_operand<G::SXROW>(lds, G::OFF_SXL, kbase, qh), acc2[hk]);
            }
          }
        }
        const f32x16 acc = acc2[0] + acc2[1];
        const int row = r0 + qh * 32 + lc;
        if constexpr (CHUNK == 1) {
          // this chunk's share of the row's dQ: the first chunk the row sees writes the fp32 row,
          // later ones add to it, the last converts it (a shared query matrix keeps fp32 partials)
          int cf = 0, cl = -1;
          if (row < L) row_chunks(row, it.ntot, wl, wr, G::CAP, cf, cl);
          const int c = kofs / G::CAP;
          if (c >= cf && c <= cl) {
            float* p32 = it.dq32seq + row * rs + dtile * 32 + g * 16;
            f32x4 v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] = f32x4{acc[4 * e], acc[4 * e + 1], acc[4 * e + 2], acc[4 * e + 3]};
              if (c != cf) v[e] += *reinterpret_cast<const f32x4*>(p32 + 4 * e);
            }
            if (c == cl && !it.shared_q) {
              const OutPtr dst = it.dqseq + (row * rs + dtile * 32 + g * 16);
              out_store8(dst, v[0] * gd.scale, v[1] * gd.scale);
              out_store8(dst + 8, v[2] * gd.scale, v[3] * gd.scale);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) *reinterpret_cast<f32x4*>(p32 + 4 * e) = v[e];
            }
          }
        } else if (row < L) {
          out_store16(it.dqseq + (row * rs + dtile * 32 + g * 16), acc, gd.scale);
        }
      }
    }
    if (j + 1 < t1) __syncthreads();  // next tile staged; dS^T and K^T staging free
  }
  if constexpr (FQ) {
    // the last tile's dQ (its dS^T is complete since the barrier after its main pass)
    if (t1 > t0 && dq_role) dq_store(dq_tile(((t1 - 1) & 1) ? G::OFF_SXL : G::OFF_SX), (t1 - 1) * G::QT);
  }
  if constexpr (CHUNK != 2)
#pragma unroll
    for (int kb = 0; kb < KACT; ++kb)
      if (st.cur[kb] >= 0) flush_block<D, NW>(st, kb, gd, it.dkseq, it.dvseq, it.dgseq, n, dv_scale);
}

// Sweeps a backward kernel holds (its launch guarantees its items need no other).
enum BwdPaths { kPathsAll = 0, kPathsNoWindow = 1, kPathsRing = 2 };

template <int D, int NW, int ACT, bool GATED, int PATHS = kPathsAll>
__device__ __forceinline__ void bwd_item(char* lds, const GroupDesc& gd, int b, int h) {
  using G = BwdGeo<D, NW>;
  BwdItem it;
  const int q0 = gd.q_off[b], k0 = gd.kv_off[b];
  it.L = gd.q_off[b + 1] - q0;
  it.n = gd.kv_off[b + 1] - k0;
  it.H = gd.num_heads;
  it.rs = (size_t)it.H * D;
  it.wl = gd.wl;
  it.wr = gd.wr;
  const int H = it.H;
  it.shared_q = gd.shared_q > 0;
  // a shared query matrix: every sequence reads its rows from row 0; its dQ rows are fp32
  // partials of sequence b at rows [b * shared_q, ...) of the workspace
  const size_t qrow = it.shared_q ? 0 : (size_t)q0;
  const size_t dqrow = it.shared_q ? (size_t)b * gd.shared_q : (size_t)q0;
  it.qseq = reinterpret_cast<const bf16*>(gd.q) + (qrow * H + h) * D;
  it.doseq = reinterpret_cast<const bf16*>(gd.dout) + ((size_t)q0 * H + h) * D;
  it.lseseq = gd.lse ? gd.lse + (size_t)q0 * H + h : nullptr;
  it.dqseq = out_ptr(gd.dq, gd.out_f32, ((size_t)q0 * H + h) * D);
  it.dq32seq = gd.dq32 ? gd.dq32 + (dqrow * H + h) * D : nullptr;
  it.dsumseq = gd.delta ? gd.delta + (size_t)q0 * H + h : nullptr;
  it.kseq = reinterpret_cast<const bf16*>(gd.k) + ((size_t)k0 * H + h) * D;
  it.vseq = reinterpret_cast<const bf16*>(gd.v) + ((size_t)k0 * H + h) * D;
  it.gseq = gd.g ? gd.g + (size_t)k0 * H + h : nullptr;
  it.dkseq = out_ptr(gd.dk, gd.out_f32, ((size_t)k0 * H + h) * D);
  it.dvseq = out_ptr(gd.dv, gd.out_f32, ((size_t)k0 * H + h) * D);
  it.dgseq = gd.dg ? gd.dg + (size_t)k0 * H + h : nullptr;
  it.kofs = 0;
  it.ntot = it.n;
  it.t0 = 0;
  it.t1 = (it.L + G::QT - 1) / G::QT;
  const int L = it.L, n = it.n;
  const size_t rs = it.rs;

  if (n <= 0) {  // no keys: dQ = 0 (a shared query matrix: zero partial rows)
    if (it.shared_q) {
      for (int idx = threadIdx.x; idx < L * (D / 4); idx += G::THREADS) {
        const int r = idx / (D / 4), c = idx % (D / 4);
        *reinterpret_cast<f32x4*>(it.dq32seq + r * rs + c * 4) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    } else {
      for (int idx = threadIdx.x; idx < L * G::CPR; idx += G::THREADS) {
        const int r = idx / G::CPR, c = idx % G::CPR;
        out_zero8(it.dqseq + (r * rs + c * 8));
      }
    }
    return;
  }
  if (L <= 0) {  // no queries: dK = dV = dG = 0
    for (int idx = threadIdx.x; idx < n * G::CPR; idx += G::THREADS) {
      const int r = idx / G::CPR, c = idx % G::CPR;
      out_zero8(it.dkseq + (r * rs + c * 8));
      out_zero8(it.dvseq + (r * rs + c * 8));
    }
    if (it.dgseq)
      for (int r = threadIdx.x; r < n; r += G::THREADS) it.dgseq[(size_t)r * H] = 0.0f;
    return;
  }
  const bool windowed = it.wl >= 0 || it.wr >= 0;
  const bool split_all = ACT != GDPA_ACT_SOFTMAX && gd.split_all;
  if constexpr (PATHS == kPathsRing) {
    // every item's window streams its keys through the ring (no key chunks, no shared queries)
    bwd_sweep<D, NW, ACT, GATED, G::KB, true>(lds, gd, it);
    return;
  }
  if (it.shared_q || bwd_needs_chunks(D, it.wl, it.wr, n, split_all)) {
    // key chunks of CAP keys, one after the other; each sweeps the query tiles whose rows see it.
    // Softmax first accumulates D_i over every chunk (a pass of its own), then the main passes.
    const int nch = (n + G::CAP - 1) / G::CAP;
    auto chunk_item = [&](int c) {
      BwdItem ci = it;
      ci.kofs = c * G::CAP;
      ci.n = n - ci.kofs < G::CAP ? n - ci.kofs : G::CAP;
      ci.kseq = it.kseq + (size_t)ci.kofs * rs;
      ci.vseq = it.vseq + (size_t)ci.kofs * rs;
      ci.gseq = it.gseq ? it.gseq + (size_t)ci.kofs * H : nullptr;
      ci.dkseq = it.dkseq + (size_t)ci.kofs * rs;
      ci.dvseq = it.dvseq + (size_t)ci.kofs * rs;
      ci.dgseq = it.dgseq ? it.dgseq + (size_t)ci.kofs * H : nullptr;
      // rows whose window reaches the chunk's keys [kofs, kofs + n)
      int rlo = 0, rhi = L - 1;
      if (it.wr >= 0 && ci.kofs - it.wr > 0) rlo = ci.kofs - it.wr;
      if (it.wl >= 0 && ci.kofs + ci.n - 1 + it.wl < L - 1) rhi = ci.kofs + ci.n - 1 + it.wl;
      ci.t0 = rlo / G::QT;
      ci.t1 = rhi >= rlo ? rhi / G::QT + 1 : ci.t0;
      return ci;
    };
    if constexpr (ACT == GDPA_ACT_SOFTMAX) {
      for (int c = 0; c < nch; ++c) {
        const BwdItem ci = chunk_item(c);
        __syncthreads();  // previous pass done with LDS
        bwd_sweep<D, NW, ACT, GATED, G::KB, false, 2>(lds, gd, ci);
      }
    }
    for (int c = 0; c < nch; ++c) {
      const BwdItem ci = chunk_item(c);
      __syncthreads();
      bwd_sweep<D, NW, ACT, GATED, G::KB, false, 1>(lds, gd, ci);
    }
    return;
  }
  if constexpr (ACT != GDPA_ACT_SOFTMAX) {
    // few rows or few keys (or split operands asked for): the hi + lo operand form, every key
    // resident (longer ones took the chunk path above)
    if (L <= kSplitTerms || n <= kSplitTerms || split_all) {
      bwd_sweep<D, NW, ACT, GATED, G::KB, false, 0, true>(lds, gd, it);
      return;
    }
  }
  // One owned block per wave suffices when all keys fit in NW blocks. Zero padding makes the
  // entries past the ends vanish for the element-wise forms (phi(0) = 0; dO and V rows past the
  // ends are zero), so only the softmax form and windows need explicit masks.
  const bool few_keys = (n + kBwdKeyBlock - 1) / kBwdKeyBlock <= G::NW;
  if (PATHS == kPathsAll && windowed) {
    if (G::KB > 1 && few_keys) bwd_sweep<D, NW, ACT, GATED, 1, true>(lds, gd, it);
    else bwd_sweep<D, NW, ACT, GATED, G::KB, true>(lds, gd, it);
  } else {
    if (G::KB > 1 && few_keys) bwd_sweep<D, NW, ACT, GATED, 1, false>(lds, gd, it);
    else bwd_sweep<D, NW, ACT, GATED, G::KB, false>(lds, gd, it);
  }
}

template <int D, int NW, int ACT, int PATHS>
__device__ __forceinline__ void bwd_dispatch_gate(char* lds, const GroupDesc& gd, int b, int h) {
  if (gd.g != nullptr) bwd_item<D, NW, ACT, true, PATHS>(lds, gd, b, h);
  else bwd_item<D, NW, ACT, false, PATHS>(lds, gd, b, h);
}

template <int D, int NW, int ASET>
__device__ __forceinline__ void bwd_dispatch_act(char* lds, const GroupDesc& gd, int b, int h) {
  constexpr int P = (ASET & kBwdWideSoftmax) ? kPathsNoWindow : (ASET & kBwdRingSoftmax) ? kPathsRing : kPathsAll;
  if constexpr ((ASET & (1 << GDPA_ACT_GELU)) != 0)
    if (gd.act == GDPA_ACT_GELU) { bwd_dispatch_gate<D, NW, GDPA_ACT_GELU, P>(lds, gd, b, h); return; }
  if constexpr ((ASET & (1 << GDPA_ACT_SILU)) != 0)
    if (gd.act == GDPA_ACT_SILU) { bwd_dispatch_gate<D, NW, GDPA_ACT_SILU, P>(lds, gd, b, h); return; }
  if constexpr ((ASET & (1 << GDPA_ACT_SOFTMAX)) != 0)
    if (gd.act == GDPA_ACT_SOFTMAX) bwd_dispatch_gate<D, NW, GDPA_ACT_SOFTMAX, P>(lds, gd, b, h);
}

template <int DSET, int ASET>
__global__ void __launch_bounds__((bwd_waves<DSET, ASET>() * kWave), 1) bwd_bf16_kernel(LaunchDesc d) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  if ((int)blockIdx.x >= d.n_items || launch_refused(d)) return;
  int g, h, b;
  unpack_item(d.items[xcd_item((int)blockIdx.x, d.n_items)], g, h, b);
  if (g >= d.n_groups) return;
  GroupDesc gd = select_group(d, g);
  if (b >= gd.num_seqs || h >= gd.num_heads) return;  // list built for another shape
  if (gd.head_acts != nullptr) gd.act = gd.head_acts[h];  // activation of this item's head
  {
    const int q0 = gd.q_off[b], q1 = gd.q_off[b + 1], k0 = gd.kv_off[b], k1 = gd.kv_off[b + 1];
    int32_t e = item_error(gd, q0, q1, k0, k1, -1);
    // key chunks (or a shared query matrix) accumulate in workspace rows the host reserves only
    // when the max_seqlen_kv hint (or the flag) asks for them
    const bool chunked = gd.shared_q || bwd_needs_chunks(gd.head_dim, gd.wl, gd.wr, k1 - k0,
                                                         gd.split_all && gd.act != GDPA_ACT_SOFTMAX);
    if (e == 0 && chunked && (gd.dq32 == nullptr || (gd.act == GDPA_ACT_SOFTMAX && gd.delta == nullptr)))
      e = GDPA_DEVICE_ERR_LENGTH;
    if (e != 0) {
      if (threadIdx.x == 0) report_error(d, e);
      return;
    }
  }
  constexpr int NW = bwd_waves<DSET, ASET>();
  if constexpr ((DSET & kDim32) != 0)
    if (gd.head_dim == 32) { bwd_dispatch_act<32, NW, ASET>(lds, gd, b, h); return; }
  if constexpr ((DSET & kDim64) != 0)
    if (gd.head_dim == 64) { bwd_dispatch_act<64, NW, ASET>(lds, gd, b, h); return; }
  if constexpr ((DSET & kDim128) != 0)
    if (gd.head_dim == 128) { bwd_dispatch_act<128, NW, ASET>(lds, gd, b, h); return; }
}

// ---- Short key blocks: one wave per (sequence, head) item -------------------------------------
//
// When every sequence has at most 32 keys (element-wise forms, no window), a whole item fits one
// wave: the wave keeps the block's K and V rows and its dK^T, dV^T accumulators in registers and
// sweeps the item's query rows 32 at a time, with Q and dO rows staged in a private LDS area for
// the transposing reads and dS^T in a private exchange tile for dQ. The four waves of a workgroup
// work on four items with no barrier between them (a workgroup-wide sweep would leave three of
// its four waves without keys).
template <int D>
struct SmallGeo {
  static constexpr int KK = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int NROW = D * 2 + 16;          // row-major Q / dO tile row (bytes)
  static constexpr int KTROW = 32 * 2 + 16;        // K^T row: 32 keys
  static constexpr int SXROW = 32 * 2 + 16;        // dS^T row (one key): 32 queries
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = OFF_Q + 32 * NROW;
  static constexpr int OFF_KT = OFF_DO + 32 * NROW;
  static constexpr int OFF_SX = OFF_KT + D * KTROW;
  static constexpr int OFF_SXL = OFF_SX + 32 * SXROW;  // rounding remainder of dS^T (few keys)
  static constexpr int BYTES = OFF_SXL + 32 * SXROW;   // per wave
  static_assert(4 * BYTES <= 160 * 1024, "LDS budget");
};

template <int DSET>
constexpr int bwd_small_lds_bytes() {
  return 4 * max3((DSET & kDim32) ? SmallGeo<32>::BYTES : 0, (DSET & kDim64) ? SmallGeo<64>::BYTES : 0,
                  (DSET & kDim128) ? SmallGeo<128>::BYTES : 0);
}

// The wave's LDS stores are complete and visible to all its lanes before its later LDS reads (and
// the compiler keeps them in that order).
__device__ inline void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int ACT, bool GATED>
__device__ __forceinline__ void bwd_small_item(char* wl, const GroupDesc& gd, int b, int h) {
  using G = SmallGeo<D>;
  const int lane = lane_id(), lc = lane & 31, g = lane >> 5;
  const int q0 = gd.q_off[b], k0 = gd.kv_off[b];
  const int L = gd.q_off[b + 1] - q0, n = gd.kv_off[b + 1] - k0;
  const int H = gd.num_heads;
  const size_t rs = (size_t)H * D;
  const bf16* qseq = reinterpret_cast<const bf16*>(gd.q) + ((size_t)q0 * H + h) * D;
  const bf16* doseq = reinterpret_cast<const bf16*>(gd.dout) + ((size_t)q0 * H + h) * D;
  const OutPtr dqseq = out_ptr(gd.dq, gd.out_f32, ((size_t)q0 * H + h) * D);
  const bf16* kseq = reinterpret_cast<const bf16*>(gd.k) + ((size_t)k0 * H + h) * D;
  const bf16* vseq = reinterpret_cast<const bf16*>(gd.v) + ((size_t)k0 * H + h) * D;
  const float* gseq = gd.g ? gd.g + (size_t)k0 * H + h : nullptr;
  const OutPtr dkseq = out_ptr(gd.dk, gd.out_f32, ((size_t)k0 * H + h) * D);
  const OutPtr dvseq = out_ptr(gd.dv, gd.out_f32, ((size_t)k0 * H + h) * D);
  float* dgseq = gd.dg ? gd.dg + (size_t)k0 * H + h : nullptr;
  constexpr int CPR = D / 8;
  if (n <= 0) {  // no keys: dQ = 0
    for (int idx = lane; idx < L * CPR; idx += kWave)
      out_zero8(dqseq + ((idx / CPR) * rs + (idx % CPR) * 8));
    return;
  }
  if (L <= 0) {  // no queries: dK = dV = dG = 0
    for (int idx = lane; idx < n * CPR; idx += kWave) {
      out_zero8(dkseq + ((idx / CPR) * rs + (idx % CPR) * 8));
      out_zero8(dvseq + ((idx / CPR) * rs + (idx % CPR) * 8));
    }
    if (dgseq)
      for (int r = lane; r < n; r += kWave) dgseq[(size_t)r * H] = 0.0f;
    return;
  }

  // the block: this lane's key lc (rows past n are zero), K^T into the private staging tile
  const bool kok = lc < n;
  bf16x8 kreg[G::KK], vreg[G::KK];
#pragma unroll
  for (int kk = 0; kk < G::KK; ++kk) {
    u32x4 ku = {0u, 0u, 0u, 0u}, vu = {0u, 0u, 0u, 0u};
    if (kok) {
      ku = *reinterpret_cast<const u32x4*>(kseq + lc * rs + g * (D / 2) + kk * 8);
      vu = *reinterpret_cast<const u32x4*>(vseq + lc * rs + g * (D / 2) + kk * 8);
    }
    kreg[kk] = as_bf16x8(ku);
    vreg[kk] = as_bf16x8(vu);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d0 = g * (D / 2) + kk * 8 + 2 * e;
      *reinterpret_cast<uint16_t*>(wl + G::OFF_KT + d0 * G::KTROW + lc * 2) = (uint16_t)(ku[e] & 0xFFFF);
      *reinterpret_cast<uint16_t*>(wl + G::OFF_KT + (d0 + 1) * G::KTROW + lc * 2) = (uint16_t)(ku[e] >> 16);
    }
  }
  float gate = 0.0f, graw = 0.0f;
  if (GATED && kok) {
    graw = gseq[(size_t)lc * H];
    gate = log_sigmoid_f(graw);
  }
  // ungated: the keys' largest ||k||^2, for the series bound of each 32-row step
  float kn2 = 0.0f;
  if constexpr (!GATED) {
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) kn2 += sumsq_bf16x8(__builtin_bit_cast(u32x4, kreg[kk]));
    kn2 = wave_max(kn2 + __shfl_xor(kn2, 32, 64));
  }
  f32x16 dk[G::DT], dv[G::DT];
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) dk[dt] = dv[dt] = f32x16{};
  float dgs = 0.0f;
  const float sc = gd.scale;
  float c1 = 0.0f, c3 = 0.0f;
  PointAct<ACT>::coeffs(GATED ? 1.0f : gd.scale, c1, c3);
  const float dv_scale = GATED ? 1.0f : gd.scale;
  float a1 = 0.0f, a3 = 0.0f, d1 = 0.0f, d3 = 0.0f;
  if constexpr (!GATED) SeriesAct<ACT>::coeffs(gd.scale, a1, a3, d1, d3);
  // few rows: dK, dV sums of at most kSplitTerms products; few keys: dQ sums likewise. Their P / dS
  // operands then carry the rounding remainder as a second bf16 term (uniform per item).
  const bool split_rows = L <= kSplitTerms || gd.split_all, split_keys = n <= kSplitTerms || gd.split_all;

  // Q and dO rows of a 32-row step: lane (row lc, half g) loads the 16-byte pieces it needs as the
  // A operand of S = Q K^T and dP = dO V^T. The next step's rows are loaded during the current
  // step (registers; the wave runs alone on its SIMD, so its own loads must cover the latency).
  u32x4 qnext[G::KK], dnext[G::KK];
  auto load_rows = [&](int rr0) {
    const int row = rr0 + lc;
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) {
      qnext[kk] = u32x4{0u, 0u, 0u, 0u};
      dnext[kk] = u32x4{0u, 0u, 0u, 0u};
      if (row < L) {
        qnext[kk] = *reinterpret_cast<const u32x4*>(qseq + row * rs + g * (D / 2) + kk * 8);
        dnext[kk] = *reinterpret_cast<const u32x4*>(doseq + row * rs + g * (D / 2) + kk * 8);
      }
    }
  };
  load_rows(0);
  for (int r0 = 0; r0 < L; r0 += 32) {
    // this step's rows as A operands, and row-major in LDS for the transposing reads
    bf16x8 qa[G::KK], da[G::KK];
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) {
      qa[kk] = as_bf16x8(qnext[kk]);
      da[kk] = as_bf16x8(dnext[kk]);
      *reinterpret_cast<u32x4*>(wl + G::OFF_Q + lc * G::NROW + g * D + kk * 16) = qnext[kk];
      *reinterpret_cast<u32x4*>(wl + G::OFF_DO + lc * G::NROW + g * D + kk * 16) = dnext[kk];
    }
    if (r0 + 32 < L) load_rows(r0 + 32);
    const int row = r0 + lc;
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < G::KK; ++kk) {
      sacc = mfma32(qa[kk], kreg[kk], sacc);
      dpacc = mfma32(da[kk], vreg[kk], dpacc);
    }
    // register r of lane (key lc, g) is row r0 + c_row(r, g); keys and rows past the ends meet
    // zero operands (phi(0) = 0, and their dO / Q rows are zero), so no mask is needed
    float p[16], ds[16];
    int series = 0;  // 2: within the shorter series' range, 1: within kSeriesBound, 0: exact
    if constexpr (!GATED) {
      // the step's rows: this lane holds half of row lc, the other half sits 32 lanes away
      float qn2 = 0.0f;
#pragma unroll
      for (int kk = 0; kk < G::KK; ++kk) qn2 += sumsq_bf16x8(__builtin_bit_cast(u32x4, qa[kk]));
      qn2 = wave_max_lanes(half32_sum(qn2));
      series = seq_series_within(gd.scale, qn2, kn2, series_short_bound_bwd<ACT>()) ? 2
               : seq_series_ok(gd.scale, qn2, kn2)                              ? 1
                                                                                : 0;
    }
    if (!GATED && series == 2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float dphi;
        SeriesAct<ACT>::value_grad_short(sacc[r], a1, d1, p[r], dphi);
        ds[r] = dpacc[r] * dphi;
      }
    } else if (!GATED && series == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float dphi;
        SeriesAct<ACT>::value_grad(sacc[r], a1, a3, d1, d3, p[r], dphi);
        ds[r] = dpacc[r] * dphi;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float dphi;
        if constexpr (GATED) PointAct<ACT>::value_grad(__builtin_fmaf(sacc[r], sc, gate), 1.0f, c1, c3, p[r], dphi);
        else PointAct<ACT>::value_grad(sacc[r], sc, c1, c3, p[r], dphi);
        ds[r] = dpacc[r] * dphi;
      }
    }
    if constexpr (GATED) {
#pragma unroll
      for (int r = 0; r < 16; ++r) dgs += ds[r];
    }
    u32x4 pu[2], du[2], plu[2], dlu[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pu[t][e] = pack_bf16x2(p[8 * t + 2 * e], p[8 * t + 2 * e + 1]);
        du[t][e] = pack_bf16x2(ds[8 * t + 2 * e], ds[8 * t + 2 * e + 1]);
        plu[t][e] = pack_bf16x2(p[8 * t + 2 * e] - bf16_lo(pu[t][e]), p[8 * t + 2 * e + 1] - bf16_hi(pu[t][e]));
        dlu[t][e] = pack_bf16x2(ds[8 * t + 2 * e] - bf16_lo(du[t][e]), ds[8 * t + 2 * e + 1] - bf16_hi(du[t][e]));
      }
    // dS^T to the private exchange tile: registers 4a..4a+3 are 4 consecutive rows
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int t = a >> 1, hlf = (a & 1) * 2;
      *reinterpret_cast<u32x2*>(wl + G::OFF_SX + lc * G::SXROW + (a * 8 + g * 4) * 2) = u32x2{du[t][hlf], du[t][hlf + 1]};
      if (split_keys)
        *reinterpret_cast<u32x2*>(wl + G::OFF_SXL + lc * G::SXROW + (a * 8 + g * 4) * 2) = u32x2{dlu[t][hlf], dlu[t][hlf + 1]};
    }
    lds_wave_sync();  // the wave's Q / dO / dS^T stores are in LDS
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 dot = tr_operand<G::NROW>(wl, G::OFF_DO, 0, t, dt);
        const bf16x8 qt = tr_operand<G::NROW>(wl, G::OFF_Q, 0, t, dt);
        dv[dt] = mfma32(dot, as_bf16x8(pu[t]), dv[dt]);
        dk[dt] = mfma32(qt, as_bf16x8(du[t]), dk[dt]);
        if (split_rows) {
          dv[dt] = mfma32(dot, as_bf16x8(plu[t]), dv[dt]);
          dk[dt] = mfma32(qt, as_bf16x8(dlu[t]), dk[dt]);
        }
      }
    // dQ^T = K^T dS^T: register r of lane (row lc, g) is d = dt*32 + g*16 + r
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt) {
      const int drow = dt * 32 + out_perm(lc);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(wl + G::OFF_KT + drow * G::KTROW + (k * 16 + g * 8) * 2));
        acc = mfma32(ka, sx_operand<G::SXROW>(wl, G::OFF_SX, k * 16, 0), acc);
        if (split_keys) acc = mfma32(ka, sx_operand<G::SXROW>(wl, G::OFF_SXL, k * 16, 0), acc);
      }
      if (row < L) out_store16(dqseq + (row * rs + dt * 32 + g * 16), acc, gd.scale);
    }
    lds_wave_sync();  // every read of this tile's LDS areas is done before the next tile's stores
  }
  // dK, dV (and dG) of the block: register r of lane (key, g) in d-tile dt is d = dt*32 + c_row(r, g)
  const float dgsum = dgs + __shfl_xor(dgs, 32);
  if (kok) {
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const size_t e = lc * rs + dt * 32 + a * 8 + g * 4;
        out_store4(dkseq + e, f32x4{dk[dt][4 * a], dk[dt][4 * a + 1], dk[dt][4 * a + 2], dk[dt][4 * a + 3]} * gd.scale);
        out_store4(dvseq + e, f32x4{dv[dt][4 * a], dv[dt][4 * a + 1], dv[dt][4 * a + 2], dv[dt][4 * a + 3]} * dv_scale);
      }
    if (dgseq != nullptr && g == 0) dgseq[(size_t)lc * H] = (1.0f / (1.0f + __expf(graw))) * dgsum;
  }
}

template <int D, int ASET>
__device__ __forceinline__ void bwd_small_dispatch(char* wl, const GroupDesc& gd, int b, int h) {
  if constexpr ((ASET & (1 << GDPA_ACT_GELU)) != 0)
    if (gd.act == GDPA_ACT_GELU) {
      if (gd.g != nullptr) bwd_small_item<D, GDPA_ACT_GELU, true>(wl, gd, b, h);
      else bwd_small_item<D, GDPA_ACT_GELU, false>(wl, gd, b, h);
      return;
    }
  if constexpr ((ASET & (1 << GDPA_ACT_SILU)) != 0)
    if (gd.act == GDPA_ACT_SILU) {
      if (gd.g != nullptr) bwd_small_item<D, GDPA_ACT_SILU, true>(wl, gd, b, h);
      else bwd_small_item<D, GDPA_ACT_SILU, false>(wl, gd, b, h);
    }
}

// Workgroup x, wave w: work item 4x + w. The items are in longest-first order, so the four waves
// of a workgroup get items of similar length.
template <int DSET, int ASET>
__global__ void __launch_bounds__(4 * kWave, 1) bwd_small_kernel(LaunchDesc d) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int w = wave_id();
  const int item = (int)blockIdx.x * 4 + w;
  if (item >= d.n_items || launch_refused(d)) return;
  int g, h, b;
  unpack_item(d.items[item], g, h, b);
  if (g >= d.n_groups) return;
  GroupDesc gd = select_group(d, g);
  if (b >= gd.num_seqs || h >= gd.num_heads) return;
  {
    // one block of at most 32 keys per item
    const int32_t e = item_error(gd, gd.q_off[b], gd.q_off[b + 1], gd.kv_off[b], gd.kv_off[b + 1], kBwdKeyBlock);
    if (e != 0) {
      if (lane_id() == 0) report_error(d, e);
      return;
    }
  }
  constexpr int WB = bwd_small_lds_bytes<DSET>() / 4;
  char* wl = lds + w * WB;
  if constexpr ((DSET & kDim32) != 0)
    if (gd.head_dim == 32) { bwd_small_dispatch<32, ASET>(wl, gd, b, h); return; }
  if constexpr ((DSET & kDim64) != 0)
    if (gd.head_dim == 64) { bwd_small_dispatch<64, ASET>(wl, gd, b, h); return; }
  if constexpr ((DSET & kDim128) != 0)
    if (gd.head_dim == 128) { bwd_small_dispatch<128, ASET>(wl, gd, b, h); return; }
}

}  // namespace gdpa
