// GDPA forward for bf16 on gfx950: one workgroup (4 waves) per (sequence, head) work item.
//
//   S = scale Q K^T [+ log sigmoid G];  O = phi(S) V   (element-wise phi)  or
//   O = softmax(S) V with running row max / sum and lse = m + ln(l)           (softmax)
//
// (Kunlun review, section 2.3 and Figure 2: QK^T / tau, activation, times V, fused so that the
// T x n score matrix never reaches HBM; gate from the reproduction README's "Core equations";
// window from the review's section 2.5.)
//
// Data flow of one item:
//   * K rows and V^T (keys contiguous, in the MFMA slot order) of the item's key range are staged
//     into LDS once with coalesced 16-byte loads; the per-key gate term is staged beside them.
//   * Each wave owns 32 or 64 query rows and keeps their Q in registers (the B operand of
//     S^T = K Q^T: a lane holds 8..64 contiguous d of one row).
//   * Per block of 32 keys: S^T on MFMA (A = K rows from LDS), mask / phi / online softmax on the
//     fp32 accumulators, convert to bf16; the accumulator layout of S^T is directly the B operand
//     of O^T = V^T P^T (A = V^T rows from LDS), so P never leaves registers.
//   * Epilogue: each lane holds 16 consecutive d of one row of O: two 16-byte stores.
// Short key ranges (personalized-FFN form: n keys per sample) are staged once and the waves sweep
// all query tiles of the sequence. A bounded window over a longer sequence keeps a ring of key
// blocks in LDS: each group of 128 rows stages only the blocks entering its key range
// [r0 - left, r0 + 128 + right). Other long ranges are swept in row groups of 128 rows whose keys
// pass through LDS in chunks, with the O accumulators and the online-softmax state
// carried across chunks in registers.
#pragma once

#include "gdpa_device.hpp"
#include "gdpa_launch.hpp"

namespace gdpa {

// Launch modes, by the problems in the launch:
//   kFwdAny       any key length: resident keys, ring window or key chunks; 4 waves per workgroup,
//                 2 workgroups/CU (2 waves per SIMD);
//   kFwdResident  d <= 64 and every key range fits in LDS (at most 16384 / d keys): only the
//                 resident path is built, whose smaller register footprint allows 8 waves per
//                 workgroup, 2 workgroups/CU (4 waves per SIMD);
//   kFwdLong8     d <= 64, some key range longer than that and no window: 8 waves as above with
//                 the key-chunk path, whose row groups of 256 rows stage each key range half as
//                 often as groups of 128.
enum FwdMode { kFwdAny = 0, kFwdResident = 1, kFwdLong8 = 2 };
template <int MODE>
constexpr int fwd_waves() { return MODE == kFwdAny ? 4 : 8; }
// minimum waves per SIMD (the second launch bound)
template <int MODE>
constexpr int fwd_waves_per_simd() { return MODE == kFwdAny ? 2 : 4; }
// Keys staged in LDS at once.
template <int D, int MODE>
constexpr int fwd_nkv() { return 16384 / D; }

template <int D, int KEYS>
struct FwdGeo {
  static constexpr int NKV = KEYS;             // keys that fit in LDS
  static constexpr int KROW = D * 2 + 16;      // bytes per staged K row (16 B pad: no bank conflicts)
  static constexpr int VROW = NKV * 2 + 16;    // bytes per staged V^T row
  static constexpr int KK = D / 16;            // MFMA k-steps over d
  static constexpr int DT = D / 32;            // 32-wide d tiles of the output
  static constexpr int OFF_V = NKV * KROW;
  static constexpr int OFF_G = OFF_V + D * VROW;
  static constexpr int OFF_KN = OFF_G + NKV * 4;  // per-wave maxima of the staged keys' ||k||^2
  static constexpr int BYTES = OFF_KN + 16 * 4;
};

constexpr int fwd_max3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }
template <int MODE>
constexpr int fwd_lds_bytes() {
  return fwd_max3(FwdGeo<32, fwd_nkv<32, MODE>()>::BYTES, FwdGeo<64, fwd_nkv<64, MODE>()>::BYTES,
                  FwdGeo<128, fwd_nkv<128, MODE>()>::BYTES);
}

// Position of local key kl inside the staged V^T row: blocks of 32 keys, halves of 16, and the
// slot order of the B operand inside each half.
__device__ inline int vt_pos(int kl) { return (kl & ~15) + slot_row(kl & 15); }

// Stage keys [k0, k0 + span) of one (sequence, head) into LDS; rows up to span_pad are zeroed.
// Every global load of the range is issued before the first LDS write, so the staging costs one
// memory latency. K rows are copied as 16-byte chunks; V is transposed in units of 4 consecutive
// keys x 8 d: the 4 keys of one d are adjacent in the V^T slot order, so each d is one 8-byte
// write.
// The keys land at LDS key positions dst + (0 .. span_pad-1) (dst a multiple of 32).
// SERIAL: keep the rounds in order (the caller holds accumulators in registers across the staging).
// KNORM: each wave also writes the largest ||k||^2 of the keys it staged to G::OFF_KN + 4 w.
template <int D, int NKV, int NT, bool SERIAL = false, bool KNORM = false>
__device__ void stage_kv(char* lds, const bf16* kb, const bf16* vb, const float* gb, int hstride,
                         int span, int span_pad, bool softmax, int dst = 0) {
  using G = FwdGeo<D, NKV>;
  constexpr int CPR = D / 8;                                  // 16-byte chunks per row
  constexpr int KI = (G::NKV * CPR + NT - 1) / NT;           // K chunks per thread (at most)
  constexpr int VI = (G::NKV / 4 * CPR + NT - 1) / NT;       // V units per thread (at most)
  constexpr int GI = (G::NKV + NT - 1) / NT;                 // gate values per thread
  // d = 128: one round per 16-byte chunk group (the d = 128 kernels have no registers to spare)
  constexpr int ROUNDS = D == 128 ? KI : 1;
  static_assert(KI % ROUNDS == 0, "staging rounds");
  const size_t rs = (size_t)hstride * D;
  float gv[GI];
#pragma unroll
  for (int i = 0; i < GI; ++i) {
    const int r = threadIdx.x + i * NT;
    gv[i] = 0.0f;
    if (gb != nullptr && r < span) gv[i] = gb[(size_t)r * hstride];
  }
  float kn2 = 0.0f;  // KNORM: largest ||k||^2 among this lane's rows
  auto stage_round = [&](int round) {
    constexpr int KR = KI / ROUNDS, VR = (VI + ROUNDS - 1) / ROUNDS;
    u32x4 kbuf[KR], vbuf[VR][4];
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      const int idx = threadIdx.x + (round * KR + i) * NT;
      const int r = idx / CPR, c = idx % CPR;
      kbuf[i] = u32x4{0u, 0u, 0u, 0u};
      if (idx < span_pad * CPR && r < span) kbuf[i] = *reinterpret_cast<const u32x4*>(kb + r * rs + c * 8);
    }
    if constexpr (KNORM) {
      // a row's CPR chunks sit in CPR consecutive lanes: their partial sums meet by lane shuffles
#pragma unroll
      for (int i = 0; i < KR; ++i) {
        float n2 = sumsq_bf16x8(kbuf[i]);
#pragma unroll
        for (int off = 1; off < CPR; off <<= 1) n2 += __shfl_xor(n2, off, 64);
        kn2 = fmaxf(kn2, n2);
      }
    }
#pragma unroll
    for (int i = 0; i < VR; ++i) {
      const int u = threadIdx.x + (round * VR + i) * NT;
      const int r4 = (u / CPR) * 4, c = u % CPR;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vbuf[i][e] = u32x4{0u, 0u, 0u, 0u};
        if (u < span_pad / 4 * CPR && r4 + e < span)
          vbuf[i][e] = *reinterpret_cast<const u32x4*>(vb + (r4 + e) * rs + c * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < KR; ++i) {
      const int idx = threadIdx.x + (round * KR + i) * NT;
      const int r = idx / CPR, c = idx % CPR;
      if (idx < span_pad * CPR) *reinterpret_cast<u32x4*>(lds + (dst + r) * G::KROW + c * 16) = kbuf[i];
    }
#pragma unroll
    for (int i = 0; i < VR; ++i) {
      const int u = threadIdx.x + (round * VR + i) * NT;
      const int r4 = (u / CPR) * 4, c = u % CPR;
      if (u < span_pad / 4 * CPR) {
        char* vt = lds + G::OFF_V + (dst + vt_pos(r4)) * 2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // d = 8c + e of keys r4 .. r4+3: 16-bit half (e & 1) of word e / 2 of each key's chunk
          const int wd = e >> 1;
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x2 pk;
          pk[0] = __builtin_amdgcn_perm(vbuf[i][1][wd], vbuf[i][0][wd], sel);
          pk[1] = __builtin_amdgcn_perm(vbuf[i][3][wd], vbuf[i][2][wd], sel);
          *reinterpret_cast<u32x2*>(vt + (c * 8 + e) * G::VROW) = pk;
        }
      }
    }
  };
  if constexpr (SERIAL) {
#pragma unroll 1
    for (int round = 0; round < ROUNDS; ++round) stage_round(round);
  } else {
#pragma unroll
    for (int round = 0; round < ROUNDS; ++round) stage_round(round);
  }
  if constexpr (KNORM) {
    kn2 = wave_max(kn2);
    if (lane_id() == 0) reinterpret_cast<float*>(lds + G::OFF_KN)[threadIdx.x >> 6] = kn2;
  }
  float* gl = reinterpret_cast<float*>(lds + G::OFF_G) + dst;
#pragma unroll
  for (int i = 0; i < GI; ++i) {
    const int r = threadIdx.x + i * NT;
    if (r < span_pad) {
      float t = 0.0f;
      if (gb != nullptr && r < span) {
        t = log_sigmoid_f(gv[i]);
        if (softmax) t *= kLog2e;
      }
      gl[r] = t;
    }
  }
}

// One wave: QS x 32 query rows starting at row0 (sequence-relative) against local key blocks
// [kb0, kb1) of the staged range, whose first key has sequence position klo.
// Q fragments of one wave tile: lane (row, g) holds d = g*D/2 + kk*8 + 0..7 of its row.
template <int D, int QS>
struct QFrags {
  bf16x8 f[QS][D / 16];
};

template <int D, int QS>
__device__ inline void load_q(QFrags<D, QS>& q, const bf16* qseq, size_t rs, int row0, int L) {
  const int lane = lane_id(), qc = lane & 31, g = lane >> 5;
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int row = row0 + qs * 32 + qc;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (row < L) u = *reinterpret_cast<const u32x4*>(qseq + row * rs + g * (D / 2) + kk * 8);
      q.f[qs][kk] = as_bf16x8(u);
    }
  }
}

// Largest ||q||^2 over the wave tile's rows (rows past the end are zero); uniform across the wave.
template <int D, int QS>
__device__ inline float q_norm_max(const QFrags<D, QS>& q) {
  float m = 0.0f;
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    float n2 = 0.0f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) n2 += sumsq_bf16x8(__builtin_bit_cast(u32x4, q.f[qs][kk]));
    n2 += __shfl_xor(n2, 32, 64);  // the two halves of the row
    m = fmaxf(m, n2);
  }
  return wave_max(m);
}

// S^T block kb (32 keys x QS*32 rows) = K_kb Q^T on MFMA, K rows from LDS.
template <int D, int NKV, int QS>
__device__ inline void scores_block(const char* lds, const QFrags<D, QS>& q, int kb, f32x16 (&s)[QS]) {
  using G = FwdGeo<D, NKV>;
  const int lane = lane_id(), qc = lane & 31, g = lane >> 5;
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) s[qs] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < G::KK; ++kk) {
    const u32x4 ku = *reinterpret_cast<const u32x4*>(lds + (kb * 32 + qc) * G::KROW + g * D + kk * 16);
    const bf16x8 kf = as_bf16x8(ku);
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) s[qs] = mfma32(kf, q.f[qs][kk], s[qs]);
  }
}

// Running state of one wave's query tile: the O accumulators and, for softmax, the running row
// maximum (log2 units) and the lane's partial row sum.
template <int D, int QS>
struct FwdAcc {
  f32x16 o[QS][D / 32];
  float m[QS], lsum[QS];
};

template <int D, int QS>
__device__ __forceinline__ void acc_init(FwdAcc<D, QS>& a) {
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    a.m[qs] = -__builtin_inff();
    a.lsum[qs] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) a.o[qs][dt] = f32x16{};
  }
}

// Adds key blocks [kb0, kb1) to the wave's tile state. Block b holds keys kbase + 32 b + (0..31)
// (keys from kend on are invalid) and sits in LDS block slot b, or b mod NKV / 32 (RING).
// GATED: the problem has a gate. MASKED: entries may need an explicit mask (the softmax form, or
// a window); without it, keys past the end meet zero K and V rows in LDS and phi(0) = 0.
// PSPLIT: at most kSplitTerms keys, so each output is a sum of that few products; P then enters
// O^T = V^T P^T as a high + low bf16 pair (its single rounding would be too coarse there).
// SERIES: ungated element-wise tile whose arguments are all proven within the series range
// (SeriesAct instead of PointAct): 1 = |x| <= kSeriesBound, 2 = within the shorter series' range.
template <int D, int NKV, int ACT, int QS, bool GATED, bool MASKED, bool RING = false, bool PIPE = true,
          bool PSPLIT = false, int SERIES = 0>
__device__ __forceinline__ void fwd_accumulate(const char* lds, const GroupDesc& gd, const QFrags<D, QS>& qf,
                                               FwdAcc<D, QS>& acc, int row0, int kbase, int kend, int kb0,
                                               int kb1) {
  using G = FwdGeo<D, NKV>;
  const int lane = lane_id(), qc = lane & 31, g = lane >> 5;
  constexpr bool softmax = ACT == GDPA_ACT_SOFTMAX;
  const float* gl = reinterpret_cast<const float*>(lds + G::OFF_G);
  auto& o = acc.o;
  auto& m = acc.m;
  auto& lsum = acc.lsum;
  const float sc = softmax ? gd.scale * kLog2e : gd.scale;
  const int wl = gd.wl, wr = gd.wr;
  constexpr int smask = RING ? G::NKV / 32 - 1 : -1;  // block -> LDS slot
  // element-wise forms: without a gate p' = s g(scale s) = phi(scale s) / scale and O is scaled
  // once in the epilogue; with a gate the argument scale s + log sigmoid(G) is formed first.
  float c1 = 0.0f, c3 = 0.0f, a1 = 0.0f, a3 = 0.0f, d1 = 0.0f, d3 = 0.0f;
  static_assert(!SERIES || (!GATED && !softmax), "series only for ungated element-wise tiles");
  if constexpr (SERIES) SeriesAct<ACT>::coeffs(gd.scale, a1, a3, d1, d3);
  else if constexpr (!softmax) PointAct<ACT>::coeffs(GATED ? 1.0f : gd.scale, c1, c3);

  // Element-wise stage and P V for block kb whose scores are in s: register r of lane (qc, g) is
  // key kbase + kb*32 + c_row(r, g), row qs*32 + qc.
  auto process = [&](int kb, const f32x16 (&s)[QS]) {
    const int slot = kb & smask;  // LDS block slot
    float p[QS][16];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x;
        if constexpr (GATED) x = __builtin_fmaf(s[qs][r], sc, gl[slot * 32 + c_row(r, g)]);
        if constexpr (softmax) p[qs][r] = GATED ? x : s[qs][r] * sc;
        else if constexpr (SERIES == 2) p[qs][r] = SeriesAct<ACT>::value_short(s[qs][r], a1);
        else if constexpr (SERIES == 1) p[qs][r] = SeriesAct<ACT>::value(s[qs][r], a1, a3);
        else p[qs][r] = GATED ? PointAct<ACT>::value(x, c1, c3) : PointAct<ACT>::value(s[qs][r], c1, c3);
      }
    if constexpr (MASKED) {
      const int kfirst = kbase + kb * 32, klast = kfirst + 31;
      bool full_block = klast < kend;
      const int rfirst = row0, rlast = row0 + QS * 32 - 1;
      if (wl >= 0 && kfirst < rlast - wl) full_block = false;
      if (wr >= 0 && klast > rfirst + wr) full_block = false;
      if (!full_block) {
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          // this lane's row sees keys [klo, khi] of the block's (register r: key kfirst + c_row(r, g))
          const int row = row0 + qs * 32 + qc;
          int klo = kfirst, khi = kend - 1;
          if (wl >= 0) klo = max(klo, row - wl);
          if (wr >= 0) khi = min(khi, row + wr);
          const LaneRange mr = lane_range(kfirst, klo, khi);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            p[qs][r] = lane_ok(mr, r, g) ? p[qs][r] : (softmax ? -__builtin_inff() : 0.0f);
        }
      }
    }
    if constexpr (softmax) {
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        float bm = p[qs][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) bm = fmaxf(bm, p[qs][r]);
        bm = half32_max(bm);
        const float mnew = fmaxf(m[qs], bm);
        const float msafe = mnew == -__builtin_inff() ? 0.0f : mnew;
        const float alpha = fast_exp2(m[qs] - msafe);
        float rs_ = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[qs][r] = fast_exp2(p[qs][r] - msafe);
          rs_ += p[qs][r];
        }
        lsum[qs] = lsum[qs] * alpha + rs_;
        m[qs] = mnew;
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt) o[qs][dt] *= alpha;
      }
    }
    // P^T as B operand: k-tile t takes registers 8t..8t+7 (PSPLIT: and the rounding remainder)
    bf16x8 pf[QS][2], pl[QS][2];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 u, ul;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u[e] = pack_bf16x2(p[qs][8 * t + 2 * e], p[qs][8 * t + 2 * e + 1]);
          if constexpr (PSPLIT)
            ul[e] = pack_bf16x2(p[qs][8 * t + 2 * e] - bf16_lo(u[e]), p[qs][8 * t + 2 * e + 1] - bf16_hi(u[e]));
        }
        pf[qs][t] = as_bf16x8(u);
        if constexpr (PSPLIT) pl[qs][t] = as_bf16x8(ul);
      }
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 vu = *reinterpret_cast<const u32x4*>(lds + G::OFF_V + (dt * 32 + out_perm(qc)) * G::VROW +
                                                         (slot * 32 + t * 16 + g * 8) * 2);
        const bf16x8 vf = as_bf16x8(vu);
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          o[qs][dt] = mfma32(vf, pf[qs][t], o[qs][dt]);
          if constexpr (PSPLIT) o[qs][dt] = mfma32(vf, pl[qs][t], o[qs][dt]);
        }
      }
  };

  if constexpr (!PIPE) {
    // one score buffer: with four waves per SIMD the other waves' element-wise work covers each
    // wave's MFMA chain, and the 16 registers of a second buffer are worth more as headroom
    f32x16 sa[QS];
    for (int kb = kb0; kb < kb1; ++kb) {
      scores_block<D, NKV, QS>(lds, qf, kb & smask, sa);
      process(kb, sa);
    }
    return;
  }
  // Software pipeline over pairs of blocks with two score buffers: the score MFMAs of the next
  // block are issued before the element-wise work of the current one, so the matrix cores run
  // while the vector units evaluate the activation; the loop body has no branches.
  f32x16 sa[QS], sb[QS];
  int kb = kb0;
  if (kb < kb1) scores_block<D, NKV, QS>(lds, qf, kb & smask, sa);
  for (; kb + 2 < kb1; kb += 2) {
    scores_block<D, NKV, QS>(lds, qf, (kb + 1) & smask, sb);
    process(kb, sa);
    scores_block<D, NKV, QS>(lds, qf, (kb + 2) & smask, sa);
    process(kb + 1, sb);
  }
  if (kb + 1 < kb1) {
    scores_block<D, NKV, QS>(lds, qf, (kb + 1) & smask, sb);
    process(kb, sa);
    process(kb + 1, sb);
  } else if (kb < kb1) {
    process(kb, sa);
  }

}

// Epilogue of one wave tile: softmax normalisation and lse, or the deferred score scale of the
// element-wise forms; each lane stores 16 consecutive d of one row.
template <int D, int NKV, int ACT, int QS, bool GATED>
__device__ __forceinline__ void fwd_finish(const GroupDesc& gd, const FwdAcc<D, QS>& acc, OutPtr oseq, float* lseq,
                                           int L, int row0) {
  using G = FwdGeo<D, NKV>;
  const int lane = lane_id(), qc = lane & 31, g = lane >> 5;
  const int H = gd.num_heads;
  const size_t rs = (size_t)H * D;
  constexpr bool softmax = ACT == GDPA_ACT_SOFTMAX;
  const float out_scale = (!softmax && !GATED) ? gd.scale : 1.0f;
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int row = row0 + qs * 32 + qc;
    float inv = out_scale, lse = 0.0f;
    if (softmax) {
      const float ltot = half32_sum(acc.lsum[qs]);
      inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
      lse = ltot > 0.0f ? (acc.m[qs] + __log2f(ltot)) * 0.69314718055994531f : -__builtin_inff();
    }
    if (row < L) {
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt) {
        const f32x16& o = acc.o[qs][dt];
        const OutPtr dst = oseq + (row * rs + dt * 32 + g * 16);
        out_store8(dst, f32x4{o[0], o[1], o[2], o[3]} * inv, f32x4{o[4], o[5], o[6], o[7]} * inv);
        out_store8(dst + 8, f32x4{o[8], o[9], o[10], o[11]} * inv, f32x4{o[12], o[13], o[14], o[15]} * inv);
      }
      if (softmax && g == 0) lseq[(size_t)row * H] = lse;
    }
  }
}

// One wave tile against staged key blocks [kb0, kb1), then its epilogue.
template <int D, int NKV, int ACT, int QS, bool GATED, bool MASKED, bool PIPE, bool PSPLIT = false,
          int SERIES = 0>
__device__ __forceinline__ void fwd_tile(const char* lds, const GroupDesc& gd, const QFrags<D, QS>& qf, OutPtr oseq,
                                         float* lseq, int L, int row0, int klo, int span, int kb0, int kb1) {
  FwdAcc<D, QS> acc;
  acc_init(acc);
  fwd_accumulate<D, NKV, ACT, QS, GATED, MASKED, false, PIPE, PSPLIT, SERIES>(lds, gd, qf, acc, row0, klo, klo + span,
                                                                              kb0, kb1);
  fwd_finish<D, NKV, ACT, QS, GATED>(gd, acc, oseq, lseq, L, row0);
}

// Whether a bounded window's key range for a group of NW * 32 rows fits in the ring of LDS blocks.
template <int D, int NKV>
__device__ __forceinline__ bool fwd_ring_fits(int wl, int wr, int group_rows) {
  if (wl < 0 || wr < 0) return false;
  return (group_rows - 1 + wr) / 32 + (wl + 31) / 32 + 1 <= FwdGeo<D, NKV>::NKV / 32;
}

// One work item: all query rows of one (sequence, head). QS: 32-row tiles per wave while the keys
// are resident or pass through the ring; QL: the same in the key-chunked sweep.
// LONG: the launch may hold key ranges longer than NKV (else only the resident path is built).
template <int D, int NKV, int NW, int ACT, int QS, int QL, bool GATED, bool MASKED, bool LONG>
__device__ __forceinline__ void fwd_item(char* lds, const GroupDesc& gd, int b, int h) {
  using G = FwdGeo<D, NKV>;
  const int q0 = gd.q_off[b], L = gd.q_off[b + 1] - q0;
  const int k0 = gd.kv_off[b], N = gd.kv_off[b + 1] - k0;
  if (L <= 0) return;
  const int H = gd.num_heads;
  const size_t rs = (size_t)H * D;
  // a shared query matrix (seed queries): every sequence reads its query rows from row 0
  const size_t qrow = gd.shared_q ? 0 : (size_t)q0;
  const bf16* qseq = reinterpret_cast<const bf16*>(gd.q) + (qrow * H + h) * D;
  const OutPtr oseq = out_ptr(gd.o, gd.out_f32, ((size_t)q0 * H + h) * D);
  float* lseq = gd.lse ? gd.lse + (size_t)q0 * H + h : nullptr;
  const bf16* kseq = reinterpret_cast<const bf16*>(gd.k) + ((size_t)k0 * H + h) * D;
  const bf16* vseq = reinterpret_cast<const bf16*>(gd.v) + ((size_t)k0 * H + h) * D;
  const float* gseq = gd.g ? gd.g + (size_t)k0 * H + h : nullptr;
  constexpr bool softmax = ACT == GDPA_ACT_SOFTMAX;
  const int w = wave_id();
  constexpr int RW = QS * 32;  // rows per wave tile

  if (N <= G::NKV) {
    // whole key range resident: stage once, sweep all query tiles
    const int span_pad = (N + 31) & ~31;
    // 4 waves: each next tile's Q is in flight during the current tile (at d = 128 this takes the
    // registers of the second score buffer, which that build gives up); 8 waves: the other waves
    // hide the load
    constexpr bool kPrefetchQ = NW == 4;
    // every wave's first tile is in flight during the staging (one memory latency)
    constexpr bool kFirstQEarly = true;
    // ungated element-wise items: tiles proven within the series range take SeriesAct
    constexpr bool kSeriesItem = !softmax && !GATED;
    QFrags<D, QS> qcur, qnext;
    if (kFirstQEarly && w * RW < L) load_q<D, QS>(qcur, qseq, rs, w * RW, L);
    stage_kv<D, NKV, NW * kWave, false, kSeriesItem>(lds, kseq, vseq, gseq, H, N, span_pad, softmax);
    __syncthreads();
    float kn2 = 0.0f;  // largest ||k||^2 of the item's keys
    if constexpr (kSeriesItem)
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) kn2 = fmaxf(kn2, reinterpret_cast<const float*>(lds + G::OFF_KN)[ww]);
    for (int row0 = w * RW; row0 < L; row0 += NW * RW) {
      // next tile's Q is loaded while this tile computes
      if (!kPrefetchQ && !(kFirstQEarly && row0 == w * RW)) load_q<D, QS>(qcur, qseq, rs, row0, L);
      if (kPrefetchQ && row0 + NW * RW < L) load_q<D, QS>(qnext, qseq, rs, row0 + NW * RW, L);
      int lo = 0, hi = N - 1;
      if (gd.wl >= 0) lo = row0 - gd.wl > 0 ? row0 - gd.wl : 0;
      if (gd.wr >= 0) hi = row0 + RW - 1 + gd.wr < N - 1 ? row0 + RW - 1 + gd.wr : N - 1;
      const int kb0 = lo / 32, kb1 = hi >= lo ? hi / 32 + 1 : kb0;
      // (8 waves: four per SIMD, no software pipeline inside a wave; 4 waves: two per SIMD, with it)
      int series = 0;  // 2: within the shorter series' range, 1: within kSeriesBound
      if constexpr (kSeriesItem) {
        const float qn2 = q_norm_max<D, QS>(qcur);
        series = seq_series_within(gd.scale, qn2, kn2, series_short_bound_fwd<ACT>()) ? 2
                 : seq_series_ok(gd.scale, qn2, kn2)                              ? 1
                                                                                  : 0;
      }
      if (N <= kSplitTerms)
        fwd_tile<D, NKV, ACT, QS, GATED, MASKED, false, true>(lds, gd, qcur, oseq, lseq, L, row0, 0, N, kb0, kb1);
      else if (kSeriesItem && series == 2)
        fwd_tile<D, NKV, ACT, QS, GATED, MASKED, (NW == 4 && D < 128), false, kSeriesItem ? 2 : 0>(
            lds, gd, qcur, oseq, lseq, L, row0, 0, N, kb0, kb1);
      else if (kSeriesItem && series == 1)
        fwd_tile<D, NKV, ACT, QS, GATED, MASKED, (NW == 4 && D < 128), false, kSeriesItem ? 1 : 0>(
            lds, gd, qcur, oseq, lseq, L, row0, 0, N, kb0, kb1);
      else
        fwd_tile<D, NKV, ACT, QS, GATED, MASKED, (NW == 4 && D < 128)>(lds, gd, qcur, oseq, lseq, L, row0, 0, N, kb0, kb1);
      if (kPrefetchQ) qcur = qnext;
    }
  } else if (LONG && D < 128 && fwd_ring_fits<D, NKV>(gd.wl, gd.wr, NW * RW)) {
    // bounded window over a long sequence: the keys pass through a ring of NKV / 32 LDS blocks
    // (block b in slot b mod NKV / 32); each group of NW * RW rows stages only the blocks that
    // enter its key range [r0 - left, r0 + NW * RW + right), so every key is read once
    constexpr int NSLOT = G::NKV / 32;
    constexpr bool kHoldQ = D < 128;
    int staged = 0;  // blocks [.., staged) are in the ring
    for (int r0 = 0; r0 < L; r0 += NW * RW) {
      const int row0 = r0 + w * RW;
      const bool active = row0 < L;
      QFrags<D, QS> qf;
      if (kHoldQ && active) load_q<D, QS>(qf, qseq, rs, row0, L);  // in flight during the staging
      const int glo = r0 - gd.wl > 0 ? r0 - gd.wl : 0;
      const int ghi = r0 + NW * RW + gd.wr < N ? r0 + NW * RW + gd.wr : N;  // exclusive
      const int blast = (ghi - 1) / 32;
      int bnext = glo / 32 > staged ? glo / 32 : staged;
      if (bnext <= blast) {
        __syncthreads();  // the slots about to be replaced are no longer read
        while (bnext <= blast) {
          const int slot = bnext & (NSLOT - 1);
          const int nblk = blast - bnext + 1 < NSLOT - slot ? blast - bnext + 1 : NSLOT - slot;
          const int k0 = bnext * 32;
          const int span = N - k0 < nblk * 32 ? N - k0 : nblk * 32;
          stage_kv<D, NKV, NW * kWave>(lds, kseq + (size_t)k0 * H * D, vseq + (size_t)k0 * H * D,
                                           gseq ? gseq + (size_t)k0 * H : nullptr, H, span, nblk * 32, softmax,
                                           slot * 32);
          bnext += nblk;
        }
        staged = blast + 1;
        __syncthreads();
      }
      if (active) {
        int lo = row0 - gd.wl > 0 ? row0 - gd.wl : 0;
        int hi = row0 + RW - 1 + gd.wr < N - 1 ? row0 + RW - 1 + gd.wr : N - 1;
        if (!kHoldQ) load_q<D, QS>(qf, qseq, rs, row0, L);
        FwdAcc<D, QS> acc;
        acc_init(acc);
        if (hi >= lo)
          fwd_accumulate<D, NKV, ACT, QS, GATED, MASKED, true, (NW == 4 && D < 128)>(lds, gd, qf, acc, row0, 0, N, lo / 32,
                                                                      hi / 32 + 1);
        fwd_finish<D, NKV, ACT, QS, GATED>(gd, acc, oseq, lseq, L, row0);
      }
    }
  } else if (LONG) {
    // long key range: row groups of NW * QL * 32 rows; for each, the group's key range (all keys,
    // or [r0 - left, r0 + rows + right) under a window) is staged in chunks of NKV keys and every
    // wave carries its tile's O and softmax state across the chunks.
    constexpr int RL = QL * 32;
    for (int r0 = 0; r0 < L; r0 += NW * RL) {
      const int row0 = r0 + w * RL;
      const bool active = row0 < L;
      int glo = 0, ghi = N;
      if (gd.wl >= 0) glo = r0 - gd.wl > 0 ? r0 - gd.wl : 0;
      if (gd.wr >= 0 && r0 + NW * RL + gd.wr < N) ghi = r0 + NW * RL + gd.wr;
      // the wave's own key range [lo, hi]
      int lo = 0, hi = N - 1;
      if (gd.wl >= 0) lo = row0 - gd.wl > 0 ? row0 - gd.wl : 0;
      if (gd.wr >= 0) hi = row0 + RL - 1 + gd.wr < N - 1 ? row0 + RL - 1 + gd.wr : N - 1;
      // d <= 64: Q stays in registers across the chunks; d = 128 reloads it per chunk (from L2)
      // to keep the register file free for the staging
      constexpr bool kHoldQ = D < 128;
      QFrags<D, QL> qf;
      if (kHoldQ && active) load_q<D, QL>(qf, qseq, rs, row0, L);
      FwdAcc<D, QL> acc;
      acc_init(acc);
      for (int kc = glo; kc < ghi; kc += G::NKV) {
        const int span = ghi - kc < G::NKV ? ghi - kc : G::NKV;
        __syncthreads();  // previous chunk done with LDS
        stage_kv<D, NKV, NW * kWave, true>(lds, kseq + (size_t)kc * H * D, vseq + (size_t)kc * H * D,
                    gseq ? gseq + (size_t)kc * H : nullptr, H, span, (span + 31) & ~31, softmax);
        __syncthreads();
        const int clo = lo > kc ? lo : kc;
        const int chi = hi < kc + span - 1 ? hi : kc + span - 1;
        if (active && chi >= clo) {
          if (!kHoldQ) load_q<D, QL>(qf, qseq, rs, row0, L);
          fwd_accumulate<D, NKV, ACT, QL, GATED, MASKED, false, (NW == 4 && D < 128)>(lds, gd, qf, acc, row0, kc, kc + span,
                                                                     (clo - kc) / 32, (chi - kc) / 32 + 1);
        }
      }
      if (active) fwd_finish<D, NKV, ACT, QL, GATED>(gd, acc, oseq, lseq, L, row0);
    }
  }
}

// Gate and mask variants of one activation: a window and the softmax form are masked; a problem
// without window or softmax runs the mask-free body.
template <int D, int NKV, int NW, int ACT, int QS, bool LONG>
__device__ __forceinline__ void fwd_dispatch_variant(char* lds, const GroupDesc& gd, int b, int h) {
  constexpr int QL = 1;  // (two tiles per wave in the key-chunked sweep spill registers)
  const bool masked = ACT == GDPA_ACT_SOFTMAX || gd.wl >= 0 || gd.wr >= 0;
  if (gd.g != nullptr) {
    if (masked) fwd_item<D, NKV, NW, ACT, QS, QL, true, true, LONG>(lds, gd, b, h);
    else if constexpr (ACT != GDPA_ACT_SOFTMAX) fwd_item<D, NKV, NW, ACT, QS, QL, true, false, LONG>(lds, gd, b, h);
  } else {
    if (masked) fwd_item<D, NKV, NW, ACT, QS, QL, false, true, LONG>(lds, gd, b, h);
    else if constexpr (ACT != GDPA_ACT_SOFTMAX) fwd_item<D, NKV, NW, ACT, QS, QL, false, false, LONG>(lds, gd, b, h);
  }
}

template <int D, int NKV, int NW, int ASET, bool LONG>
__device__ __forceinline__ void fwd_dispatch_act(char* lds, const GroupDesc& gd, int b, int h) {
  if constexpr ((ASET & (1 << GDPA_ACT_GELU)) != 0)
    if (gd.act == GDPA_ACT_GELU) { fwd_dispatch_variant<D, NKV, NW, GDPA_ACT_GELU, 1, LONG>(lds, gd, b, h); return; }
  if constexpr ((ASET & (1 << GDPA_ACT_SILU)) != 0)
    if (gd.act == GDPA_ACT_SILU) { fwd_dispatch_variant<D, NKV, NW, GDPA_ACT_SILU, 1, LONG>(lds, gd, b, h); return; }
  if constexpr ((ASET & (1 << GDPA_ACT_SOFTMAX)) != 0)
    if (gd.act == GDPA_ACT_SOFTMAX) fwd_dispatch_variant<D, NKV, NW, GDPA_ACT_SOFTMAX, 1, LONG>(lds, gd, b, h);
}

template <int DSET, int ASET, int MODE>
__global__ void __launch_bounds__(fwd_waves<MODE>() * kWave, fwd_waves_per_simd<MODE>()) fwd_bf16_kernel(LaunchDesc d) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  if ((int)blockIdx.x >= d.n_items || launch_refused(d)) return;
  int g, h, b;
  unpack_item(d.items[xcd_item((int)blockIdx.x, d.n_items)], g, h, b);
  if (g >= d.n_groups) return;
  GroupDesc gd = select_group(d, g);
  if (b >= gd.num_seqs || h >= gd.num_heads) return;  // list built for another shape
  {
    // the resident-only build holds at most 16384 / d keys per item
    const int32_t e = item_error(gd, gd.q_off[b], gd.q_off[b + 1], gd.kv_off[b], gd.kv_off[b + 1],
                                 MODE == kFwdResident ? 16384 / gd.head_dim : -1);
    if (e != 0) {
      if (threadIdx.x == 0) report_error(d, e);
      return;
    }
  }
  if (gd.head_acts != nullptr) gd.act = gd.head_acts[h];  // activation of this item's head
  constexpr int NW = fwd_waves<MODE>();
  constexpr bool LONG = MODE != kFwdResident;
  if constexpr ((DSET & kDim32) != 0)
    if (gd.head_dim == 32) { fwd_dispatch_act<32, fwd_nkv<32, MODE>(), NW, ASET, LONG>(lds, gd, b, h); return; }
  if constexpr ((DSET & kDim64) != 0)
    if (gd.head_dim == 64) { fwd_dispatch_act<64, fwd_nkv<64, MODE>(), NW, ASET, LONG>(lds, gd, b, h); return; }
  if constexpr ((DSET & kDim128) != 0)
    if (gd.head_dim == 128) { fwd_dispatch_act<128, fwd_nkv<128, MODE>(), NW, ASET, LONG>(lds, gd, b, h); return; }
}

template <int MODE>
hipError_t launch_fwd_bf16_t(const LaunchDesc& d, int dim_set, int act_set, hipStream_t stream) {
  const dim3 grid(d.n_items);
  constexpr int kAll = (1 << GDPA_ACT_GELU) | (1 << GDPA_ACT_SILU) | (1 << GDPA_ACT_SOFTMAX);
#define GDPA_LAUNCH(DS, AS) \
  hipLaunchKernelGGL((fwd_bf16_kernel<DS, AS, MODE>), grid, dim3(fwd_waves<MODE>() * kWave), \
                     (fwd_lds_bytes<MODE>()), stream, d)
#define GDPA_LAUNCH_ACTS(DS)                                          \
  switch (act_set) {                                                  \
    case 1 << GDPA_ACT_GELU: GDPA_LAUNCH(DS, 1 << GDPA_ACT_GELU); break;  \
    case 1 << GDPA_ACT_SILU: GDPA_LAUNCH(DS, 1 << GDPA_ACT_SILU); break;  \
    case 1 << GDPA_ACT_SOFTMAX: GDPA_LAUNCH(DS, 1 << GDPA_ACT_SOFTMAX); break; \
    default: GDPA_LAUNCH(DS, kAll); break;                            \
  }
  if constexpr (MODE != kFwdAny) {  // d <= 64 only (d = 128 does not fit 128 registers)
    switch (dim_set) {
      case kDim32: GDPA_LAUNCH_ACTS(kDim32); break;
      case kDim64: GDPA_LAUNCH_ACTS(kDim64); break;
      default: GDPA_LAUNCH_ACTS(kDim32 | kDim64); break;
    }
  } else {
    switch (dim_set) {
      case kDim32: GDPA_LAUNCH_ACTS(kDim32); break;
      case kDim64: GDPA_LAUNCH_ACTS(kDim64); break;
      case kDim128: GDPA_LAUNCH_ACTS(kDim128); break;
      default: GDPA_LAUNCH_ACTS(kDim32 | kDim64 | kDim128); break;  // several head dims
    }
  }
#undef GDPA_LAUNCH_ACTS
#undef GDPA_LAUNCH
  return hipGetLastError();
}

}  // namespace gdpa
