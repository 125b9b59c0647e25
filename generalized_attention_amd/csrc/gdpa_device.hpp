// Device-side building blocks of the gfx950 GDPA kernels: descriptor types, the bf16 MFMA
// fragment conventions, element-wise activations, and small LDS/global helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdpa.h"

namespace gdpa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kThreads = 256;  // 4 waves per workgroup
constexpr int kNumBuckets = 1024;

// ----------------------------------------------------------------------------------------------
// Per-group descriptor handed to the kernels by value (kernel arguments).
// ----------------------------------------------------------------------------------------------
struct GroupDesc {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  void* o;
  float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* delta;  // softmax backward: D_i = sum_j p_ij dp_ij per (row, head), in the workspace
  float* dq32;   // backward in key chunks: fp32 dQ accumulation rows (workspace), row stride H*d
  const int32_t* q_off;
  const int32_t* kv_off;
  const int32_t* head_acts;  // activation per head, or null (act for every head)
  int32_t num_seqs;
  int32_t num_heads;
  int32_t head_dim;
  int32_t act;
  float scale;
  int32_t wl;
  int32_t wr;
  int32_t seq_base;   // index of this group's first sequence in the global sequence numbering
  int32_t shared_q;   // rows of a query matrix shared by every sequence (0: per-sequence queries)
  int32_t out_f32;    // bf16 problem whose outputs o, dq, dk, dv are float32
  int32_t total_q;    // rows of o / dout (and of q unless shared)
  int32_t total_kv;   // rows of k, v
  int32_t max_q;      // max_seqlen_q hint
  int32_t max_kv;     // max_seqlen_kv hint
  int32_t self_attn;  // query and key sequences are the same rows
  int32_t split_all;  // element-wise backward: P and dS as high + low bf16 pairs in every item
  int32_t short_keys; // backward: the group's items run the one-wave short-key kernel; the work
                      // list puts them after every other group's items
};

struct LaunchDesc {
  GroupDesc grp[GDPA_MAX_GROUPS];
  int32_t n_groups;
  int32_t n_seqs_total;
  int32_t n_items;
  int32_t work_shift;  // bucket = min(kNumBuckets-1, work >> work_shift)
  int32_t* items;      // [n_items] packed (group, head, seq): longest first within each class (other
                       // groups, then short-key groups)
  int32_t* scratch;    // builder scratch: [n_seqs_total] bucket keys + [2*kNumBuckets] counters
  int32_t* err;        // device error word (GDPA_DEVICE_ERR_* bits) in the workspace
  int32_t check_err;   // validation ran first: kernels return at once if the word is non-zero
  int32_t plan_sig;    // signature of the work list these problems give (item count, short-key split)
  int32_t check_plan;  // planned call: kernels compare the list's signature (err[1]) with plan_sig
};
// passed by value as the kernels' argument (the argument block holds at most 4 KB)
static_assert(sizeof(LaunchDesc) <= 4096, "kernel argument size");

// Debug validation found bad offsets, or a planned call's work list was built for other problems:
// the main kernels leave every output untouched (the second case reports GDPA_DEVICE_ERR_PLAN).
__device__ inline bool launch_refused(const LaunchDesc& d) {
  if (d.check_err && *d.err != 0) return true;
  if (d.check_plan && d.err[1] != d.plan_sig) {
    if (threadIdx.x == 0) atomicOr(d.err, GDPA_DEVICE_ERR_PLAN);
    return true;
  }
  return false;
}

// The item's own offsets, checked before any tensor access: row ranges inside their tensors,
// lengths within what the launch provisioned (kv_cap keys, or any if kv_cap < 0; a shared query
// matrix has shared_q rows), equal lengths under a window. Returns GDPA_DEVICE_ERR_* bits.
__device__ inline int32_t item_error(const GroupDesc& gd, int q0, int q1, int k0, int k1, int kv_cap) {
  int32_t e = 0;
  if (q0 < 0 || q1 < q0 || q1 > gd.total_q || k0 < 0 || k1 < k0 || k1 > gd.total_kv) return GDPA_DEVICE_ERR_OFFSETS;
  if ((kv_cap >= 0 && k1 - k0 > kv_cap) || (gd.shared_q && q1 - q0 > gd.shared_q)) e |= GDPA_DEVICE_ERR_LENGTH;
  if ((gd.wl >= 0 || gd.wr >= 0) && q1 - q0 != k1 - k0) e |= GDPA_DEVICE_ERR_SELF;
  return e;
}

// Record error bits from one lane of the item (the item then writes nothing).
__device__ inline void report_error(const LaunchDesc& d, int32_t e) { atomicOr(d.err, e); }

// Copy of group g's descriptor (g is uniform across the workgroup). A chain of uniform selects
// instead of a dynamic index into the kernel-argument table keeps the table out of scratch.
__device__ inline GroupDesc select_group(const LaunchDesc& d, int g) {
  GroupDesc gd = d.grp[0];
#pragma unroll
  for (int i = 1; i < GDPA_MAX_GROUPS; ++i)
    if (i == g) gd = d.grp[i];
  return gd;
}

// List position of the item that workgroup x of a launch over n items takes. The dispatcher hands
// consecutive workgroups to the 8 XCDs in turn, and each XCD has an L2 of its own; the heads of one
// sequence are consecutive in the list and share the cache lines of the row-interleaved [T, H]
// float arrays (gate, lse, dG: H heads' 4-byte entries of a row side by side). So each run of 8
// consecutive list items goes to one XCD: in round r = k / 8, the k-th workgroup of XCD c takes
// item 64 r + 8 c' + k % 8 with c' = c in even rounds and 7 - c in odd ones. The list order is kept
// at the granularity of 64 items, and the alternation cancels the skew that a fixed order would give
// (in a longest-first list XCD 0 would take the longest run of every round); a ragged tail keeps its
// positions.
constexpr int kXcds = 8;
__device__ inline int xcd_item(int x, int n) {
  const int full = n & ~(kXcds * kXcds - 1);
  if (x >= full) return x;
  const int c = x % kXcds, k = x / kXcds, r = k / kXcds;
  const int cs = (r & 1) ? kXcds - 1 - c : c;
  return r * (kXcds * kXcds) + cs * kXcds + k % kXcds;
}

// Packed work item: group (5 bits) | head (8 bits) | sequence (19 bits).
__host__ __device__ inline int32_t pack_item(int g, int h, int b) {
  return (int32_t)(((uint32_t)g << 27) | ((uint32_t)h << 19) | (uint32_t)b);
}
__device__ inline void unpack_item(int32_t it, int& g, int& h, int& b) {
  uint32_t u = (uint32_t)it;
  g = (int)(u >> 27);
  h = (int)((u >> 19) & 0xFF);
  b = (int)(u & 0x7FFFF);
}

// ----------------------------------------------------------------------------------------------
// MFMA conventions (v_mfma_f32_32x32x16_bf16, one wave):
//   A (32 x 16, M x K): lane l holds row l%32, k-slots (l/32)*8 + e, e = 0..7
//   B (16 x 32, K x N): lane l holds column l%32, k-slots (l/32)*8 + e
//   C (32 x 32):        lane l holds column l%32, register r holds row (r/4)*8 + (l/32)*4 + r%4
// Any bijection between k-slots and the true contraction index works if A and B use the same
// one; the kernels choose bijections that make every operand a contiguous 16-byte read.
// ----------------------------------------------------------------------------------------------
__device__ inline f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: A (16 x 32): lane l holds row l%16, k-slots (l/16)*8 + e;
// B (32 x 16): lane l holds column l%16, k-slots (l/16)*8 + e; C (16 x 16): lane l holds column
// l%16, register r holds row (l/16)*4 + r.
__device__ inline f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes, lane j supplies the
// address of 4 consecutive 16-bit values, forming row j of a 16 x 4 matrix M; lane i receives
// M[(i >> 2) + 4e][i & 3] for e = 0..3. Choosing row j = (4 consecutive columns starting at
// c0 + 4 (j & 3)) of line l0 + (j >> 2) therefore gives lane i the 4 values of column c0 + i on
// lines l0 .. l0+3: a column read out of a row-major tile.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ inline u32x2 lds_read_tr16(const char* lds, int byte_offset) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds + byte_offset));
  return __builtin_bit_cast(u32x2, v);
}

// C-register -> row mapping of a 32x32 MFMA result, for lane half g = lane/32.
__device__ __host__ inline constexpr int c_row(int r, int g) { return (r / 4) * 8 + g * 4 + (r % 4); }

// Allowed entries of one lane in a 32x32 pair as a range of the index its registers run over
// (rows for a lane holding a key, keys for a lane holding a row): register r, at index
// first + c_row(r, g), is allowed iff (unsigned)(base + c_row(r, g)) <= span. lo..hi: the lane's
// allowed range of that index (empty when hi < lo).
struct LaneRange {
  int base;
  unsigned span;
};
__device__ inline LaneRange lane_range(int first, int lo, int hi) {
  LaneRange m;
  const bool empty = hi < lo;
  m.base = empty ? -(1 << 30) : first - lo;
  m.span = empty ? 0u : (unsigned)(hi - lo);
  return m;
}
__device__ inline bool lane_ok(const LaneRange& m, int r, int g) {
  return (unsigned)(m.base + c_row(r, g)) <= m.span;
}

// When a C tile (rows = a contraction index of the next product) is fed back as a B operand,
// B k-tile t (16 slots) takes C registers 8t..8t+7. Slot s = g*8+e of k-tile t then carries
// row c_row(8t+e, g) = 16t + slot_row(s). slot_row is an involution on 0..15 that swaps the two
// middle quads: [0..3, 8..11, 4..7, 12..15].
__device__ __host__ inline constexpr int slot_row(int s) {
  return ((s & 7) >> 2) * 8 + (s >> 3) * 4 + (s & 3);
}

// Output-row permutation of a C tile whose A operand rows are chosen so that each lane ends up
// holding 16 consecutive output columns: C row m of d-tile dt carries output index
// dt*32 + out_perm(m), so register r of lane half g is output index dt*32 + g*16 + r.
__device__ __host__ inline constexpr int out_perm(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }

// ----------------------------------------------------------------------------------------------
// bf16 helpers (round to nearest even; gfx950 has a packed convert instruction)
// ----------------------------------------------------------------------------------------------
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// One v_cvt_pk_bf16_f32 (round to nearest even) for two values; a is the low half.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ inline float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

__device__ inline bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

// An output tensor of a bf16 problem: bf16 elements, or float32 ones when the caller asked for
// float32 outputs. Offsets count elements; stores take fp32 values and round them only for bf16.
struct OutPtr {
  char* p;
  int32_t f32;
  __device__ inline OutPtr operator+(size_t e) const { return OutPtr{p + (e << (f32 ? 2 : 1)), f32}; }
};
__device__ inline OutPtr out_ptr(void* base, int32_t f32, size_t e) { return OutPtr{static_cast<char*>(base), f32} + e; }
// 8 consecutive elements a[0..3], b[0..3] (16-byte aligned for bf16, 32-byte for float32)
__device__ inline void out_store8(OutPtr o, const f32x4& a, const f32x4& b) {
  if (o.f32) {
    reinterpret_cast<f32x4*>(o.p)[0] = a;
    reinterpret_cast<f32x4*>(o.p)[1] = b;
  } else {
    *reinterpret_cast<u32x4*>(o.p) = u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                           pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
  }
}
// 4 consecutive elements
__device__ inline void out_store4(OutPtr o, const f32x4& a) {
  if (o.f32) *reinterpret_cast<f32x4*>(o.p) = a;
  else *reinterpret_cast<u32x2*>(o.p) = u32x2{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
}
// 16 consecutive elements: a C tile's registers 0..15 of one lane, times s
__device__ inline void out_store16(OutPtr o, const f32x16& c, float s) {
  out_store8(o, f32x4{c[0], c[1], c[2], c[3]} * s, f32x4{c[4], c[5], c[6], c[7]} * s);
  out_store8(o + 8, f32x4{c[8], c[9], c[10], c[11]} * s, f32x4{c[12], c[13], c[14], c[15]} * s);
}
__device__ inline void out_zero8(OutPtr o) {
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  out_store8(o, z, z);
}

// ----------------------------------------------------------------------------------------------
// Activations in fp32 registers.
//   The bf16 kernels round P to bf16 right after, so the activations use short forms whose
//   error is far below a bf16 ulp:
//   - SiLU: x * rcp(1 + 2^(-x log2 e)) with the hardware exp2 / reciprocal.
//   - GELU: x * Phi(x) with Phi(x) ~ sigmoid(1.5976 x + 0.07056 x^3), the logistic
//     approximation of the normal CDF of Bowling, Khasawneh, Kaewkuekool and Cho (2009,
//     J. Industrial Eng. & Management), |error| < 1.5e-4 on Phi.
//   The fp32 kernels use the exact erf form (erff of the device math library).
// ----------------------------------------------------------------------------------------------
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// sigmoid(z) given t = -z*log2(e)
__device__ inline float sigmoid_from_t(float t) { return fast_rcp(1.0f + fast_exp2(t)); }

// Both element-wise activations are x * g(x) with g(x) = sigmoid(a1 x + a3 x^3):
//   SiLU: a1 = 1, a3 = 0 (exact);  GELU: a1 = 1.5976, a3 = 0.07056 (Phi approximation above).
// The kernels evaluate g through t = -log2(e) (a1 x + a3 x^3) = x (c1 + c3 x^2), so that with the
// score scale folded into c1, c3 a raw accumulator s gives phi(scale s) / scale = s g(scale s).
template <int ACT>
struct PointAct {
  static constexpr float a1 = ACT == GDPA_ACT_GELU ? 1.5976f : 1.0f;
  static constexpr float a3 = ACT == GDPA_ACT_GELU ? 0.07056f : 0.0f;
  // coefficients of t for an argument that is `scale` times the variable passed in
  __device__ static inline void coeffs(float scale, float& c1, float& c3) {
    c1 = -kLog2e * a1 * scale;
    c3 = -kLog2e * a3 * scale * scale * scale;
  }
  __device__ static inline float t_of(float x, float c1, float c3) {
    if constexpr (ACT == GDPA_ACT_SILU) return x * c1;
    else return x * __builtin_fmaf(x * x, c3, c1);
  }
  // x * g(x') where x' = scale * x is encoded in c1, c3
  __device__ static inline float value(float x, float c1, float c3) {
    return x * fast_rcp(1.0f + fast_exp2(t_of(x, c1, c3)));
  }
  // value p = x g and derivative phi'(x') = g + x' g (1 - g)(a1 + 3 a3 x'^2), for x' = scale x.
  // 1 - g is formed from g, not as e g: where the argument is far below zero, 2^t overflows to
  // +inf and g to 0, and e g would be inf * 0.  Its absolute error (half an ulp of 1) stays far
  // below the bf16 rounding of the result wherever x' (1 - g) is not negligible.
  __device__ static inline void value_grad(float x, float scale, float c1, float c3, float& p, float& dphi) {
    const float e = fast_exp2(t_of(x, c1, c3));
    const float g = fast_rcp(1.0f + e);
    p = x * g;
    const float somg = __builtin_fmaf(g, -scale, scale);  // scale (1 - g)
    if constexpr (ACT == GDPA_ACT_SILU) {
      dphi = __builtin_fmaf(p, somg, g);
    } else {
      const float xs = x * scale;
      const float k = __builtin_fmaf(xs * xs, 3.0f * a3, a1);
      dphi = __builtin_fmaf(p * somg, k, g);
    }
  }
};

// Small-argument series of the same activations, exact forms (no logistic approximation): for
// |x| <= kSeriesBound
//   phi(x)  = x (1/2 + x (A + B x^2))      SiLU: Taylor series of x sigmoid(x) (A = 1/4, B = -1/48)
//   phi'(x) = 1/2 + x (C + D x^2)          GELU: Taylor series of x Phi(x), Phi the normal CDF
//                                                (A = phi0, B = -phi0/6, C = 2 phi0, D = -2 phi0/3,
//                                                phi0 = 1/sqrt(2 pi))
// The first omitted terms (x^6 / 480 and x^5 / 80 for SiLU, phi0 x^6 / 40 and 3 phi0 x^5 / 20 for
// GELU) leave relative errors of at most 5e-6 (SiLU), 3e-5 (SiLU'), 2.5e-5 (GELU) and 1.9e-4
// (GELU', at x = -1/4) over |x| <= 1/4: a tenth of the bf16 rounding of P and dS (2^-9) or less,
// and of the order of the exact path's own GELU approximation (1.5e-4 in Phi). The kernels take this path for a tile only where a bound proves every argument of the
// tile within the range (seq_series_ok); other tiles use PointAct. Four and two plain
// multiply-adds replace the two transcendentals (a quarter-rate exp2 and reciprocal) and the
// arithmetic around them.
constexpr float kSeriesBound = 0.25f;
template <int ACT>
struct SeriesAct {
  static constexpr float kPhi0 = 0.3989422804014327f;
  static constexpr float A = ACT == GDPA_ACT_GELU ? kPhi0 : 0.25f;
  static constexpr float B = ACT == GDPA_ACT_GELU ? -kPhi0 / 6.0f : -1.0f / 48.0f;
  static constexpr float C = ACT == GDPA_ACT_GELU ? 2.0f * kPhi0 : 0.5f;
  static constexpr float D = ACT == GDPA_ACT_GELU ? -2.0f * kPhi0 / 3.0f : -1.0f / 12.0f;
  // coefficients for a raw score s with argument x = scale s, in the convention of PointAct for
  // ungated scores: value p' = phi(x) / scale = s (1/2 + s (a1 + a3 s^2)); derivative
  // phi'(x) = 1/2 + s (d1 + d3 s^2)
  __host__ __device__ static inline void coeffs(float scale, float& a1, float& a3, float& d1, float& d3) {
    const float s3 = scale * scale * scale;
    a1 = A * scale;
    a3 = B * s3;
    d1 = C * scale;
    d3 = D * s3;
  }
  __host__ __device__ static inline float value(float s, float a1, float a3) {
    const float w = s * s;
    const float c = __builtin_fmaf(s, __builtin_fmaf(w, a3, a1), 0.5f);
    return s * c;
  }
  __host__ __device__ static inline void value_grad(float s, float a1, float a3, float d1, float d3, float& p,
                                                    float& dphi) {
    const float w = s * s;
    p = s * __builtin_fmaf(s, __builtin_fmaf(w, a3, a1), 0.5f);
    dphi = __builtin_fmaf(s, __builtin_fmaf(w, d3, d1), 0.5f);
  }
  // One term fewer, for tiles proven within the smaller ranges below: phi(x) = x (1/2 + A x),
  // phi'(x) = 1/2 + C x (two and one multiply-adds).
  __host__ __device__ static inline float value_short(float s, float a1) { return s * __builtin_fmaf(s, a1, 0.5f); }
  __host__ __device__ static inline void value_grad_short(float s, float a1, float d1, float& p, float& dphi) {
    p = s * __builtin_fmaf(s, a1, 0.5f);
    dphi = __builtin_fmaf(s, d1, 0.5f);
  }
};

// Ranges of the shorter series. The omitted terms B x^4 and D x^3 leave relative errors of about
// 2 |B| x^3 (phi) and 2 |D| x^3 (phi'): x^3 / 24 and x^3 / 6 for SiLU, phi0 x^3 / 3 and
// 4 phi0 x^3 / 3 for GELU. The forward needs phi only: over |x| <= 0.16 (SiLU) and 0.11 (GELU)
// its error is at most 1.9e-4; the backward needs both: over |x| <= 0.1 (SiLU) and 0.07 (GELU)
// phi' is off by at most 1.9e-4 (SiLU) and 2.1e-4 (GELU), and phi by 5e-5. That is about a tenth
// of the bf16 rounding of P and dS (2^-9), the level of the longer series' own error.
template <int ACT>
__host__ __device__ constexpr float series_short_bound_fwd() { return ACT == GDPA_ACT_GELU ? 0.11f : 0.16f; }
template <int ACT>
__host__ __device__ constexpr float series_short_bound_bwd() { return ACT == GDPA_ACT_GELU ? 0.07f : 0.1f; }

// Every argument x = scale <q, k> of a tile lies in the series range when
// scale^2 max ||q||^2 max ||k||^2 <= kSeriesBound^2 (Cauchy-Schwarz), with a margin for the fp32
// accumulation of the scores and of the squared norms. False for NaN or infinite norms.
__host__ __device__ inline bool seq_series_within(float scale, float qn2, float kn2, float bound) {
  return scale * scale * qn2 * kn2 <= bound * bound * 0.998f;
}
__host__ __device__ inline bool seq_series_ok(float scale, float qn2, float kn2) {
  return seq_series_within(scale, qn2, kn2, kSeriesBound);
}

// Sum of squares of the 8 bf16 values of a 16-byte chunk (each product is exact in fp32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline float sumsq_bf16x8(const u32x4& u) {
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2_t v = __builtin_bit_cast(bf16x2_t, u[e]);
    acc = __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
  }
  return acc;
}

// Maximum over the lanes of a wave (lanes whose value is not needed must hold something <= it).
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Lane exchanges inside rows of 16 lanes through DPP operand modifiers: a VALU instruction reads
// the other lane's register directly, with no LDS round trip (each ds_bpermute shuffle of a chain
// waits for the LDS). Call with every lane active.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]: lane i ^ 1
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]: lane i ^ 2
constexpr int kDppHalfMirror = 0x141; // lane 7 - i inside each group of 8
constexpr int kDppMirror = 0x140;     // lane 15 - i inside each row of 16
template <int CTRL>
__device__ inline float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of N consecutive lanes (N = 1, 2, 4, 8 or 16), on every lane of the
// group. Each step adds the partner's partial sum: after the first two steps every lane of a quad
// holds the same quad sum, so the mirrored lane of the other quad (or half-row) carries the value
// that lane i ^ 4 (i ^ 8) would: the result is that of the xor butterfly.
template <int N>
__device__ inline float group_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
  if constexpr (N >= 2) v += dpp_mov<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp_mov<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp_mov<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_mov<kDppMirror>(v);
  return v;
}

// This lane's value combined with lane l ^ 32's (or l ^ 16's) by a commutative operation, with one
// VALU lane swap instead of an LDS round trip: v_permlane32_swap (v_permlane16_swap) of a register
// with itself returns two registers that hold, on every lane, its own value and its partner's (in
// an order that depends on the half), so the sum or the maximum of the two needs no lane select and
// equals that of the shuffle exactly. Call with every lane active.
__device__ inline float half32_sum(float v) {
  const int x = __builtin_bit_cast(int, v);
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}
__device__ inline float half32_max(float v) {
  const int x = __builtin_bit_cast(int, v);
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ inline float half16_max(float v) {
  const int x = __builtin_bit_cast(int, v);
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}

// Maximum over each row of 16 lanes, on every lane of the row (the wave's maximum is then the
// largest of lanes 0, 16, 32 and 48).
__device__ inline float row16_max(float v) {
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  return fmaxf(v, dpp_mov<kDppMirror>(v));
}

// Maximum over the lanes of a wave, the same on every lane, without LDS or scalar registers: rows of
// 16 lanes by DPP, then across rows by the two lane swaps (the same value as wave_max).
__device__ inline float wave_max_lanes(float v) { return half32_max(half16_max(row16_max(v))); }

// log sigmoid(g) in fp32, overflow-free: min(g, 0) - log1p(exp(-|g|)).
__device__ inline float log_sigmoid_f(float g) {
  return fminf(g, 0.0f) - log1pf(__expf(-fabsf(g)));
}

__device__ inline int lane_id() { return (int)(threadIdx.x & 63); }
// The wave index is the same on every lane; readfirstlane puts it (and everything derived from
// it) in scalar registers, so tests on it become scalar branches instead of exec-masked ones.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

}  // namespace gdpa
