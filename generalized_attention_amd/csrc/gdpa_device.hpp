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
};

struct LaunchDesc {
  GroupDesc grp[GDPA_MAX_GROUPS];
  int32_t n_groups;
  int32_t n_seqs_total;
  int32_t n_items;
  int32_t work_shift;  // bucket = min(kNumBuckets-1, work >> work_shift)
  int32_t* items;      // [n_items] packed (group, head, seq) in longest-first order
  int32_t* scratch;    // builder scratch: [n_seqs_total] bucket keys + [2*kNumBuckets] counters
};
// passed by value as the kernels' argument (the argument block holds at most 4 KB)
static_assert(sizeof(LaunchDesc) <= 4096, "kernel argument size");

// Copy of group g's descriptor (g is uniform across the workgroup). A chain of uniform selects
// instead of a dynamic index into the kernel-argument table keeps the table out of scratch.
__device__ inline GroupDesc select_group(const LaunchDesc& d, int g) {
  GroupDesc gd = d.grp[0];
#pragma unroll
  for (int i = 1; i < GDPA_MAX_GROUPS; ++i)
    if (i == g) gd = d.grp[i];
  return gd;
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

// log sigmoid(g) in fp32, overflow-free: min(g, 0) - log1p(exp(-|g|)).
__device__ inline float log_sigmoid_f(float g) {
  return fminf(g, 0.0f) - log1pf(__expf(-fabsf(g)));
}

__device__ inline int lane_id() { return (int)(threadIdx.x & 63); }
// The wave index is the same on every lane; readfirstlane puts it (and everything derived from
// it) in scalar registers, so tests on it become scalar branches instead of exec-masked ones.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

}  // namespace gdpa
