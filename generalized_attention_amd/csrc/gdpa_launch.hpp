// Host-side launch entry points of the kernels (internal to libgdpa).
#pragma once

#include <hip/hip_runtime.h>

#include "gdpa_device.hpp"

namespace gdpa {

// Which head dims a launch contains (bit 0: 32, bit 1: 64, bit 2: 128).
enum DimSet { kDim32 = 1, kDim64 = 2, kDim128 = 4 };

hipError_t launch_schedule(const LaunchDesc& d, hipStream_t stream);
// Offsets validation into the device error word (debug), and a plain clear of the word.
hipError_t launch_validate(const LaunchDesc& d, hipStream_t stream);
hipError_t launch_clear_error(int32_t* err, hipStream_t stream);
// act_set: bit (1 << act) for every activation present in the launch.
// key_mode: 1 = d <= 64 and every key range fits the forward's LDS (16384 / d keys); 2 = d <= 64,
// no window and some key range longer than that; 0 = any.
hipError_t launch_fwd_bf16(const LaunchDesc& d, int dim_set, int act_set, int key_mode, hipStream_t stream);
// small: every problem has at most 32 keys per sequence, an element-wise activation and no window
// (one wave per work item). softmax_form: which kernel a softmax launch at d <= 64 takes (4 waves
// and every sweep, or the 8-wave kernels of kBwdWideSoftmax / kBwdRingSoftmax).
enum BwdSoftmaxForm { kSoftmaxAnySweep = 0, kSoftmaxNoWindow = 1, kSoftmaxRingWindow = 2 };
hipError_t launch_bwd_bf16(const LaunchDesc& d, int dim_set, int act_set, bool small, BwdSoftmaxForm softmax_form,
                           hipStream_t stream);
// fp32 kernels are flat over (row, head) / (key, head); prefix tables over groups.
struct Fp32Aux {
  int64_t row_pre[GDPA_MAX_GROUPS + 1];   // prefix of total_q * H
  int64_t key_pre[GDPA_MAX_GROUPS + 1];   // prefix of total_kv * H
  int64_t row_base[GDPA_MAX_GROUPS];      // offset of each group's rows*heads in ws_delta
  float* ws_delta;                        // softmax backward: D_i per (row, head)
};
hipError_t launch_fwd_fp32(const LaunchDesc& d, const Fp32Aux& aux, hipStream_t stream);
hipError_t launch_bwd_fp32(const LaunchDesc& d, const Fp32Aux& aux, hipStream_t stream);

// Keys of one (sequence, head) whose K and V^T fit in the forward kernel's LDS at once.
inline constexpr int fwd_kv_capacity(int d) { return 16384 / d; }
// Backward: a workgroup holds 256 keys (128 at d = 128) for the whole sweep over query tiles of
// 64 rows: 4 waves owning 64 keys each (32 at d = 128), or, in launches without d = 128 and
// without the softmax form (or with it and one of the two flags below in the activation set),
// 8 waves (two per SIMD) owning 32 keys each.
constexpr int kBwdWaves = 4;
// Activation-set flags of the 8-wave softmax launches at d <= 64. Each compiles only the sweeps
// its items can take (a sweep compiled into the kernel but never run still costs registers in
// all of it): no window in the launch (resident keys or key chunks), or every group's window
// streaming its keys through the ring (bwd_ring_ok).
constexpr int kBwdWideSoftmax = 1 << 3;
constexpr int kBwdRingSoftmax = 1 << 4;
template <int DSET, int ASET>
constexpr int bwd_waves() {
  return ((DSET & kDim128) ||
          ((ASET & (1 << GDPA_ACT_SOFTMAX)) && !(ASET & (kBwdWideSoftmax | kBwdRingSoftmax)))) ? 4 : 8;
}
constexpr int kBwdKeyBlock = 32;
// A sum of at most this many products (dK / dV of an item with that few query rows, O / dQ of one
// with that few keys) takes its P / dS operands as two bf16 terms, high part and rounding
// remainder: with few terms a product can be many times the output's RMS, and a single bf16
// rounding of its operand (2^-9 relative) would then exceed 2e-2 of that RMS.
constexpr int kSplitTerms = 16;
constexpr int kBwdQueryTile = 64;
inline constexpr int bwd_keys_per_wave(int d) { return d == 128 ? 32 : 64; }
inline constexpr int bwd_capacity(int d) { return kBwdWaves * bwd_keys_per_wave(d); }
// A bounded window whose key span for one query tile fits in the ring of resident blocks with one
// block to spare (misalignment): keys stream through the ring as the tiles advance.
inline __host__ __device__ bool bwd_ring_ok(int d, int wl, int wr) {
  return wl >= 0 && wr >= 0 && kBwdQueryTile - 1 + wl + wr <= bwd_capacity(d) - kBwdKeyBlock;
}
// Otherwise a sequence with more keys than are resident is processed in key chunks, one after the
// other, with dQ (and the softmax row term) accumulated in fp32 workspace rows. The ring path has
// no split-operand form: with split operands everywhere, long windowed items run in key chunks.
inline __host__ __device__ bool bwd_needs_chunks(int d, int wl, int wr, int n, bool split_all) {
  return n > bwd_capacity(d) && (!bwd_ring_ok(d, wl, wr) || split_all);
}
inline bool bwd_may_chunk(int d, int wl, int wr, int max_kv, bool split_all) {
  return bwd_needs_chunks(d, wl, wr, max_kv, split_all);
}

// Shared-query groups: sum the per-sequence fp32 dQ rows into dq (bf16); nothing when the
// launch was refused (d.check_err and a non-zero error word).
hipError_t launch_reduce_shared_dq(const LaunchDesc& d, const GroupDesc& gd, hipStream_t stream);

}  // namespace gdpa
