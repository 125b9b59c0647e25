// C ABI of libgdpa: host-side argument validation, workspace layout and kernel launches.
// Every check here runs before the first HIP call of a request, so an invalid request enqueues
// nothing and can be tested without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gdpa.h"
#include "gdpa_check.hpp"
#include "gdpa_launch.hpp"

namespace gdpa {

// ---- Library-owned scratch for callers that cannot allocate (gdpa_bwd_noalloc) ----------------
//
// One array per GPU, in device memory for as long as the process runs. In host code `scratch` is
// only a stand-in symbol: its device address is looked up once per device and kept in
// scratch_ptr[device]; kernels and copies get that address, never the symbol itself.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static_assert(kScratchBytes == GDPA_NOALLOC_SCRATCH_BYTES, "documented scratch size");
__device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace: a 256-byte header (the device error word at GDPA_WS_ERROR_OFFSET), the work list,
// the builder's per-sequence keys, the softmax row terms and the fp32 dQ rows.
struct WsLayout {
  size_t items = 0, keys = 0, delta = 0, dq32 = 0, total = 0;
  int64_t n_items = 0, n_seqs = 0, delta_rows = 0, dq32_floats = 0;
  int64_t delta_base[GDPA_MAX_GROUPS] = {};
  int64_t dq32_base[GDPA_MAX_GROUPS] = {};
  bool has_delta[GDPA_MAX_GROUPS] = {};  // the group reserved row terms / fp32 dQ rows
  bool has_dq32[GDPA_MAX_GROUPS] = {};
};

bool shared_q(const gdpa_problem& p) { return (p.flags & GDPA_FLAG_SHARED_Q) != 0; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_problem(const gdpa_problem& p) {
  if (p.num_seqs < 0 || p.num_seqs >= (1 << 19)) return GDPA_ERR_INVALID_ARGUMENT;
  if (p.num_heads < 1 || p.num_heads > 256) return GDPA_ERR_INVALID_ARGUMENT;
  if (p.head_dim != 32 && p.head_dim != 64 && p.head_dim != 128) return GDPA_ERR_UNSUPPORTED;
  if (p.dtype != GDPA_DTYPE_BF16 && p.dtype != GDPA_DTYPE_FP32) return GDPA_ERR_INVALID_ARGUMENT;
  if (p.act < GDPA_ACT_GELU || p.act > GDPA_ACT_SOFTMAX) return GDPA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(p.scale)) return GDPA_ERR_INVALID_ARGUMENT;
  if (p.window_left < -1 || p.window_right < -1) return GDPA_ERR_INVALID_ARGUMENT;
  if ((p.flags & ~(GDPA_FLAG_PLANNED | GDPA_FLAG_SHARED_Q | GDPA_FLAG_FP32_OUT | GDPA_FLAG_VALIDATE |
                   GDPA_FLAG_SPLIT_OPERANDS)) != 0)
    return GDPA_ERR_INVALID_ARGUMENT;
  if (shared_q(p) && p.self_attention) return GDPA_ERR_INVALID_ARGUMENT;
  if (shared_q(p) && p.dtype != GDPA_DTYPE_BF16) return GDPA_ERR_UNSUPPORTED;
  if (p.self_attention != 0 && p.self_attention != 1) return GDPA_ERR_INVALID_ARGUMENT;
  if (p.total_q < 0 || p.total_kv < 0 || p.max_seqlen_q < 0 || p.max_seqlen_kv < 0)
    return GDPA_ERR_INVALID_ARGUMENT;
  if (p.total_q >= (int64_t)1 << 31 || p.total_kv >= (int64_t)1 << 31) return GDPA_ERR_UNSUPPORTED;
  const bool windowed = p.window_left >= 0 || p.window_right >= 0;
  if (windowed && !p.self_attention) return GDPA_ERR_INVALID_ARGUMENT;
  if (p.self_attention && (p.total_q != p.total_kv || p.max_seqlen_q != p.max_seqlen_kv))
    return GDPA_ERR_INVALID_ARGUMENT;
  if (p.num_seqs > 0 && (!p.q_offsets || !p.kv_offsets)) return GDPA_ERR_INVALID_ARGUMENT;
  if (p.num_seqs == 0 && (p.total_q != 0 || p.total_kv != 0)) return GDPA_ERR_INVALID_ARGUMENT;
  // (a shared query matrix has max_seqlen_q rows of its own, whatever the sequences use)
  if ((!shared_q(p) && (int64_t)p.max_seqlen_q > p.total_q) || (int64_t)p.max_seqlen_kv > p.total_kv)
    return GDPA_ERR_INVALID_ARGUMENT;
  return GDPA_OK;
}

// bf16 backward in key chunks (long key ranges, or a shared query matrix): fp32 dQ rows and, for
// softmax, the row term D_i live in the workspace.
bool bwd_chunked(const gdpa_problem& p) {
  return p.dtype == GDPA_DTYPE_BF16 &&
         (shared_q(p) || bwd_may_chunk(p.head_dim, p.window_left, p.window_right, p.max_seqlen_kv,
                                       (p.flags & GDPA_FLAG_SPLIT_OPERANDS) != 0));
}

// The problem may contain softmax heads (its own act, or any head when the activation is per head).
bool may_softmax(const gdpa_problem& p) { return p.act == GDPA_ACT_SOFTMAX || p.head_acts != nullptr; }

int check_tensors(const gdpa_problem& p, const gdpa_tensors& t, int pass) {
  const bool rows = p.total_q > 0, keys = p.total_kv > 0;
  const bool qrows = shared_q(p) ? p.max_seqlen_q > 0 : rows;  // rows of q and dq
  if (qrows && (!t.q || !aligned16(t.q))) return GDPA_ERR_INVALID_ARGUMENT;
  if (keys && (!t.k || !t.v || !aligned16(t.k) || !aligned16(t.v))) return GDPA_ERR_INVALID_ARGUMENT;
  if (t.dg && !t.g) return GDPA_ERR_INVALID_ARGUMENT;
  if ((t.g && !aligned16(t.g)) || (t.lse && ((uintptr_t)t.lse & 3u))) return GDPA_ERR_INVALID_ARGUMENT;
  if (pass == 0) {
    if (rows && (!t.o || !aligned16(t.o))) return GDPA_ERR_INVALID_ARGUMENT;
    if (rows && may_softmax(p) && !t.lse) return GDPA_ERR_INVALID_ARGUMENT;
    if (t.dg) return GDPA_ERR_INVALID_ARGUMENT;
  } else {
    if (rows && (!t.dout || !aligned16(t.dout))) return GDPA_ERR_INVALID_ARGUMENT;
    if (qrows && (!t.dq || !aligned16(t.dq))) return GDPA_ERR_INVALID_ARGUMENT;
    if (keys && (!t.dk || !t.dv || !aligned16(t.dk) || !aligned16(t.dv))) return GDPA_ERR_INVALID_ARGUMENT;
    if (rows && may_softmax(p) && !t.lse) return GDPA_ERR_INVALID_ARGUMENT;
  }
  return GDPA_OK;
}

int layout(const gdpa_problem* ps, int n_groups, int pass, WsLayout* L) {
  if (!ps || n_groups < 1 || n_groups > GDPA_MAX_GROUPS) return GDPA_ERR_INVALID_ARGUMENT;
  if (pass != 0 && pass != 1) return GDPA_ERR_INVALID_ARGUMENT;
  for (int g = 0; g < n_groups; ++g) {
    int rc = check_problem(ps[g]);
    if (rc != GDPA_OK) return rc;
    if (ps[g].dtype != ps[0].dtype || (ps[g].flags & GDPA_FLAG_PLANNED) != (ps[0].flags & GDPA_FLAG_PLANNED))
      return GDPA_ERR_INVALID_ARGUMENT;
    L->n_items += (int64_t)ps[g].num_seqs * ps[g].num_heads;
    L->n_seqs += ps[g].num_seqs;
    L->delta_base[g] = L->delta_rows;
    // softmax backward: per-row D_i (fp32: between its two kernels; bf16: across key chunks)
    if (pass == 1 && may_softmax(ps[g]) && (ps[g].dtype == GDPA_DTYPE_FP32 || bwd_chunked(ps[g]))) {
      L->delta_rows += ps[g].total_q * ps[g].num_heads;
      L->has_delta[g] = true;
    }
    L->dq32_base[g] = L->dq32_floats;
    if (pass == 1 && bwd_chunked(ps[g])) {
      const int64_t rows = shared_q(ps[g]) ? (int64_t)ps[g].num_seqs * ps[g].max_seqlen_q : ps[g].total_q;
      L->dq32_floats += rows * ps[g].num_heads * ps[g].head_dim;
      L->has_dq32[g] = true;
    }
  }
  if (L->n_items >= ((int64_t)1 << 31) || L->n_seqs >= ((int64_t)1 << 31)) return GDPA_ERR_UNSUPPORTED;
  L->items = kAlign;  // after the header
  L->keys = L->items + align_up((size_t)L->n_items * 4);
  L->delta = L->keys + align_up((size_t)L->n_seqs * 4);
  L->dq32 = L->delta + align_up((size_t)L->delta_rows * 4);
  L->total = L->dq32 + align_up((size_t)L->dq32_floats * 4);
  return GDPA_OK;
}

int bit_length(uint64_t x) {
  int n = 0;
  while (x) { ++n; x >>= 1; }
  return n;
}

// The backward runs a group's items one wave each (bwd_small_kernel) when every sequence has at
// most 32 keys and the form is element-wise, without a window or a shared query matrix.
bool short_key_group(const gdpa_problem& p) {
  return p.dtype == GDPA_DTYPE_BF16 && p.max_seqlen_kv <= 32 && p.act != GDPA_ACT_SOFTMAX && !p.head_acts &&
         p.window_left < 0 && p.window_right < 0 && !shared_q(p);
}

void fill_desc(const gdpa_problem* ps, const gdpa_tensors* ts, int n_groups, void* ws, const WsLayout& L,
               LaunchDesc* d) {
  std::memset(d, 0, sizeof(*d));
  d->n_groups = n_groups;
  d->n_items = (int32_t)L.n_items;
  d->n_seqs_total = (int32_t)L.n_seqs;
  char* base = static_cast<char*>(ws);
  d->items = reinterpret_cast<int32_t*>(base + L.items);
  d->scratch = reinterpret_cast<int32_t*>(base + L.keys);
  d->err = reinterpret_cast<int32_t*>(base + GDPA_WS_ERROR_OFFSET);
  d->check_err = 0;
  // work-list signature: item count and the short-key split (both fixed by the problems alone)
  int64_t n_short = 0;
  for (int g = 0; g < n_groups; ++g)
    if (short_key_group(ps[g])) n_short += (int64_t)ps[g].num_seqs * ps[g].num_heads;
  d->plan_sig = (int32_t)(((uint32_t)L.n_items * 2654435761u) ^ ((uint32_t)n_short * 40503u) ^ 0x5bd1e995u);
  d->check_plan = (ps[0].dtype == GDPA_DTYPE_BF16 && (ps[0].flags & GDPA_FLAG_PLANNED)) ? 1 : 0;
  uint64_t max_work = 1;
  int seq_base = 0;
  for (int g = 0; g < n_groups; ++g) {
    const gdpa_problem& p = ps[g];
    const gdpa_tensors& t = ts[g];
    GroupDesc& gd = d->grp[g];
    gd.q = t.q; gd.k = t.k; gd.v = t.v; gd.g = t.g; gd.o = t.o; gd.lse = t.lse;
    gd.dout = t.dout; gd.dq = t.dq; gd.dk = t.dk; gd.dv = t.dv; gd.dg = t.dg;
    // (null where the group reserved none: the kernels refuse an item that would need them)
    gd.delta = L.has_delta[g] ? reinterpret_cast<float*>(base + L.delta) + L.delta_base[g] : nullptr;
    gd.dq32 = L.has_dq32[g] ? reinterpret_cast<float*>(base + L.dq32) + L.dq32_base[g] : nullptr;
    gd.shared_q = shared_q(p) ? p.max_seqlen_q : 0;
    gd.out_f32 = p.dtype == GDPA_DTYPE_BF16 && (p.flags & GDPA_FLAG_FP32_OUT) ? 1 : 0;
    gd.split_all = (p.flags & GDPA_FLAG_SPLIT_OPERANDS) ? 1 : 0;
    gd.short_keys = short_key_group(p) ? 1 : 0;
    gd.q_off = p.q_offsets;
    gd.kv_off = p.kv_offsets;
    gd.num_seqs = p.num_seqs;
    gd.num_heads = p.num_heads;
    gd.head_dim = p.head_dim;
    gd.act = p.act;
    gd.head_acts = p.head_acts;
    gd.scale = p.scale;
    gd.wl = p.window_left;
    gd.wr = p.window_right;
    gd.total_q = (int32_t)p.total_q;
    gd.total_kv = (int32_t)p.total_kv;
    gd.max_q = p.max_seqlen_q;
    gd.max_kv = p.max_seqlen_kv;
    gd.self_attn = p.self_attention;
    gd.seq_base = seq_base;
    seq_base += p.num_seqs;
    uint64_t n = (uint64_t)p.max_seqlen_kv;
    if (p.window_left >= 0 && p.window_right >= 0) {
      const uint64_t w = (uint64_t)p.window_left + p.window_right + 1;
      n = n < w ? n : w;
    }
    const uint64_t work = ((uint64_t)p.max_seqlen_q + 32) * (n + 32) * (uint64_t)p.head_dim;
    if (work > max_work) max_work = work;
  }
  const int bl = bit_length(max_work);
  d->work_shift = bl > 10 ? bl - 10 : 0;
}

// GDPA_DEBUG=1 in the environment, or GDPA_FLAG_VALIDATE in any problem: validate the offsets first.
bool validate_requested(const gdpa_problem* ps, int n_groups) {
  for (int g = 0; g < n_groups; ++g)
    if (ps[g].flags & GDPA_FLAG_VALIDATE) return true;
  const char* env = std::getenv("GDPA_DEBUG");
  return env != nullptr && env[0] == '1' && env[1] == '\0';
}

int run(const gdpa_problem* ps, const gdpa_tensors* ts, int n_groups, void* ws, size_t ws_bytes, void* stream,
        int pass) {
  WsLayout L;
  int rc = layout(ps, n_groups, pass, &L);
  if (rc != GDPA_OK) return rc;
  if (!ts) return GDPA_ERR_INVALID_ARGUMENT;
  for (int g = 0; g < n_groups; ++g)
    if ((rc = check_tensors(ps[g], ts[g], pass)) != GDPA_OK) return rc;
  if (!ws || ((uintptr_t)ws % kAlign) != 0 || ws_bytes < L.total) return GDPA_ERR_WORKSPACE;
  bool shared_rows = false;  // a shared query matrix still gets its (zero) dq rows
  for (int g = 0; g < n_groups; ++g) shared_rows |= pass == 1 && shared_q(ps[g]) && ps[g].max_seqlen_q > 0;
  if (L.n_items == 0 && !shared_rows) return GDPA_OK;  // nothing to compute

  LaunchDesc d;
  fill_desc(ps, ts, n_groups, ws, L, &d);
  const bool validate = validate_requested(ps, n_groups);
  d.check_err = validate ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (ps[0].dtype == GDPA_DTYPE_FP32) {
    Fp32Aux aux;
    std::memset(&aux, 0, sizeof(aux));
    for (int g = 0; g < n_groups; ++g) {
      aux.row_pre[g + 1] = aux.row_pre[g] + ps[g].total_q * ps[g].num_heads;
      aux.key_pre[g + 1] = aux.key_pre[g] + ps[g].total_kv * ps[g].num_heads;
      aux.row_base[g] = L.delta_base[g];
    }
    aux.ws_delta = reinterpret_cast<float*>(static_cast<char*>(ws) + L.delta);
    // (no work list: the error word is cleared, or set by the validation, by a kernel of its own)
    e = validate ? launch_validate(d, s) : launch_clear_error(d.err, s);
    if (e == hipSuccess) e = pass == 0 ? launch_fwd_fp32(d, aux, s) : launch_bwd_fp32(d, aux, s);
  } else {
    e = (ps[0].flags & GDPA_FLAG_PLANNED) ? hipSuccess : launch_schedule(d, s);  // clears the error word
    if (e == hipSuccess && validate) e = launch_validate(d, s);
    if (e == hipSuccess) {
      // forward mode 1: d <= 64 and every key range resident in LDS; 2: d <= 64, a longer key
      // range and no window (windows keep the 4-wave ring); 0 otherwise. The backward runs the
      // short-key groups' items (the tail of the work list) one wave each in a launch of their
      // own, and every other group's items in the kernel family their head dims and activations
      // select.
      bool any_long = false, any_window = false, any_d128 = false, all_ring = true;
      int dims = 0, acts = 0, dims_short = 0, acts_short = 0;
      int64_t n_short = 0;
      for (int g = 0; g < n_groups; ++g) {
        const gdpa_problem& p = ps[g];
        any_long |= p.max_seqlen_kv > fwd_kv_capacity(p.head_dim);
        any_window |= p.window_left >= 0 || p.window_right >= 0;
        any_d128 |= p.head_dim == 128;
        const int ds = p.head_dim == 32 ? kDim32 : p.head_dim == 64 ? kDim64 : kDim128;
        const int as = p.head_acts ? (1 << GDPA_ACT_GELU) | (1 << GDPA_ACT_SILU) | (1 << GDPA_ACT_SOFTMAX)
                                   : 1 << p.act;
        if (pass == 1 && short_key_group(p)) {
          n_short += (int64_t)p.num_seqs * p.num_heads;
          dims_short |= ds;
          acts_short |= as;
        } else {
          dims |= ds;
          acts |= as;
          all_ring &= bwd_ring_ok(p.head_dim, p.window_left, p.window_right);
        }
      }
      if (pass == 0) {
        const int key_mode = any_d128 ? 0 : !any_long ? 1 : any_window ? 0 : 2;
        e = launch_fwd_bf16(d, dims, acts, key_mode, s);
      } else {
        LaunchDesc main = d;
        main.n_items = d.n_items - (int32_t)n_short;
        // softmax at d <= 64: 8 waves without windows, or with every window in the ring
        const BwdSoftmaxForm form = !any_window ? kSoftmaxNoWindow : all_ring ? kSoftmaxRingWindow : kSoftmaxAnySweep;
        e = launch_bwd_bf16(main, dims, acts, false, form, s);
        if (e == hipSuccess && n_short > 0) {
          LaunchDesc tail = d;
          tail.items = d.items + main.n_items;
          tail.n_items = (int32_t)n_short;
          e = launch_bwd_bf16(tail, dims_short, acts_short, true, kSoftmaxNoWindow, s);
        }
      }
    }
    for (int g = 0; g < n_groups && e == hipSuccess; ++g)
      if (pass == 1 && shared_q(ps[g])) e = launch_reduce_shared_dq(d, d.grp[g], s);
  }
  return e == hipSuccess ? GDPA_OK : GDPA_ERR_HIP;
}

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device (looked up on the first call there).
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace gdpa

extern "C" {

size_t gdpa_workspace_size(const gdpa_problem* problems, int32_t n_groups, int32_t pass) {
  gdpa::WsLayout L;
  if (gdpa::layout(problems, n_groups, pass, &L) != GDPA_OK) return 0;
  return L.total;
}

int gdpa_fwd(const gdpa_problem* problem, const gdpa_tensors* tensors, void* ws, size_t ws_bytes, void* stream) {
  return gdpa::run(problem, tensors, 1, ws, ws_bytes, stream, 0);
}

int gdpa_bwd(const gdpa_problem* problem, const gdpa_tensors* tensors, void* ws, size_t ws_bytes, void* stream) {
  return gdpa::run(problem, tensors, 1, ws, ws_bytes, stream, 1);
}

int gdpa_bwd_noalloc(const gdpa_problem* problem, const gdpa_tensors* tensors, void* stream) {
  gdpa::WsLayout L;
  int rc = gdpa::layout(problem, 1, 1, &L);
  if (rc != GDPA_OK) return rc;
  if (problem->flags & GDPA_FLAG_PLANNED) return GDPA_ERR_INVALID_ARGUMENT;  // the scratch holds no plan of its own
  if (L.total > gdpa::kScratchBytes) return GDPA_ERR_WORKSPACE;
  // every argument check before the first HIP call (the address lookup)
  if (!tensors) return GDPA_ERR_INVALID_ARGUMENT;
  if ((rc = gdpa::check_tensors(*problem, *tensors, 1)) != GDPA_OK) return rc;
  void* ws = nullptr;
  if (gdpa::scratch_on_current_device(&ws) != hipSuccess) return GDPA_ERR_HIP;
  return gdpa::run(problem, tensors, 1, ws, gdpa::kScratchBytes, stream, 1);
}

int gdpa_fwd_grouped(const gdpa_problem* problems, const gdpa_tensors* tensors, int32_t n_groups, void* ws,
                     size_t ws_bytes, void* stream) {
  return gdpa::run(problems, tensors, n_groups, ws, ws_bytes, stream, 0);
}

int gdpa_bwd_grouped(const gdpa_problem* problems, const gdpa_tensors* tensors, int32_t n_groups, void* ws,
                     size_t ws_bytes, void* stream) {
  return gdpa::run(problems, tensors, n_groups, ws, ws_bytes, stream, 1);
}

int gdpa_plan(const gdpa_problem* problems, int32_t n_groups, void* ws, size_t ws_bytes, void* stream) {
  gdpa::WsLayout L;
  int rc = gdpa::layout(problems, n_groups, 0, &L);
  if (rc != GDPA_OK) return rc;
  if (!ws || ((uintptr_t)ws % gdpa::kAlign) != 0 || ws_bytes < L.total) return GDPA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // nothing to order: no later call launches a kernel (no items), or fp32 calls, which need no
  // list and clear the error word themselves
  if (L.n_items == 0 || problems[0].dtype != GDPA_DTYPE_BF16) return GDPA_OK;
  gdpa::LaunchDesc d;
  gdpa_tensors none[GDPA_MAX_GROUPS];
  std::memset(none, 0, sizeof(none));
  gdpa::fill_desc(problems, none, n_groups, ws, L, &d);
  return gdpa::launch_schedule(d, s) == hipSuccess ? GDPA_OK : GDPA_ERR_HIP;
}

int gdpa_validate_offsets(const gdpa_problem* problem, const int32_t* q_offsets_host,
                          const int32_t* kv_offsets_host) {
  if (!problem) return GDPA_ERR_INVALID_ARGUMENT;
  gdpa_problem p = *problem;
  // the device pointers are not read here: stand in host copies so the problem checks pass
  p.q_offsets = q_offsets_host;
  p.kv_offsets = kv_offsets_host;
  int rc = gdpa::check_problem(p);
  if (rc != GDPA_OK) return rc;
  if (p.num_seqs > 0 && (!q_offsets_host || !kv_offsets_host)) return GDPA_ERR_INVALID_ARGUMENT;
  gdpa::OffsetsRules r;
  r.num_seqs = p.num_seqs;
  r.self_attention = p.self_attention;
  r.total_q = p.total_q;
  r.total_kv = p.total_kv;
  r.max_q = p.max_seqlen_q;
  r.max_kv = p.max_seqlen_kv;
  int32_t bits = 0;
  for (int b = 0; b < p.num_seqs; ++b) bits |= gdpa::seq_offsets_error(r, q_offsets_host, kv_offsets_host, b);
  return bits;
}

const char* gdpa_strerror(int status) {
  switch (status) {
    case GDPA_OK: return "ok";
    case GDPA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case GDPA_ERR_UNSUPPORTED: return "unsupported problem shape";
    case GDPA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case GDPA_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int gdpa_version(void) { return 300; }  // 0.3.0: device error word, offsets validation, gdpa_bwd_noalloc

}  // extern "C"
