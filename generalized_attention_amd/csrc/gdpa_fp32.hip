// GDPA in fp32 (exact-erf GELU, accurate exp): one thread per (row, head) for the forward and
// the dQ part of the backward, one thread per (key, head) for dK / dV / dG.
//
// fp32 problems are the small, latency-bound correctness configurations; their tolerance is an
// absolute 1e-5, so these kernels use the device math library (erff, expf, log1pf) instead of the
// bf16 kernels' short activation forms. Same definition as the bf16 kernels (Kunlun review,
// section 2.3 / Figure 2; reproduction README "Core equations"; review section 2.5 for windows).
#include "gdpa_device.hpp"
#include "gdpa_launch.hpp"

namespace gdpa {

namespace {

__device__ inline float sigmoid_exact(float x) {
  if (x >= 0.0f) return 1.0f / (1.0f + expf(-x));
  const float e = expf(x);
  return e / (1.0f + e);
}
__device__ inline float log_sigmoid_exact(float x) { return fminf(x, 0.0f) - log1pf(expf(-fabsf(x))); }
__device__ inline float act_f(int act, float x) {
  if (act == GDPA_ACT_GELU) return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
  return x * sigmoid_exact(x);
}
__device__ inline float act_g(int act, float x) {
  if (act == GDPA_ACT_GELU)
    return 0.5f * (1.0f + erff(x * 0.70710678118654752f)) + x * 0.39894228040143268f * expf(-0.5f * x * x);
  const float s = sigmoid_exact(x);
  return s * (1.0f + x * (1.0f - s));
}

// Sequence b that owns global row `row` (offsets non-decreasing, B >= 1).
__device__ inline int seq_of(const int32_t* off, int B, int64_t row) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ inline void key_range(const GroupDesc& gd, int i, int n, int& lo, int& hi) {
  lo = 0;
  hi = n - 1;
  if (gd.wl >= 0 && i - gd.wl > lo) lo = i - gd.wl;
  if (gd.wr >= 0 && i + gd.wr < hi) hi = i + gd.wr;
}

}  // namespace

// The row's (or key's) sequence b found by the search must own it, and b's offsets must pass the
// item check; otherwise the thread records the error and writes nothing.
__device__ inline bool fp32_guard(const GroupDesc& gd, int b, int64_t pos, bool is_key, int32_t* err) {
  const int q0 = gd.q_off[b], q1 = gd.q_off[b + 1], k0 = gd.kv_off[b], k1 = gd.kv_off[b + 1];
  int32_t e = item_error(gd, q0, q1, k0, k1, -1);
  if (e == 0 && (is_key ? (pos < k0 || pos >= k1) : (pos < q0 || pos >= q1))) e = GDPA_DEVICE_ERR_OFFSETS;
  if (e != 0) atomicOr(err, e);
  return e == 0;
}

template <int D>
__device__ void fwd_row(const GroupDesc& gd, int64_t grow, int h, int32_t* err) {
  const int H = gd.num_heads;
  const int b = seq_of(gd.q_off, gd.num_seqs, grow);
  if (!fp32_guard(gd, b, grow, false, err)) return;
  const int q0 = gd.q_off[b], k0 = gd.kv_off[b];
  const int i = (int)(grow - q0), n = gd.kv_off[b + 1] - k0;
  const float* q = reinterpret_cast<const float*>(gd.q) + (grow * H + h) * D;
  const float* K = reinterpret_cast<const float*>(gd.k);
  const float* V = reinterpret_cast<const float*>(gd.v);
  float qr[D], acc[D];
  for (int c = 0; c < D; ++c) { qr[c] = q[c]; acc[c] = 0.0f; }
  int lo, hi;
  key_range(gd, i, n, lo, hi);
  const int act = gd.head_acts ? gd.head_acts[h] : gd.act;
  const bool softmax = act == GDPA_ACT_SOFTMAX;
  float m = -__builtin_inff(), l = 0.0f;
  for (int j = lo; j <= hi; ++j) {
    const float* kj = K + ((int64_t)(k0 + j) * H + h) * D;
    float s = 0.0f;
    for (int c = 0; c < D; ++c) s = fmaf(qr[c], kj[c], s);
    s *= gd.scale;
    if (gd.g) s += log_sigmoid_exact(gd.g[(int64_t)(k0 + j) * H + h]);
    const float* vj = V + ((int64_t)(k0 + j) * H + h) * D;
    float p;
    if (softmax) {
      const float mn = fmaxf(m, s);
      const float a = expf(m - mn);
      p = expf(s - mn);
      l = l * a + p;
      for (int c = 0; c < D; ++c) acc[c] *= a;
      m = mn;
    } else {
      p = act_f(act, s);
    }
    for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vj[c], acc[c]);
  }
  const float inv = softmax ? (l > 0.0f ? 1.0f / l : 0.0f) : 1.0f;
  float* o = reinterpret_cast<float*>(gd.o) + (grow * H + h) * D;
  for (int c = 0; c < D; ++c) o[c] = acc[c] * inv;
  const float lse = l > 0.0f ? m + logf(l) : -__builtin_inff();
  if (softmax && gd.lse) gd.lse[grow * H + h] = lse;
}

template <int D>
__device__ void bwd_row(const GroupDesc& gd, int64_t grow, int h, const float* ws_lse, float* ws_delta, int32_t* err) {
  const int H = gd.num_heads;
  const int b = seq_of(gd.q_off, gd.num_seqs, grow);
  if (!fp32_guard(gd, b, grow, false, err)) return;
  const int q0 = gd.q_off[b], k0 = gd.kv_off[b];
  const int i = (int)(grow - q0), n = gd.kv_off[b + 1] - k0;
  const float* q = reinterpret_cast<const float*>(gd.q) + (grow * H + h) * D;
  const float* dO = reinterpret_cast<const float*>(gd.dout) + (grow * H + h) * D;
  const float* K = reinterpret_cast<const float*>(gd.k);
  const float* V = reinterpret_cast<const float*>(gd.v);
  float qr[D], dor[D], dq[D];
  for (int c = 0; c < D; ++c) { qr[c] = q[c]; dor[c] = dO[c]; dq[c] = 0.0f; }
  int lo, hi;
  key_range(gd, i, n, lo, hi);
  const int act = gd.head_acts ? gd.head_acts[h] : gd.act;
  const bool softmax = act == GDPA_ACT_SOFTMAX;
  const float lse = softmax ? ws_lse[grow * H + h] : 0.0f;
  // softmax: D_i = sum_j p_ij dp_ij first
  float Dsum = 0.0f;
  if (softmax) {
    for (int j = lo; j <= hi; ++j) {
      const float* kj = K + ((int64_t)(k0 + j) * H + h) * D;
      const float* vj = V + ((int64_t)(k0 + j) * H + h) * D;
      float s = 0.0f, dp = 0.0f;
      for (int c = 0; c < D; ++c) { s = fmaf(qr[c], kj[c], s); dp = fmaf(dor[c], vj[c], dp); }
      s *= gd.scale;
      if (gd.g) s += log_sigmoid_exact(gd.g[(int64_t)(k0 + j) * H + h]);
      Dsum += expf(s - lse) * dp;
    }
    ws_delta[grow * H + h] = Dsum;
  }
  for (int j = lo; j <= hi; ++j) {
    const float* kj = K + ((int64_t)(k0 + j) * H + h) * D;
    const float* vj = V + ((int64_t)(k0 + j) * H + h) * D;
    float s = 0.0f, dp = 0.0f;
    for (int c = 0; c < D; ++c) { s = fmaf(qr[c], kj[c], s); dp = fmaf(dor[c], vj[c], dp); }
    s *= gd.scale;
    if (gd.g) s += log_sigmoid_exact(gd.g[(int64_t)(k0 + j) * H + h]);
    const float ds = softmax ? expf(s - lse) * (dp - Dsum) : dp * act_g(act, s);
    for (int c = 0; c < D; ++c) dq[c] = fmaf(ds, kj[c], dq[c]);
  }
  float* o = reinterpret_cast<float*>(gd.dq) + (grow * H + h) * D;
  for (int c = 0; c < D; ++c) o[c] = dq[c] * gd.scale;
}

template <int D>
__device__ void bwd_key(const GroupDesc& gd, int64_t gkey, int h, const float* ws_lse, const float* ws_delta,
                        int32_t* err) {
  const int H = gd.num_heads;
  const int b = seq_of(gd.kv_off, gd.num_seqs, gkey);
  if (!fp32_guard(gd, b, gkey, true, err)) return;
  const int q0 = gd.q_off[b], k0 = gd.kv_off[b];
  const int j = (int)(gkey - k0), L = gd.q_off[b + 1] - q0, n = gd.kv_off[b + 1] - k0;
  const float* kj = reinterpret_cast<const float*>(gd.k) + (gkey * H + h) * D;
  const float* vj = reinterpret_cast<const float*>(gd.v) + (gkey * H + h) * D;
  const float* Q = reinterpret_cast<const float*>(gd.q);
  const float* DO = reinterpret_cast<const float*>(gd.dout);
  float kr[D], vr[D], dk[D], dv[D];
  for (int c = 0; c < D; ++c) { kr[c] = kj[c]; vr[c] = vj[c]; dk[c] = 0.0f; dv[c] = 0.0f; }
  const float gate = gd.g ? log_sigmoid_exact(gd.g[gkey * H + h]) : 0.0f;
  const int act = gd.head_acts ? gd.head_acts[h] : gd.act;
  const bool softmax = act == GDPA_ACT_SOFTMAX;
  // queries that see key j: i - wl <= j <= i + wr  <=>  j - wr <= i <= j + wl
  int ilo = 0, ihi = L - 1;
  if (gd.wr >= 0 && j - gd.wr > ilo) ilo = j - gd.wr;
  if (gd.wl >= 0 && j + gd.wl < ihi) ihi = j + gd.wl;
  float dssum = 0.0f;
  for (int i = ilo; i <= ihi && j < n; ++i) {
    const int64_t grow = q0 + i;
    const float* qi = Q + (grow * H + h) * D;
    const float* doi = DO + (grow * H + h) * D;
    float s = 0.0f, dp = 0.0f;
    for (int c = 0; c < D; ++c) { s = fmaf(qi[c], kr[c], s); dp = fmaf(doi[c], vr[c], dp); }
    s = s * gd.scale + gate;
    float p, ds;
    if (softmax) {
      p = expf(s - ws_lse[grow * H + h]);  // softmax only: ws_lse = forward lse
      ds = p * (dp - ws_delta[grow * H + h]);
    } else {
      p = act_f(act, s);
      ds = dp * act_g(act, s);
    }
    dssum += ds;
    for (int c = 0; c < D; ++c) {
      dk[c] = fmaf(ds, qi[c], dk[c]);
      dv[c] = fmaf(p, doi[c], dv[c]);
    }
  }
  float* dko = reinterpret_cast<float*>(gd.dk) + (gkey * H + h) * D;
  float* dvo = reinterpret_cast<float*>(gd.dv) + (gkey * H + h) * D;
  for (int c = 0; c < D; ++c) { dko[c] = dk[c] * gd.scale; dvo[c] = dv[c]; }
  if (gd.dg) gd.dg[gkey * H + h] = sigmoid_exact(-gd.g[gkey * H + h]) * dssum;
}

// Flat thread index -> (group, row or key of that group, head); `pre` is the prefix over groups
// of rows*heads (or keys*heads).
__device__ inline bool flat_to(const int64_t* pre, int n_groups, const LaunchDesc& d, int64_t t, int& g,
                               int64_t& row, int& h) {
  if (t >= pre[n_groups]) return false;
  g = 0;
  while (g + 1 < n_groups && t >= pre[g + 1]) ++g;
  const int64_t local = t - pre[g];
  const int H = d.grp[g].num_heads;
  row = local / H;
  h = (int)(local % H);
  return true;
}


__global__ void __launch_bounds__(256) fwd_fp32_kernel(LaunchDesc d, Fp32Aux aux) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int g, h;
  int64_t row;
  if (launch_refused(d) || !flat_to(aux.row_pre, d.n_groups, d, t, g, row, h)) return;
  const GroupDesc& gd = d.grp[g];
  if (gd.head_dim == 32) fwd_row<32>(gd, row, h, d.err);
  else if (gd.head_dim == 64) fwd_row<64>(gd, row, h, d.err);
  else fwd_row<128>(gd, row, h, d.err);
}

__global__ void __launch_bounds__(256) bwd_fp32_rows_kernel(LaunchDesc d, Fp32Aux aux) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int g, h;
  int64_t row;
  if (launch_refused(d) || !flat_to(aux.row_pre, d.n_groups, d, t, g, row, h)) return;
  const GroupDesc& gd = d.grp[g];
  const float* wl = gd.lse;
  float* wd = aux.ws_delta + aux.row_base[g];
  if (gd.head_dim == 32) bwd_row<32>(gd, row, h, wl, wd, d.err);
  else if (gd.head_dim == 64) bwd_row<64>(gd, row, h, wl, wd, d.err);
  else bwd_row<128>(gd, row, h, wl, wd, d.err);
}

__global__ void __launch_bounds__(256) bwd_fp32_keys_kernel(LaunchDesc d, Fp32Aux aux) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int g, h;
  int64_t key;
  if (launch_refused(d) || !flat_to(aux.key_pre, d.n_groups, d, t, g, key, h)) return;
  const GroupDesc& gd = d.grp[g];
  const float* wl = gd.lse;
  const float* wd = aux.ws_delta + aux.row_base[g];
  if (gd.head_dim == 32) bwd_key<32>(gd, key, h, wl, wd, d.err);
  else if (gd.head_dim == 64) bwd_key<64>(gd, key, h, wl, wd, d.err);
  else bwd_key<128>(gd, key, h, wl, wd, d.err);
}

static int64_t blocks_for(int64_t n) { return (n + 255) / 256; }
// both are kernel arguments of the fp32 kernels (the argument block holds at most 4 KB)
static_assert(sizeof(LaunchDesc) + sizeof(Fp32Aux) <= 4096, "kernel argument size");

hipError_t launch_fwd_fp32(const LaunchDesc& d, const Fp32Aux& aux, hipStream_t stream) {
  const int64_t n = aux.row_pre[d.n_groups];
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_fp32_kernel, dim3((unsigned)blocks_for(n)), dim3(256), 0, stream, d, aux);
  return hipGetLastError();
}

hipError_t launch_bwd_fp32(const LaunchDesc& d, const Fp32Aux& aux, hipStream_t stream) {
  const int64_t nr = aux.row_pre[d.n_groups], nk = aux.key_pre[d.n_groups];
  if (nr > 0) hipLaunchKernelGGL(bwd_fp32_rows_kernel, dim3((unsigned)blocks_for(nr)), dim3(256), 0, stream, d, aux);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nk > 0) hipLaunchKernelGGL(bwd_fp32_keys_kernel, dim3((unsigned)blocks_for(nk)), dim3(256), 0, stream, d, aux);
  return hipGetLastError();
}

}  // namespace gdpa
