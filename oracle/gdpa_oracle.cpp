// Plain fp64 CPU reference ("oracle") for generalized dot-product attention (GDPA).
//
// TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the benchmark's
// CPU-baseline leg may load or call this library. The product path never does: it shares no
// code, header, table or helper with it.
//
// What it computes is the operator's plain definition, one (sequence b, head h) pair at a
// time, one query row at a time, with no blocking, fusion or online rescaling:
//
//   s_ij = scale * <q_i, k_j> + log sigmoid(G_jh)          (gate term only when G is given)
//   pointwise form:  p_ij = phi(s_ij) for allowed j, 0 otherwise;   phi in {GELU, SiLU}
//   softmax form:    p_ij = exp(s_ij - m_i) / l_i over the allowed j; lse_i = m_i + ln l_i
//   o_i = sum_j p_ij v_j
//
// Sources (Kunlun paper review, liuzhao09.github.io, section 2.3 "GDPA" and Figure 2): the
// personalized FFN is recast as multi-head cross-attention whose queries are the sequence
// tokens and whose per-head keys and values come from the non-sequence context; the scores are
// divided by a temperature and passed through an element-wise activation such as GELU instead
// of a softmax. The gated-softmax form with the additive log-sigmoid gate is the "Core
// equations" paragraph of the Kunlun reproduction README (daiwk.github.io). The sliding window
// (query t sees keys t-w .. t+w) is section 2.5 of the review; here the two sides of the window
// are separate arguments so that the causal window (left w, right 0) is expressible.
//
// Backward (gradients of the same definition, by the chain rule):
//   dp_ij = <do_i, v_j>
//   pointwise: ds_ij = dp_ij * phi'(s_ij);  softmax: ds_ij = p_ij (dp_ij - sum_k p_ik dp_ik)
//   dq_i = scale * sum_j ds_ij k_j;  dk_j = scale * sum_i ds_ij q_i;  dv_j = sum_i p_ij do_i
//   dG_jh = sigmoid(-G_jh) * sum_i ds_ij
//
// Layouts: q, o, dout, dq are [total_q, H, d]; k, v, dk, dv are [total_kv, H, d]; g, dg are
// [total_kv, H]; lse is [total_q, H]; all row-major float64. Offsets are int64 [B+1]. The
// position of query row i and key row j inside their sequence (0-based) defines the window.
//
// Shared queries (PMA-style pooling: one learnable query matrix attends over every sequence;
// review, sections 2.3-2.4): q and dq are then [S, H, d] and query row i of every sequence is
// row i of q, so that o_bi uses q_i and dq_i = sum over sequences b of the gradient through o_bi.

#include <atomic>
#include <cmath>
#include <cstdint>
#include <limits>
#include <thread>
#include <vector>

namespace {

enum { ACT_GELU = 0, ACT_SILU = 1, ACT_SOFTMAX = 2 };

const double kSqrt2 = 1.4142135623730950488;
const double kInvSqrt2Pi = 0.39894228040143267794;

double sigmoid(double x) {
  if (x >= 0) return 1.0 / (1.0 + std::exp(-x));
  double e = std::exp(x);
  return e / (1.0 + e);
}

// log(sigmoid(x)) = -log(1 + exp(-x)), written so that neither branch overflows.
double log_sigmoid(double x) {
  if (x >= 0) return -std::log1p(std::exp(-x));
  return x - std::log1p(std::exp(x));
}

// GELU with the exact Gaussian CDF: x * Phi(x), Phi(x) = (1 + erf(x / sqrt 2)) / 2.
double gelu(double x) { return x * 0.5 * (1.0 + std::erf(x / kSqrt2)); }
double gelu_grad(double x) {
  return 0.5 * (1.0 + std::erf(x / kSqrt2)) + x * kInvSqrt2Pi * std::exp(-0.5 * x * x);
}

// SiLU: x * sigmoid(x); derivative sigmoid(x) * (1 + x (1 - sigmoid(x))).
double silu(double x) { return x * sigmoid(x); }
double silu_grad(double x) {
  double s = sigmoid(x);
  return s * (1.0 + x * (1.0 - s));
}

double phi(int act, double x) { return act == ACT_GELU ? gelu(x) : silu(x); }
double phi_grad(int act, double x) { return act == ACT_GELU ? gelu_grad(x) : silu_grad(x); }

struct Problem {
  int B, H, d;
  const int64_t* q_off;
  const int64_t* kv_off;
  const double *q, *k, *v, *g;
  int act;
  double scale;
  int wl, wr;  // window sides, -1 = unbounded
  const int* head_acts;  // activation of each head, or NULL: every head uses act
  int shared_q;          // S > 0: one [S, H, d] query matrix for every sequence; 0: per sequence
};

// Query row i of sequence b, head h.
const double* query_row(const Problem& p, int b, int64_t i, int h) {
  const int64_t row = (p.shared_q > 0 ? 0 : p.q_off[b]) + i;
  return p.q + (row * p.H + h) * p.d;
}

// Activation of head h (heads may each use their own; review section 2.3 lets phi vary by head).
int act_of(const Problem& p, int h) { return p.head_acts ? p.head_acts[h] : p.act; }

// Allowed key range [lo, hi] of query position i in a sequence with lk keys (empty if hi < lo).
void allowed_range(const Problem& p, int64_t i, int64_t lk, int64_t* lo, int64_t* hi) {
  int64_t a = 0, b = lk - 1;
  if (p.wl >= 0 && i - p.wl > a) a = i - p.wl;
  if (p.wr >= 0 && i + p.wr < b) b = i + p.wr;
  *lo = a;
  *hi = b;
}

double dot(const double* x, const double* y, int n) {
  double s = 0.0;
  for (int c = 0; c < n; ++c) s += x[c] * y[c];
  return s;
}

// Row i of sequence b, head h: scores s[j] and probabilities/activations pr[j] for j in
// [lo, hi] (stored at index j - lo). Returns lse (softmax) or 0.
double score_row(const Problem& p, int b, int h, int64_t i, int64_t lo, int64_t hi,
                 std::vector<double>& s, std::vector<double>& pr) {
  const int H = p.H, d = p.d;
  const int64_t k0 = p.kv_off[b];
  const double* qi = query_row(p, b, i, h);
  int64_t n = hi - lo + 1;
  s.assign(n > 0 ? n : 0, 0.0);
  pr.assign(n > 0 ? n : 0, 0.0);
  for (int64_t j = lo; j <= hi; ++j) {
    const double* kj = p.k + ((k0 + j) * H + h) * d;
    double sij = p.scale * dot(qi, kj, d);
    if (p.g) sij += log_sigmoid(p.g[(k0 + j) * H + h]);
    s[j - lo] = sij;
  }
  const int act = act_of(p, h);
  if (act != ACT_SOFTMAX) {
    for (int64_t t = 0; t < n; ++t) pr[t] = phi(act, s[t]);
    return 0.0;
  }
  if (n <= 0) return -std::numeric_limits<double>::infinity();
  double m = -std::numeric_limits<double>::infinity();
  for (int64_t t = 0; t < n; ++t) m = s[t] > m ? s[t] : m;
  double l = 0.0;
  for (int64_t t = 0; t < n; ++t) l += std::exp(s[t] - m);
  for (int64_t t = 0; t < n; ++t) pr[t] = std::exp(s[t] - m) / l;
  return m + std::log(l);
}

void fwd_item(const Problem& p, int b, int h, double* o, double* lse) {
  const int H = p.H, d = p.d;
  const int64_t q0 = p.q_off[b], lq = p.q_off[b + 1] - q0;
  const int64_t k0 = p.kv_off[b], lk = p.kv_off[b + 1] - k0;
  std::vector<double> s, pr;
  for (int64_t i = 0; i < lq; ++i) {
    int64_t lo, hi;
    allowed_range(p, i, lk, &lo, &hi);
    double l = score_row(p, b, h, i, lo, hi, s, pr);
    double* oi = o + ((q0 + i) * H + h) * d;
    for (int c = 0; c < d; ++c) oi[c] = 0.0;
    for (int64_t j = lo; j <= hi; ++j) {
      const double* vj = p.v + ((k0 + j) * H + h) * d;
      for (int c = 0; c < d; ++c) oi[c] += pr[j - lo] * vj[c];
    }
    if (lse) lse[(q0 + i) * H + h] = l;
  }
}

// dq receives the gradient of query row i at ((dq_row0 + i) * H + h) * d.
void bwd_item(const Problem& p, int b, int h, const double* dout, double* dq, int64_t dq_row0,
              double* dk, double* dv, double* dg) {
  const int H = p.H, d = p.d;
  const int64_t q0 = p.q_off[b], lq = p.q_off[b + 1] - q0;
  const int64_t k0 = p.kv_off[b], lk = p.kv_off[b + 1] - k0;
  for (int64_t j = 0; j < lk; ++j) {
    double* dkj = dk + ((k0 + j) * H + h) * d;
    double* dvj = dv + ((k0 + j) * H + h) * d;
    for (int c = 0; c < d; ++c) dkj[c] = dvj[c] = 0.0;
    if (dg) dg[(k0 + j) * H + h] = 0.0;
  }
  std::vector<double> s, pr, dp, ds;
  for (int64_t i = 0; i < lq; ++i) {
    int64_t lo, hi;
    allowed_range(p, i, lk, &lo, &hi);
    score_row(p, b, h, i, lo, hi, s, pr);
    const int64_t n = hi >= lo ? hi - lo + 1 : 0;
    const double* qi = query_row(p, b, i, h);
    const double* doi = dout + ((q0 + i) * H + h) * d;
    dp.assign(n, 0.0);
    ds.assign(n, 0.0);
    for (int64_t j = lo; j <= hi; ++j) dp[j - lo] = dot(doi, p.v + ((k0 + j) * H + h) * d, d);
    const int act = act_of(p, h);
    if (act == ACT_SOFTMAX) {
      double D = 0.0;
      for (int64_t t = 0; t < n; ++t) D += pr[t] * dp[t];
      for (int64_t t = 0; t < n; ++t) ds[t] = pr[t] * (dp[t] - D);
    } else {
      for (int64_t t = 0; t < n; ++t) ds[t] = dp[t] * phi_grad(act, s[t]);
    }
    double* dqi = dq + ((dq_row0 + i) * H + h) * d;
    for (int c = 0; c < d; ++c) dqi[c] = 0.0;
    for (int64_t j = lo; j <= hi; ++j) {
      const double* kj = p.k + ((k0 + j) * H + h) * d;
      double* dkj = dk + ((k0 + j) * H + h) * d;
      double* dvj = dv + ((k0 + j) * H + h) * d;
      const double dsij = ds[j - lo], pij = pr[j - lo];
      for (int c = 0; c < d; ++c) {
        dqi[c] += p.scale * dsij * kj[c];
        dkj[c] += p.scale * dsij * qi[c];
        dvj[c] += pij * doi[c];
      }
      if (dg) dg[(k0 + j) * H + h] += sigmoid(-p.g[(k0 + j) * H + h]) * dsij;
    }
  }
}

bool valid(const Problem& p) {
  if (p.B < 0 || p.H <= 0 || p.d <= 0) return false;
  if (p.act < ACT_GELU || p.act > ACT_SOFTMAX) return false;
  if (p.head_acts)
    for (int h = 0; h < p.H; ++h)
      if (p.head_acts[h] < ACT_GELU || p.head_acts[h] > ACT_SOFTMAX) return false;
  if (p.wl < -1 || p.wr < -1) return false;
  if (!p.q_off || !p.kv_off) return false;
  if (p.q_off[0] != 0 || p.kv_off[0] != 0) return false;
  for (int b = 0; b < p.B; ++b)
    if (p.q_off[b + 1] < p.q_off[b] || p.kv_off[b + 1] < p.kv_off[b]) return false;
  if (p.shared_q < 0) return false;
  if (p.shared_q > 0)
    for (int b = 0; b < p.B; ++b)
      if (p.q_off[b + 1] - p.q_off[b] > p.shared_q) return false;
  return true;
}

template <class F>
void parallel_items(int B, int H, int nthreads, F&& f) {
  const int n_items = B * H;
  if (nthreads <= 0) nthreads = (int)std::thread::hardware_concurrency();
  if (nthreads < 1) nthreads = 1;
  if (nthreads > n_items) nthreads = n_items > 0 ? n_items : 1;
  std::atomic<int> next(0);
  auto worker = [&]() {
    for (int it = next.fetch_add(1); it < n_items; it = next.fetch_add(1)) f(it / H, it % H);
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < nthreads; ++t) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// Element-wise helpers, exported so that tests can pin them to closed-form values.
double gdpa_oracle_phi(int act, double x) { return phi(act, x); }
double gdpa_oracle_phi_grad(int act, double x) { return phi_grad(act, x); }
double gdpa_oracle_log_sigmoid(double x) { return log_sigmoid(x); }

// Forward. g may be NULL (no gate). lse may be NULL; it is written for the softmax heads.
// head_acts may be NULL (every head uses act) or hold one activation per head. shared_q > 0:
// q is one [shared_q, H, d] matrix for every sequence (each sequence has at most shared_q rows).
// Returns 0, or -1 for invalid arguments (nothing written). nthreads <= 0 means all cores.
int gdpa_oracle_fwd(int B, int H, int d, const int64_t* q_off, const int64_t* kv_off,
                    const double* q, const double* k, const double* v, const double* g, int act,
                    double scale, int window_left, int window_right, double* o, double* lse,
                    int nthreads, const int* head_acts, int shared_q) {
  Problem p{B, H, d, q_off, kv_off, q, k, v, g, act, scale, window_left, window_right, head_acts, shared_q};
  if (!valid(p)) return -1;
  if (p.q_off[B] > 0 && (!q || !o)) return -1;
  if (p.kv_off[B] > 0 && (!k || !v)) return -1;
  parallel_items(B, H, nthreads, [&](int b, int h) { fwd_item(p, b, h, o, lse); });
  return 0;
}

// Backward: gradients of sum(dout * o) with respect to q, k, v (and G when dg != NULL).
// With shared queries, dq is [shared_q, H, d]: each sequence's query gradients are formed apart,
// then added over the sequences.
int gdpa_oracle_bwd(int B, int H, int d, const int64_t* q_off, const int64_t* kv_off,
                    const double* q, const double* k, const double* v, const double* g, int act,
                    double scale, int window_left, int window_right, const double* dout,
                    double* dq, double* dk, double* dv, double* dg, int nthreads,
                    const int* head_acts, int shared_q) {
  Problem p{B, H, d, q_off, kv_off, q, k, v, g, act, scale, window_left, window_right, head_acts, shared_q};
  if (!valid(p)) return -1;
  if (dg && !g) return -1;
  if ((p.q_off[B] > 0 || shared_q > 0) && (!q || !dq)) return -1;
  if (p.q_off[B] > 0 && !dout) return -1;
  if (p.kv_off[B] > 0 && (!k || !v || !dk || !dv)) return -1;
  if (shared_q == 0) {
    parallel_items(B, H, nthreads, [&](int b, int h) { bwd_item(p, b, h, dout, dq, p.q_off[b], dk, dv, dg); });
    return 0;
  }
  // per-sequence query gradients: rows [b * S, b * S + L_b) of part
  const int64_t S = shared_q;
  std::vector<double> part((size_t)B * S * H * d, 0.0);
  parallel_items(B, H, nthreads, [&](int b, int h) { bwd_item(p, b, h, dout, part.data(), b * S, dk, dv, dg); });
  for (int64_t x = 0; x < S * H * d; ++x) {
    double acc = 0.0;
    for (int b = 0; b < B; ++b) acc += part[(size_t)b * S * H * d + x];
    dq[x] = acc;
  }
  return 0;
}

}  // extern "C"
