// Host side of the OSCAR INT2 KV-cache library: the C ABI declared in
// include/oscar.h, offline calibration, page pools / sequences (block tables,
// region planning, prefix forks) and argument checking for the HIP launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>
#include <thread>
#include <tuple>
#include <vector>

#include "oscar.h"
#include "oscar_internal.h"

using namespace oscar;

namespace {

thread_local std::string g_err;

// Event pairs around the main kernel of each launch while profiling is on.
// They are created once and reused after each read (an event created per
// launch cost the host several microseconds a step, which at one request
// shows in the step time), and live as long as the thread.
struct ProfileState {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  size_t used = 0;  // pool[0, used): recorded since the last read
  // the next pair (nullptr, nullptr after an error)
  std::pair<hipEvent_t, hipEvent_t> acquire() {
    if (used == pool.size()) {
      hipEvent_t a = nullptr, b = nullptr;
      if (hipEventCreate(&a) != hipSuccess) return {nullptr, nullptr};
      if (hipEventCreate(&b) != hipSuccess) {
        (void)hipEventDestroy(a);
        return {nullptr, nullptr};
      }
      pool.emplace_back(a, b);
    }
    return pool[used++];
  }
};
thread_local ProfileState g_prof;

oscar_status fail(oscar_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

oscar_status ok() {
  g_err.clear();
  return OSCAR_OK;
}

oscar_status check_shape(const oscar_shape* s) {
  if (!s) return fail(OSCAR_EINVAL, "shape is NULL");
  if (s->head_dim != kHeadDim) return fail(OSCAR_EUNSUPPORTED, "head_dim %d unsupported (only %d)", s->head_dim, kHeadDim);
  if (s->page_size != kPage) return fail(OSCAR_EUNSUPPORTED, "page_size %d unsupported (only %d)", s->page_size, kPage);
  if (s->group != 32 && s->group != 64) return fail(OSCAR_EUNSUPPORTED, "group %d unsupported (32 or 64)", s->group);
  if (s->n_kv_heads < 1 || s->n_q_heads < 1 || s->n_q_heads % s->n_kv_heads)
    return fail(OSCAR_EINVAL, "n_q_heads %d must be a positive multiple of n_kv_heads %d", s->n_q_heads, s->n_kv_heads);
  const int g = s->n_q_heads / s->n_kv_heads;
  if (g > 16) return fail(OSCAR_EUNSUPPORTED, "query heads per KV head %d > 16", g);
  if (g * (kHeadDim / s->group) > 64) return fail(OSCAR_EUNSUPPORTED, "gqa * groups = %d > 64", g * (kHeadDim / s->group));
  if (s->sink < 0 || s->recent < 0) return fail(OSCAR_EINVAL, "sink/recent must be >= 0");
  if (s->recent % kPage) return fail(OSCAR_EUNSUPPORTED, "recent %d must be a multiple of %d", s->recent, kPage);
  if (s->sink > (1 << 26) || s->recent > (1 << 26)) return fail(OSCAR_EINVAL, "sink/recent too large");
  if (s->scale_bits != 0 && s->scale_bits != 16 && s->scale_bits != 8)
    return fail(OSCAR_EUNSUPPORTED, "scale_bits %d unsupported (16 or 8)", s->scale_bits);
  return OSCAR_OK;
}

int ng_of(const oscar_shape* s) { return kHeadDim / s->group; }
// 16-row tiles of one (request, KV head) in a decode launch: three at
// 32-channel groups are padded to four (one wide wavefront, see tile_split)
int ct_of(const oscar_shape* s) {
  const int t = (s->n_q_heads / s->n_kv_heads * ng_of(s) + 15) / 16;
  return ng_of(s) == 4 && t == 3 ? 4 : t;
}
int mb_of(const oscar_shape* s) { return s->scale_bits == 8 ? 2 : 4; }
int64_t int2_block(const oscar_shape* s) { return Int2Layout{ng_of(s), mb_of(s)}.bytes(); }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

oscar_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(OSCAR_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// ----------------------------------------------------------------------------
// Calibration ([IT] 2.2.A; [ES] "Lo que OSCAR hace diferente")
// ----------------------------------------------------------------------------

// Cyclic Jacobi eigenvalue method for a symmetric matrix a (n x n, row-major,
// overwritten).  On return w holds the eigenvalues and column k of v the
// eigenvector of w[k].
void jacobi_eigen(int n, std::vector<double>& a, std::vector<double>& v, std::vector<double>& w) {
  v.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) v[(size_t)i * n + i] = 1.0;
  auto A = [&](int i, int j) -> double& { return a[(size_t)i * n + j]; };
  double scale = 0.0;
  for (double x : a) scale = std::max(scale, std::fabs(x));
  if (scale == 0.0) scale = 1.0;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int i = 0; i < n; ++i)
      for (int j = i + 1; j < n; ++j) off += A(i, j) * A(i, j);
    if (std::sqrt(off) <= 1e-300 || std::sqrt(off) < 1e-17 * scale) break;
    for (int p = 0; p < n - 1; ++p) {
      for (int q = p + 1; q < n; ++q) {
        const double apq = A(p, q);
        if (apq == 0.0) continue;
        const double app = A(p, p), aqq = A(q, q);
        // skip rotations that cannot change the diagonal any more
        if (sweep > 3 && std::fabs(apq) < 1e-18 * (std::fabs(app) + std::fabs(aqq)) ) {
          A(p, q) = A(q, p) = 0.0;
          continue;
        }
        const double theta = (aqq - app) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0);
        const double s = t * c;
        for (int k = 0; k < n; ++k) {
          const double akp = A(k, p), akq = A(k, q);
          A(k, p) = c * akp - s * akq;
          A(k, q) = s * akp + c * akq;
        }
        for (int k = 0; k < n; ++k) {
          const double apk = A(p, k), aqk = A(q, k);
          A(p, k) = c * apk - s * aqk;
          A(q, k) = s * apk + c * aqk;
        }
        A(p, q) = A(q, p) = 0.0;
        for (int k = 0; k < n; ++k) {
          double* row = &v[(size_t)k * n];
          const double vkp = row[p], vkq = row[q];
          row[p] = c * vkp - s * vkq;
          row[q] = s * vkp + c * vkq;
        }
      }
    }
  }
  w.resize(n);
  for (int i = 0; i < n; ++i) w[i] = A(i, i);
}

// Eigenbasis of a symmetric matrix, eigenvalues descending, each eigenvector
// signed so that its largest-magnitude entry is positive (first index on ties).
void eig_desc(int n, const std::vector<double>& c, std::vector<double>& lam, std::vector<double>& u) {
  std::vector<double> a = c, v, w;
  jacobi_eigen(n, a, v, w);
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return w[x] > w[y]; });
  lam.resize(n);
  u.assign((size_t)n * n, 0.0);
  for (int k = 0; k < n; ++k) {
    const int src = order[k];
    lam[k] = w[src];
    int imax = 0;
    double best = -1.0;
    for (int i = 0; i < n; ++i) {
      const double m = std::fabs(v[(size_t)i * n + src]);
      if (m > best) {
        best = m;
        imax = i;
      }
    }
    const double sgn = v[(size_t)imax * n + src] < 0 ? -1.0 : 1.0;
    for (int i = 0; i < n; ++i) u[(size_t)i * n + k] = sgn * v[(size_t)i * n + src];
  }
}

int bit_reverse(int j, int bits) {
  int r = 0;
  for (int b = 0; b < bits; ++b) {
    r = (r << 1) | (j & 1);
    j >>= 1;
  }
  return r;
}

// R = U H P_br with H the orthonormal Sylvester Walsh-Hadamard matrix (natural
// order) and (M P_br)[i][j] = M[i][rev(j)].
void composite_rotation(int n, const std::vector<double>& u, std::vector<double>& r) {
  int bits = 0;
  while ((1 << bits) < n) ++bits;
  const double inv = 1.0 / std::sqrt((double)n);
  std::vector<double> uh((size_t)n * n);
  for (int i = 0; i < n; ++i)
    for (int m = 0; m < n; ++m) {
      double s = 0.0;
      for (int k = 0; k < n; ++k) s += u[(size_t)i * n + k] * ((__builtin_popcount(k & m) & 1) ? -inv : inv);
      uh[(size_t)i * n + m] = s;
    }
  r.resize((size_t)n * n);
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) r[(size_t)i * n + j] = uh[(size_t)i * n + bit_reverse(j, bits)];
}

// c-quantile with linear interpolation between order statistics (the
// lerp is evaluated from the nearer end, as numerically stable lerps do).
double quantile_linear(std::vector<double>& x, double c) {
  const size_t n = x.size();
  const double h = (double)(n - 1) * c;
  size_t lo = (size_t)std::floor(h);
  if (lo >= n - 1) {
    std::nth_element(x.begin(), x.begin() + (n - 1), x.end());
    return x[n - 1];
  }
  std::nth_element(x.begin(), x.begin() + lo, x.end());
  const double a = x[lo];
  const double b = *std::min_element(x.begin() + lo + 1, x.end());
  const double t = h - (double)lo;
  const double diff = b - a;
  return t >= 0.5 ? b - diff * (1.0 - t) : a + diff * t;
}

void calibrate_head(const oscar_shape* sh, int64_t n, const float* q, const float* k, const float* v, int kvh,
                    float* r_k32, float* r_v32, double* eig_k, double* eig_v) {
  const int d = kHeadDim, hq = sh->n_q_heads, hkv = sh->n_kv_heads, g = hq / hkv;
  const double norm = 1.0 / ((double)n * g);
  std::vector<double> cq((size_t)d * d, 0.0), cs((size_t)d * d, 0.0);
  std::vector<double> qrow(d), logit((size_t)n), o(d);
  std::vector<double> kk((size_t)n * d), vv((size_t)n * d);
  for (int64_t t = 0; t < n; ++t)
    for (int j = 0; j < d; ++j) {
      kk[(size_t)t * d + j] = k[((size_t)t * hkv + kvh) * d + j];
      vv[(size_t)t * d + j] = v[((size_t)t * hkv + kvh) * d + j];
    }
  const double inv_sqrt_d = 1.0 / std::sqrt((double)d);
  for (int h = 0; h < g; ++h) {
    const int qh = kvh * g + h;
    for (int64_t t = 0; t < n; ++t) {
      for (int j = 0; j < d; ++j) qrow[j] = q[((size_t)t * hq + qh) * d + j];
      // C_Q += q^T q
      for (int i = 0; i < d; ++i) {
        const double qi = qrow[i];
        double* row = &cq[(size_t)i * d];
        for (int j = 0; j < d; ++j) row[j] += qi * qrow[j];
      }
      // causal attention output row o_t = sum_{s<=t} softmax_s(q.k_s/sqrt d) v_s
      double mx = -std::numeric_limits<double>::infinity();
      for (int64_t s = 0; s <= t; ++s) {
        const double* ks = &kk[(size_t)s * d];
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += qrow[j] * ks[j];
        logit[s] = acc * inv_sqrt_d;
        mx = std::max(mx, logit[s]);
      }
      double den = 0.0;
      for (int64_t s = 0; s <= t; ++s) {
        logit[s] = std::exp(logit[s] - mx);
        den += logit[s];
      }
      std::fill(o.begin(), o.end(), 0.0);
      for (int64_t s = 0; s <= t; ++s) {
        const double p = logit[s] / den;
        const double* vs = &vv[(size_t)s * d];
        for (int j = 0; j < d; ++j) o[j] += p * vs[j];
      }
      // C_S += o^T o   (V^T S^T S V = (S V)^T (S V))
      for (int i = 0; i < d; ++i) {
        const double oi = o[i];
        double* row = &cs[(size_t)i * d];
        for (int j = 0; j < d; ++j) row[j] += oi * o[j];
      }
    }
  }
  for (auto& x : cq) x *= norm;
  for (auto& x : cs) x *= norm;
  std::vector<double> lam, u, r;
  for (int which = 0; which < 2; ++which) {
    eig_desc(d, which ? cs : cq, lam, u);
    composite_rotation(d, u, r);
    float* r32 = (which ? r_v32 : r_k32) + (size_t)kvh * d * d;
    for (size_t i = 0; i < (size_t)d * d; ++i) r32[i] = (float)r[i];
    double* e = which ? eig_v : eig_k;
    if (e)
      for (int i = 0; i < d; ++i) e[(size_t)kvh * d + i] = lam[i];
  }
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================

extern "C" {

const char* oscar_last_error(void) { return g_err.c_str(); }

int64_t oscar_int2_block_bytes(const oscar_shape* shape) {
  if (check_shape(shape) != OSCAR_OK) return -1;
  return int2_block(shape);
}

int64_t oscar_bf16_block_bytes(const oscar_shape* shape) {
  if (check_shape(shape) != OSCAR_OK) return -1;
  return kBf16BlockBytes;
}

oscar_status oscar_calibrate_host_rotation(const oscar_shape* shape, int32_t rotation, int64_t n, const float* q,
                                           const float* k, const float* v, double clip_pct_k, double clip_pct_v,
                                           float* r_k_out, float* r_v_out, double* eig_k_out, double* eig_v_out,
                                           float* tau_k_out, float* tau_v_out) {
  oscar_status st = check_shape(shape);
  if (st) return st;
  if (rotation != OSCAR_ROTATION_OSCAR && rotation != OSCAR_ROTATION_IDENTITY && rotation != OSCAR_ROTATION_HADAMARD)
    return fail(OSCAR_EINVAL, "rotation %d unknown", rotation);
  if (n < 1) return fail(OSCAR_EINVAL, "n = %lld calibration tokens", (long long)n);
  if (!q || !k || !v || !r_k_out || !r_v_out || !tau_k_out || !tau_v_out)
    return fail(OSCAR_EINVAL, "NULL calibration pointer");
  if (!(clip_pct_k > 0.0 && clip_pct_k <= 1.0) || !(clip_pct_v > 0.0 && clip_pct_v <= 1.0))
    return fail(OSCAR_EINVAL, "clip quantiles must lie in (0, 1]");
  const int d = kHeadDim, hkv = shape->n_kv_heads;
  if (rotation != OSCAR_ROTATION_OSCAR) {
    // the pages' baselines: no rotation, or the data-oblivious H P_br (the
    // composite with U = I); neither reads the covariances
    std::vector<double> r((size_t)d * d, 0.0), eye((size_t)d * d, 0.0);
    for (int i = 0; i < d; ++i) eye[(size_t)i * d + i] = 1.0;
    if (rotation == OSCAR_ROTATION_HADAMARD)
      composite_rotation(d, eye, r);
    else
      r = eye;
    for (int h = 0; h < hkv; ++h)
      for (size_t i = 0; i < (size_t)d * d; ++i) r_k_out[(size_t)h * d * d + i] = r_v_out[(size_t)h * d * d + i] = (float)r[i];
    for (double* e : {eig_k_out, eig_v_out})
      if (e)
        for (size_t i = 0; i < (size_t)hkv * d; ++i) e[i] = std::numeric_limits<double>::quiet_NaN();
  } else {
    std::vector<std::thread> pool;
    const unsigned hw = std::max(1u, std::thread::hardware_concurrency());
    for (int h0 = 0; h0 < hkv; h0 += (int)hw) {
      pool.clear();
      for (int h = h0; h < std::min(hkv, h0 + (int)hw); ++h)
        pool.emplace_back(calibrate_head, shape, n, q, k, v, h, r_k_out, r_v_out, eig_k_out, eig_v_out);
      for (auto& t : pool) t.join();
    }
  }
  // thresholds: quantile of |x R| over tokens, KV heads, channels (fp32 R)
  for (int which = 0; which < 2; ++which) {
    const float* x = which ? v : k;
    const float* r32 = which ? r_v_out : r_k_out;
    std::vector<double> vals((size_t)n * hkv * d);
    for (int h = 0; h < hkv; ++h) {
      const float* R = r32 + (size_t)h * d * d;
      for (int64_t t = 0; t < n; ++t) {
        const float* row = x + ((size_t)t * hkv + h) * d;
        double* out = &vals[((size_t)h * n + t) * d];
        for (int j = 0; j < d; ++j) out[j] = 0.0;
        for (int i = 0; i < d; ++i) {
          const double xi = row[i];
          const float* rr = R + (size_t)i * d;
          for (int j = 0; j < d; ++j) out[j] += xi * (double)rr[j];
        }
        for (int j = 0; j < d; ++j) out[j] = std::fabs(out[j]);
      }
    }
    const double tau = quantile_linear(vals, which ? clip_pct_v : clip_pct_k);
    *(which ? tau_v_out : tau_k_out) = (float)tau;
  }
  return ok();
}

oscar_status oscar_calibrate_host(const oscar_shape* shape, int64_t n, const float* q, const float* k,
                                  const float* v, double clip_pct_k, double clip_pct_v, float* r_k_out,
                                  float* r_v_out, double* eig_k_out, double* eig_v_out, float* tau_k_out,
                                  float* tau_v_out) {
  return oscar_calibrate_host_rotation(shape, OSCAR_ROTATION_OSCAR, n, q, k, v, clip_pct_k, clip_pct_v, r_k_out,
                                       r_v_out, eig_k_out, eig_v_out, tau_k_out, tau_v_out);
}

}  // extern "C"

// ----------------------------------------------------------------------------
// Pools and sequences (host bookkeeping)
// ----------------------------------------------------------------------------

struct oscar_pool {
  oscar_shape shape;
  std::vector<int32_t> ref[2];    // 0: INT2, 1: bf16
  std::vector<int32_t> free_[2];  // stacks of free page ids
};

struct oscar_seq {
  int64_t len = 0;
  std::vector<int32_t> int2;  // logical INT2 page -> physical (-1 = none)
  std::vector<int32_t> bf16;  // [sink pages][ring pages] -> physical (-1 = none)
};

namespace {

int sink_pages(const oscar_shape& s) { return (s.sink + kPage - 1) / kPage; }
int ring_pages(const oscar_shape& s) { return s.recent / kPage; }

// region of position p in a request of length t
enum { kSink = 0, kInt2 = 1, kRecent = 2 };
int region(const oscar_shape& s, int64_t p, int64_t t) {
  if (p < s.sink) return kSink;
  if (p >= t - s.recent) return kRecent;
  return kInt2;
}
int64_t bf16_logical_slot(const oscar_shape& s, int64_t p) {
  if (p < s.sink) return p;
  return (int64_t)sink_pages(s) * kPage + (p - s.sink) % s.recent;
}

int32_t alloc_page(oscar_pool* pool, int kind) {
  auto& fl = pool->free_[kind];
  const int32_t id = fl.back();
  fl.pop_back();
  pool->ref[kind][id] = 1;
  return id;
}

void drop_page(oscar_pool* pool, int kind, int32_t id) {
  if (id < 0) return;
  if (--pool->ref[kind][id] == 0) pool->free_[kind].push_back(id);
}

}  // namespace

extern "C" {

oscar_status oscar_pool_create(const oscar_shape* shape, int64_t n_int2_pages, int64_t n_bf16_pages,
                               oscar_pool** out) {
  oscar_status st = check_shape(shape);
  if (st) return st;
  if (!out) return fail(OSCAR_EINVAL, "out is NULL");
  if (n_int2_pages < 0 || n_bf16_pages < 0 || n_int2_pages > (1LL << 27) || n_bf16_pages > (1LL << 27))
    return fail(OSCAR_EINVAL, "page counts must lie in [0, 2^27]");
  oscar_pool* p = new (std::nothrow) oscar_pool;
  if (!p) return fail(OSCAR_ENOMEM, "host allocation failed");
  p->shape = *shape;
  for (int kind = 0; kind < 2; ++kind) {
    const int64_t n = kind ? n_bf16_pages : n_int2_pages;
    p->ref[kind].assign((size_t)n, 0);
    p->free_[kind].resize((size_t)n);
    for (int64_t i = 0; i < n; ++i) p->free_[kind][(size_t)i] = (int32_t)(n - 1 - i);  // pop order 0, 1, 2 ...
  }
  *out = p;
  return ok();
}

oscar_status oscar_pool_destroy(oscar_pool* pool) {
  delete pool;
  return ok();
}

oscar_status oscar_pool_free_pages(const oscar_pool* pool, int64_t* int2_free, int64_t* bf16_free) {
  if (!pool) return fail(OSCAR_EINVAL, "pool is NULL");
  if (int2_free) *int2_free = (int64_t)pool->free_[0].size();
  if (bf16_free) *bf16_free = (int64_t)pool->free_[1].size();
  return ok();
}

oscar_status oscar_seq_create(oscar_pool* pool, oscar_seq** out) {
  if (!pool || !out) return fail(OSCAR_EINVAL, "NULL argument");
  oscar_seq* s = new (std::nothrow) oscar_seq;
  if (!s) return fail(OSCAR_ENOMEM, "host allocation failed");
  s->bf16.assign((size_t)(sink_pages(pool->shape) + ring_pages(pool->shape)), -1);
  *out = s;
  return ok();
}

oscar_status oscar_seq_release(oscar_pool* pool, oscar_seq* seq) {
  if (!pool || !seq) return fail(OSCAR_EINVAL, "NULL argument");
  for (int32_t id : seq->int2) drop_page(pool, 0, id);
  for (int32_t id : seq->bf16) drop_page(pool, 1, id);
  delete seq;
  return ok();
}

int64_t oscar_seq_length(const oscar_seq* seq) { return seq ? seq->len : -1; }

oscar_status oscar_seq_plan_append(oscar_pool* pool, oscar_seq* seq, int64_t n_new, int32_t* int2_slots,
                                   int32_t* bf16_slots, int32_t* age_src, int32_t* age_dst, int64_t* n_age) {
  if (!pool || !seq || n_new < 0) return fail(OSCAR_EINVAL, "bad pool/seq/n_new");
  if (n_new > 0 && (!int2_slots || !bf16_slots)) return fail(OSCAR_EINVAL, "NULL slot array");
  if (!n_age) return fail(OSCAR_EINVAL, "n_age is NULL");
  const oscar_shape& sh = pool->shape;
  const int64_t t0 = seq->len, t1 = seq->len + n_new;
  if (t1 > (int64_t)std::numeric_limits<int32_t>::max() / 2) return fail(OSCAR_EINVAL, "sequence too long");
  // positions that age out of the recent window
  int64_t a0 = 0, a1 = 0;
  if (sh.recent > 0) {
    a0 = std::max<int64_t>(sh.sink, t0 - sh.recent);
    a1 = std::min<int64_t>(t0, t1 - sh.recent);
  }
  const int64_t n_age_out = std::max<int64_t>(0, a1 - a0);
  if (n_age_out > 0 && (!age_src || !age_dst)) return fail(OSCAR_EINVAL, "NULL age-out arrays");
  // pages needed
  std::vector<int64_t> need_int2, need_bf16;
  auto want_int2 = [&](int64_t p) {
    const int64_t lp = p / kPage;
    if (lp >= (int64_t)seq->int2.size() || seq->int2[(size_t)lp] < 0)
      if (need_int2.empty() || need_int2.back() != lp) need_int2.push_back(lp);
  };
  auto want_bf16 = [&](int64_t p) {
    const int64_t lp = bf16_logical_slot(sh, p) / kPage;
    if (seq->bf16[(size_t)lp] < 0 && std::find(need_bf16.begin(), need_bf16.end(), lp) == need_bf16.end())
      need_bf16.push_back(lp);
  };
  for (int64_t p = a0; p < a1; ++p) want_int2(p);
  for (int64_t p = t0; p < t1; ++p) {
    if (region(sh, p, t1) == kInt2)
      want_int2(p);
    else
      want_bf16(p);
  }
  std::sort(need_int2.begin(), need_int2.end());
  need_int2.erase(std::unique(need_int2.begin(), need_int2.end()), need_int2.end());
  if ((int64_t)need_int2.size() > (int64_t)pool->free_[0].size())
    return fail(OSCAR_ENOMEM, "INT2 pool exhausted (%zu pages needed, %zu free)", need_int2.size(),
                pool->free_[0].size());
  if ((int64_t)need_bf16.size() > (int64_t)pool->free_[1].size())
    return fail(OSCAR_ENOMEM, "bf16 pool exhausted (%zu pages needed, %zu free)", need_bf16.size(),
                pool->free_[1].size());
  for (int64_t lp : need_int2) {
    if (lp >= (int64_t)seq->int2.size()) seq->int2.resize((size_t)lp + 1, -1);
    seq->int2[(size_t)lp] = alloc_page(pool, 0);
  }
  for (int64_t lp : need_bf16) seq->bf16[(size_t)lp] = alloc_page(pool, 1);
  auto int2_phys = [&](int64_t p) { return seq->int2[(size_t)(p / kPage)] * kPage + (int32_t)(p % kPage); };
  auto bf16_phys = [&](int64_t p) {
    const int64_t ls = bf16_logical_slot(sh, p);
    return seq->bf16[(size_t)(ls / kPage)] * kPage + (int32_t)(ls % kPage);
  };
  for (int64_t p = a0; p < a1; ++p) {
    age_src[p - a0] = bf16_phys(p);
    age_dst[p - a0] = int2_phys(p);
  }
  *n_age = n_age_out;
  for (int64_t p = t0; p < t1; ++p) {
    if (region(sh, p, t1) == kInt2) {
      int2_slots[p - t0] = int2_phys(p);
      bf16_slots[p - t0] = -1;
    } else {
      int2_slots[p - t0] = -1;
      bf16_slots[p - t0] = bf16_phys(p);
    }
  }
  seq->len = t1;
  return ok();
}

oscar_status oscar_seq_fork(oscar_pool* pool, const oscar_seq* parent, oscar_seq** child, int32_t* copy_src,
                            int32_t* copy_dst, int32_t* copy_kind, int64_t* n_copies) {
  if (!pool || !parent || !child || !n_copies) return fail(OSCAR_EINVAL, "NULL argument");
  const oscar_shape& sh = pool->shape;
  const int64_t t = parent->len;
  // first position that can still be written into INT2 storage
  const int64_t first_write = std::max<int64_t>(sh.sink, sh.recent > 0 ? t - sh.recent : t);
  std::vector<int> copy_int2, copy_bf16;
  for (size_t lp = 0; lp < parent->int2.size(); ++lp)
    if (parent->int2[lp] >= 0 && (int64_t)(lp * kPage + kPage - 1) >= first_write) copy_int2.push_back((int)lp);
  const int sp = sink_pages(sh);
  for (size_t lp = 0; lp < parent->bf16.size(); ++lp) {
    if (parent->bf16[lp] < 0) continue;
    const bool ring = (int)lp >= sp;
    const bool sink_open = !ring && t < sh.sink;
    if (ring || sink_open) copy_bf16.push_back((int)lp);
  }
  const size_t nc = copy_int2.size() + copy_bf16.size();
  if (nc > 0 && (!copy_src || !copy_dst || !copy_kind)) return fail(OSCAR_EINVAL, "NULL copy arrays");
  if (copy_int2.size() > pool->free_[0].size() || copy_bf16.size() > pool->free_[1].size())
    return fail(OSCAR_ENOMEM, "pool exhausted while forking");
  oscar_seq* c = new (std::nothrow) oscar_seq;
  if (!c) return fail(OSCAR_ENOMEM, "host allocation failed");
  c->len = t;
  c->int2 = parent->int2;
  c->bf16 = parent->bf16;
  size_t k = 0;
  for (int lp : copy_int2) {
    const int32_t id = alloc_page(pool, 0);
    copy_src[k] = parent->int2[(size_t)lp];
    copy_dst[k] = id;
    copy_kind[k++] = 0;
    c->int2[(size_t)lp] = id;
  }
  for (int lp : copy_bf16) {
    const int32_t id = alloc_page(pool, 1);
    copy_src[k] = parent->bf16[(size_t)lp];
    copy_dst[k] = id;
    copy_kind[k++] = 1;
    c->bf16[(size_t)lp] = id;
  }
  for (size_t lp = 0; lp < c->int2.size(); ++lp)
    if (c->int2[lp] >= 0 && c->int2[lp] == parent->int2[lp]) ++pool->ref[0][(size_t)c->int2[lp]];
  for (size_t lp = 0; lp < c->bf16.size(); ++lp)
    if (c->bf16[lp] >= 0 && c->bf16[lp] == parent->bf16[lp]) ++pool->ref[1][(size_t)c->bf16[lp]];
  *n_copies = (int64_t)nc;
  *child = c;
  return ok();
}

oscar_status oscar_block_tables(const oscar_pool* pool, const oscar_seq* const* seqs, int32_t n, int32_t* int2_bt,
                                int32_t max_int2_pages, int32_t* bf16_bt, int32_t max_bf16_pages,
                                int32_t* ctx_lens) {
  if (!pool || (n > 0 && (!seqs || !ctx_lens))) return fail(OSCAR_EINVAL, "NULL argument");
  if (n < 0 || max_int2_pages < 0 || max_bf16_pages < 0) return fail(OSCAR_EINVAL, "negative size");
  for (int32_t i = 0; i < n; ++i) {
    const oscar_seq* s = seqs[i];
    if (!s) return fail(OSCAR_EINVAL, "sequence %d is NULL", i);
    if ((int64_t)s->int2.size() > max_int2_pages)
      return fail(OSCAR_EINVAL, "sequence %d needs %zu INT2 pages > row width %d", i, s->int2.size(), max_int2_pages);
    if ((int64_t)s->bf16.size() > max_bf16_pages)
      return fail(OSCAR_EINVAL, "sequence %d needs %zu bf16 pages > row width %d", i, s->bf16.size(), max_bf16_pages);
    if (int2_bt)
      for (int32_t j = 0; j < max_int2_pages; ++j)
        int2_bt[(int64_t)i * max_int2_pages + j] = j < (int32_t)s->int2.size() ? s->int2[(size_t)j] : -1;
    if (bf16_bt)
      for (int32_t j = 0; j < max_bf16_pages; ++j)
        bf16_bt[(int64_t)i * max_bf16_pages + j] = j < (int32_t)s->bf16.size() ? s->bf16[(size_t)j] : -1;
    ctx_lens[i] = (int32_t)s->len;
  }
  return ok();
}

oscar_status oscar_plan_decode_step(oscar_pool* pool, oscar_seq* const* seqs, int32_t n, int32_t* int2_slots,
                                    int32_t* bf16_slots, int32_t* age_src, int32_t* age_dst, int32_t* n_age,
                                    int32_t* ctx_lens, int32_t* tables_changed) {
  if (!pool || n < 0 || (n > 0 && (!seqs || !int2_slots || !bf16_slots || !age_src || !age_dst || !ctx_lens)) ||
      !n_age || !tables_changed)
    return fail(OSCAR_EINVAL, "NULL argument");
  const oscar_shape& sh = pool->shape;
  // page needs first, so that exhaustion changes nothing
  int64_t need[2] = {0, 0};
  for (int32_t i = 0; i < n; ++i) {
    const oscar_seq* s = seqs[i];
    if (!s) return fail(OSCAR_EINVAL, "sequence %d is NULL", i);
    const int64_t t0 = s->len, t1 = t0 + 1;
    if (sh.recent > 0 && t0 - sh.recent >= sh.sink) {
      const int64_t p = t0 - sh.recent;  // leaves the window
      const int64_t lp = p / kPage;
      if (lp >= (int64_t)s->int2.size() || s->int2[(size_t)lp] < 0) ++need[0];
    }
    if (region(sh, t0, t1) == kInt2) {
      const int64_t lp = t0 / kPage;
      if (lp >= (int64_t)s->int2.size() || s->int2[(size_t)lp] < 0) ++need[0];
    } else {
      const int64_t lp = bf16_logical_slot(sh, t0) / kPage;
      if (s->bf16[(size_t)lp] < 0) ++need[1];
    }
  }
  if (need[0] > (int64_t)pool->free_[0].size() || need[1] > (int64_t)pool->free_[1].size())
    return fail(OSCAR_ENOMEM, "pool exhausted in decode step");
  int32_t na = 0;
  *tables_changed = (need[0] + need[1]) > 0;
  for (int32_t i = 0; i < n; ++i) {
    int64_t n_age_i = 0;
    int32_t src = -1, dst = -1;
    oscar_status st = oscar_seq_plan_append(pool, seqs[i], 1, &int2_slots[i], &bf16_slots[i], &src, &dst, &n_age_i);
    if (st) return st;
    age_src[i] = n_age_i ? src : -1;
    age_dst[i] = n_age_i ? dst : -1;
    na += n_age_i ? 1 : 0;
    ctx_lens[i] = (int32_t)seqs[i]->len;
  }
  *n_age = na;
  return ok();
}

// ----------------------------------------------------------------------------
// Launches
// ----------------------------------------------------------------------------

static oscar_status check_cache(const oscar_cache* c, bool need_int2, bool need_bf16) {
  if (!c) return fail(OSCAR_EINVAL, "cache is NULL");
  if (need_int2 && (!c->int2_pages || c->n_int2_pages < 1 || !aligned(c->int2_pages, 256)))
    return fail(OSCAR_EINVAL, "INT2 storage missing or not 256-byte aligned");
  if (need_bf16 && (!c->bf16_pages || c->n_bf16_pages < 1 || !aligned(c->bf16_pages, 256)))
    return fail(OSCAR_EINVAL, "bf16 storage missing or not 256-byte aligned");
  return OSCAR_OK;
}

// The clip thresholds must be finite and >= 0.  With fp16 scale and zero they
// must also be at most 65504, the largest finite fp16: every clipped value then
// has |x| <= 65504, so z = fp16(mn) and s = fp16((mx - mn) / 3) are finite and
// every code (x - z) / s is a finite number before its clamp to 0..3.  (FP8
// scale and zero saturate at 448 instead of overflowing.)
static oscar_status check_layer(const oscar_layer* l, const oscar_shape* shape) {
  if (!l || !l->r_k) return fail(OSCAR_EINVAL, "layer rotation R_K missing");
  if (!aligned(l->r_k, 16) || (l->r_v && !aligned(l->r_v, 16)))
    return fail(OSCAR_EINVAL, "rotations must be 16-byte aligned");
  if (l->r_prep && !aligned(l->r_prep, 256)) return fail(OSCAR_EINVAL, "prepared digits must be 256-byte aligned");
  if (!std::isfinite(l->tau_k) || !std::isfinite(l->tau_v) || l->tau_k < 0 || l->tau_v < 0)
    return fail(OSCAR_EINVAL, "clip thresholds must be finite and >= 0");
  if (mb_of(shape) == 4 && (l->tau_k > 65504.f || l->tau_v > 65504.f))
    return fail(OSCAR_EINVAL, "clip thresholds above 65504 would overflow the fp16 scale and zero");
  return OSCAR_OK;
}

oscar_status oscar_quant_write(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                               const void* k_bf16, const void* v_bf16, const int32_t* int2_slots, int64_t n,
                               void* stream) {
  oscar_status st = check_shape(shape);
  if (st) return st;
  if (n < 0) return fail(OSCAR_EINVAL, "n < 0");
  if (n == 0) return ok();
  if ((st = check_layer(layer, shape)) || (st = check_cache(cache, true, false))) return st;
  if (!k_bf16 || !v_bf16 || !int2_slots) return fail(OSCAR_EINVAL, "NULL input");
  if (!aligned(k_bf16, 16) || !aligned(v_bf16, 16)) return fail(OSCAR_EINVAL, "inputs must be 16-byte aligned");
  if (n > (1LL << 31) / 16) return fail(OSCAR_EINVAL, "n too large");
  QuantParams p{};
  p.k_src = (const uint16_t*)k_bf16;
  p.v_src = (const uint16_t*)v_bf16;
  p.dst_slots = int2_slots;
  p.int2_pages = (uint8_t*)cache->int2_pages;
  p.n_int2_pages = cache->n_int2_pages;
  p.r_k = layer->r_k;
  p.r_v = layer->r_v;
  p.tau_k = layer->tau_k;
  p.tau_v = layer->tau_v;
  p.n = n;
  p.n_kv = shape->n_kv_heads;
  p.group = shape->group;
  p.mb = mb_of(shape);
  p.r_prep = (const uint8_t*)layer->r_prep;
  return hip_status(launch_quant_write(p, 0, (hipStream_t)stream), "quant_write launch");
}

size_t oscar_layer_prep_bytes(const oscar_shape* shape) {
  if (check_shape(shape) != OSCAR_OK) return 0;
  return (size_t)shape->n_kv_heads * 2 * kRPrepBytes;
}

oscar_status oscar_layer_prepare(const oscar_shape* shape, const oscar_layer* layer, void* prep, size_t prep_bytes,
                                 void* stream) {
  oscar_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_layer(layer, shape))) return st;
  if (!prep || !aligned(prep, 256)) return fail(OSCAR_EINVAL, "prep must be a 256-byte aligned device buffer");
  if (prep_bytes < oscar_layer_prep_bytes(shape))
    return fail(OSCAR_EINVAL, "prep %zu bytes < %zu needed", prep_bytes, oscar_layer_prep_bytes(shape));
  return hip_status(launch_prepare_r(layer->r_k, layer->r_v, shape->n_kv_heads, (uint8_t*)prep, (hipStream_t)stream),
                    "prepare launch");
}

oscar_status oscar_requant_from_bf16(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                                     const int32_t* src_bf16_slots, const int32_t* dst_int2_slots, int64_t n,
                                     void* stream) {
  oscar_status st = check_shape(shape);
  if (st) return st;
  if (n < 0) return fail(OSCAR_EINVAL, "n < 0");
  if (n == 0) return ok();
  if ((st = check_layer(layer, shape)) || (st = check_cache(cache, true, true))) return st;
  if (!src_bf16_slots || !dst_int2_slots) return fail(OSCAR_EINVAL, "NULL slot array");
  QuantParams p{};
  p.bf16_pages = (const uint8_t*)cache->bf16_pages;
  p.n_bf16_pages = cache->n_bf16_pages;
  p.src_slots = src_bf16_slots;
  p.dst_slots = dst_int2_slots;
  p.int2_pages = (uint8_t*)cache->int2_pages;
  p.n_int2_pages = cache->n_int2_pages;
  p.r_k = layer->r_k;
  p.r_v = layer->r_v;
  p.tau_k = layer->tau_k;
  p.tau_v = layer->tau_v;
  p.n = n;
  p.n_kv = shape->n_kv_heads;
  p.group = shape->group;
  p.mb = mb_of(shape);
  p.r_prep = (const uint8_t*)layer->r_prep;
  return hip_status(launch_quant_write(p, 1, (hipStream_t)stream), "requant launch");
}

oscar_status oscar_bf16_write(const oscar_shape* shape, const oscar_cache* cache, const void* k_bf16,
                              const void* v_bf16, const int32_t* bf16_slots, int64_t n, void* stream) {
  oscar_status st = check_shape(shape);
  if (st) return st;
  if (n < 0) return fail(OSCAR_EINVAL, "n < 0");
  if (n == 0) return ok();
  if ((st = check_cache(cache, false, true))) return st;
  if (!k_bf16 || !v_bf16 || !bf16_slots) return fail(OSCAR_EINVAL, "NULL input");
  if (!aligned(k_bf16, 4) || !aligned(v_bf16, 4)) return fail(OSCAR_EINVAL, "inputs must be 4-byte aligned");
  if (n > (1LL << 31)) return fail(OSCAR_EINVAL, "n too large");
  return hip_status(launch_bf16_write((const uint16_t*)k_bf16, (const uint16_t*)v_bf16, bf16_slots, n,
                                      shape->n_kv_heads, (uint8_t*)cache->bf16_pages, cache->n_bf16_pages,
                                      (hipStream_t)stream),
                    "bf16_write launch");
}

oscar_status oscar_copy_pages(const oscar_shape* shape, const oscar_cache* cache, int32_t kind,
                              const int32_t* src_pages, const int32_t* dst_pages, int64_t n, void* stream) {
  oscar_status st = check_shape(shape);
  if (st) return st;
  if (kind != 0 && kind != 1) return fail(OSCAR_EINVAL, "kind must be 0 or 1");
  if (n < 0) return fail(OSCAR_EINVAL, "n < 0");
  if (n == 0) return ok();
  if ((st = check_cache(cache, kind == 0, kind == 1))) return st;
  if (!src_pages || !dst_pages) return fail(OSCAR_EINVAL, "NULL page arrays");
  const int64_t blk = kind == 0 ? int2_block(shape) : kBf16BlockBytes;
  return hip_status(launch_copy_pages((uint8_t*)(kind == 0 ? cache->int2_pages : cache->bf16_pages),
                                      blk * shape->n_kv_heads, kind == 0 ? cache->n_int2_pages : cache->n_bf16_pages,
                                      src_pages, dst_pages, n, (hipStream_t)stream),
                    "copy_pages launch");
}

static const int kAutoMaxSplits = 64;         // chunked prefill
static const int kAutoMaxSplitsDecode = 128;  // decode

// compute units of the current device (256 on MI355X; also the answer when no
// device can be queried, so the choice below is deterministic on a host)
static int device_cus() {
  static int cached = 0;
  if (cached > 0) return cached;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      n > 0)
    cached = n;
  else
    cached = 256;
  (void)hipGetLastError();
  return cached;
}

// 0 automatic, 1 never, 2 wherever the tile split allows (oscar_decode_set_small_grid)
static std::atomic<int> g_small_grid_mode{0};

int32_t oscar_decode_set_small_grid(int32_t mode) {
  if (mode < 0 || mode > 2) return -1;
  return g_small_grid_mode.exchange(mode);
}

// The small-grid form's INT2 kernel holds the bf16 item's registers: two
// wavefronts per SIMD.  Its grid (INT2 items and bf16 splits) must fit that.
static int64_t small_grid_waves() { return 8 * (int64_t)device_cus(); }
// fewest splits worth lowering the count to for that form (32K-token requests,
// 8 KV heads: 8 requests at 28 splits 64.5 against 72.5 us a step in the
// standard form at 128; 16 requests at 12 splits 115.5 against 103.8 at 64)
static const int kSmallGridMinSplits = 24;
// Long requests take the whole fit (every SIMD two wavefronts) when each of
// its splits keeps this many pages (one request of 100K tokens, 8 KV heads:
// 252 splits of 24.8 pages, 39.0 against 42.5 us a step at 128).  A count
// between the two leaves some SIMDs one wavefront and others two, and the
// latter end the launch (64K tokens: 170 splits 36.1 against 35.3 us at 128).
static const int kSmallGridPagesPerSplit = 24;

// Automatic split count for a decode with sb bf16 splits (sb < 0: the
// all-bf16 baseline, whose splits never take the small-grid form).
static int32_t decode_auto_splits(const oscar_shape* shape, int32_t batch, int32_t max_int2_pages, int sb) {
  if (check_shape(shape) != OSCAR_OK || batch < 1) return 1;
  // Work items run in rounds of the items that fit the device at once (4
  // SIMDs per compute unit, waves_per_simd(ct) wavefronts per SIMD, whole
  // items of w wavefronts each: tile_split; three-wavefront items fit five to
  // a compute unit, not 16/3).  A count just above a whole number of rounds leaves a
  // nearly empty last round that costs a full item time.  Take the count that
  // fills two whole rounds (some slack for uneven requests, few partial
  // results), within [1, 128] and at least 16 pages per split.  Small batches
  // reach the bounds: at one request of 32K tokens (8 KV heads) 128 splits
  // measured fastest in the standard form (64: 43.5 us a step, 128: 40.0,
  // 256: 44.6, the combine's merge growing with the split count).
  const int64_t pairs = (int64_t)batch * shape->n_kv_heads;
  const TileSplit ts = tile_split(ct_of(shape));
  const int64_t cap = (int64_t)device_cus() * ((4 * waves_per_simd(ts.ct)) / ts.w);
  const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(kAutoMaxSplitsDecode, max_int2_pages / 16));
  int64_t s = std::max<int64_t>(1, std::min<int64_t>(2 * cap / pairs, smax));
  // Small grids (oscar_decode_set_small_grid not 1, one-wavefront items): the
  // count that fits the small-grid form's two wavefronts per SIMD, when that
  // leaves at least kSmallGridMinSplits (2, 4 and 8 requests of 32K tokens at
  // 8 KV heads: 124, 60 and 28 splits, 11-15 % shorter steps than the standard
  // form at 128); long requests take the whole fit, past 128, when each of its
  // splits keeps kSmallGridPagesPerSplit pages
  if (sb >= 0 && g_small_grid_mode.load() != 1 && ts.w == 1) {
    const int64_t fit = small_grid_waves() / pairs - sb;
    if (fit >= kSmallGridMinSplits) {
      s = std::min(s, fit);
      if (max_int2_pages / fit >= kSmallGridPagesPerSplit) s = fit;
    }
  }
  return (int32_t)s;
}

// The most INT2 splits the automatic count can take for this batch (at least
// one bf16 split beside them).
static int64_t decode_auto_splits_max(const oscar_shape* shape, int32_t batch) {
  int64_t m = kAutoMaxSplitsDecode;
  if (check_shape(shape) == OSCAR_OK && g_small_grid_mode.load() != 1 && tile_split(ct_of(shape)).w == 1) {
    const int64_t pairs = (int64_t)std::max<int32_t>(batch, 1) * shape->n_kv_heads;
    m = std::max<int64_t>(m, small_grid_waves() / pairs - 1);
  }
  return m;
}

int32_t oscar_decode_auto_splits(const oscar_shape* shape, int32_t batch, int32_t max_int2_pages) {
  return decode_auto_splits(shape, batch, max_int2_pages, 4);
}

size_t oscar_decode_workspace_bytes(const oscar_shape* shape, int32_t batch, int32_t splits_int2,
                                    int32_t splits_bf16) {
  if (check_shape(shape) != OSCAR_OK || batch < 0 || splits_int2 < 0 || splits_bf16 < 0) return 0;
  const int64_t si = splits_int2 == 0 ? decode_auto_splits_max(shape, batch) : splits_int2;
  const int sb = splits_bf16 == 0 ? kAutoMaxSplitsDecode : splits_bf16;
  return decode_workspace_bytes(batch, shape->n_q_heads, shape->n_kv_heads, ct_of(shape), (int)(si + sb));
}

struct StepWrites {
  const void* k_new;
  const void* v_new;
  const int32_t* step_slots;
  bool host_tables;  // step_slots and ctx_lens in host memory: copied into the launch arguments
};

// The split-K workspace of a decode launch: caller memory, or (use_scratch)
// the library's own device array, whose address is looked up once per device.
struct DecodeWorkspace {
  void* ptr;
  size_t bytes;
  bool use_scratch;
};

static oscar_status decode_common(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                                  const void* q, int32_t batch, const int32_t* int2_bt, int32_t max_int2_pages,
                                  const int32_t* bf16_bt, int32_t max_bf16_pages, const int32_t* ctx_lens,
                                  int32_t splits_int2, int32_t splits_bf16, float* out, DecodeWorkspace ws,
                                  void* stream, bool baseline, const StepWrites* writes = nullptr) {
  oscar_status st = check_shape(shape);
  if (st) return st;
  if (batch < 0) return fail(OSCAR_EINVAL, "batch < 0");
  if (batch == 0) return ok();
  if (!q || !ctx_lens || !out || (!ws.use_scratch && !ws.ptr)) return fail(OSCAR_EINVAL, "NULL argument");
  if (!aligned(q, 16) || !aligned(out, 16) || (!ws.use_scratch && !aligned(ws.ptr, 256)))
    return fail(OSCAR_EINVAL, "q/out must be 16-byte and workspace 256-byte aligned");
  if (!bf16_bt || max_bf16_pages < 1) return fail(OSCAR_EINVAL, "bf16 block table missing");
  if (!baseline) {
    if ((st = check_layer(layer, shape)) || (st = check_cache(cache, true, true))) return st;
    if (!int2_bt || max_int2_pages < 1) return fail(OSCAR_EINVAL, "INT2 block table missing");
  } else {
    if ((st = check_cache(cache, false, true))) return st;
  }
  if (splits_int2 < 0 || splits_bf16 < 0 || splits_int2 > 4096 || splits_bf16 > 4096)
    return fail(OSCAR_EINVAL, "splits out of range");
  DecodeParams p{};
  p.int2_pages = baseline ? nullptr : (const uint8_t*)cache->int2_pages;
  p.n_int2_pages = baseline ? 0 : cache->n_int2_pages;
  p.bf16_pages = (const uint8_t*)cache->bf16_pages;
  p.n_bf16_pages = cache->n_bf16_pages;
  p.q = (const uint16_t*)q;
  p.r_k = baseline ? nullptr : layer->r_k;
  p.r_v = baseline ? nullptr : layer->r_v;
  p.int2_bt = int2_bt;
  p.max_int2_pages = max_int2_pages;
  p.bf16_bt = bf16_bt;
  p.max_bf16_pages = max_bf16_pages;
  p.ctx_lens = ctx_lens;
  p.batch = batch;
  p.n_q = shape->n_q_heads;
  p.n_kv = shape->n_kv_heads;
  p.g = p.n_q / p.n_kv;
  p.ng = baseline ? 4 : ng_of(shape);
  p.ct = baseline ? 1 : ct_of(shape);
  p.mb = mb_of(shape);
  p.q_heads = p.n_q;
  p.g_real = p.g;
  p.chunk = 1;
  p.chunk0 = 0;
  if (baseline) {
    p.sink = 1 << 28;
    p.recent = 0;
    p.splits_int2 = 0;
    p.splits_bf16 = splits_bf16 ? splits_bf16 : decode_auto_splits(shape, batch, max_bf16_pages, -1);
  } else {
    p.sink = shape->sink;
    p.recent = shape->recent;
    // up to four bf16 splits run inside the combine kernel (one per wavefront);
    // the bf16 region is at most sink + recent tokens
    p.splits_bf16 = splits_bf16 ? splits_bf16 : 4;
    p.bf16_in_combine = p.splits_bf16 <= 4;
    p.splits_int2 = splits_int2 ? splits_int2 : decode_auto_splits(shape, batch, max_int2_pages, p.splits_bf16);
    // Small grids: the bf16 splits join the INT2 kernel's launch and the
    // combine takes a work group per query head (one request: the standard
    // form runs eight work groups of dependent loads on 256 compute units).
    // The INT2 kernel then holds the bf16 item's registers (two wavefronts per
    // SIMD), so its grid must fit that; its items must be one wavefront.
    const int mode = g_small_grid_mode.load();
    const int64_t waves = (int64_t)batch * p.n_kv * (p.splits_int2 + p.splits_bf16);
    p.small_grid = batch > 0 && tile_split(p.ct).w == 1 && mode != 1 && (mode == 2 || waves <= small_grid_waves());
    if (p.small_grid) p.bf16_in_combine = 0;
    // P' = p s 2^sp stays below 2^15: s <= 2 tau_v / 3 (rounded to fp16), p <= 1
    const double smax = 2.0 * (double)layer->tau_v / 3.0;
    p.p_scale_exp = 0.f;
    if (std::isfinite(smax) && smax > 0) p.p_scale_exp = (float)std::clamp((int)std::floor(std::log2(32768.0 / smax)) - 1, -60, 60);
  }
  const size_t need = decode_workspace_bytes(batch, p.n_q, p.n_kv, p.ct, p.splits_int2 + p.splits_bf16);
  if (ws.use_scratch) {
    if (need > kDecodeScratchBytes)
      return fail(OSCAR_EINVAL,
                  "this decode needs %zu bytes of split-K workspace, more than the %zu bytes the allocation-free "
                  "entry point holds: use fewer splits, a smaller batch, or oscar_decode_attn with a workspace",
                  need, kDecodeScratchBytes);
    if ((st = hip_status(decode_scratch((hipStream_t)stream, &ws.ptr, &ws.bytes), "scratch address lookup")))
      return st;
  }
  if (ws.bytes < need) return fail(OSCAR_EINVAL, "workspace %zu bytes < %zu needed", ws.bytes, need);
  decode_workspace_carve(p, ws.ptr);
  p.out = out;
  ArgTables tabs{};
  if (writes) {
    p.has_step = 1;
    p.step_slots = writes->step_slots;
    if (writes->host_tables) {
      // the host arrays go into the prologue's launch arguments; the prologue
      // copies the lengths to the workspace, where the later kernels read them
      for (int r = 0; r < 4; ++r)
        std::copy(writes->step_slots + (int64_t)r * batch, writes->step_slots + (int64_t)(r + 1) * batch,
                  tabs.v[r]);
      std::copy(ctx_lens, ctx_lens + batch, tabs.v[4]);
      p.arg_tables = 1;
      p.step_slots = nullptr;
      p.ctx_lens = p.ctx_w;
    }
    p.k_new = (const uint16_t*)writes->k_new;
    p.v_new = (const uint16_t*)writes->v_new;
    p.int2_w = (uint8_t*)cache->int2_pages;
    p.bf16_w = (uint8_t*)cache->bf16_pages;
    p.tau_k = layer->tau_k;
    p.tau_v = layer->tau_v;
    // The prologue holds R_K and R_V in LDS (one work group per compute unit):
    // when twice the (request, KV head) count still fits one round, the writes
    // take work groups of their own beside the q operands; when three times
    // does, one per matrix (K, V), each staging only its own R.
    const int64_t pairs = (int64_t)p.batch * p.n_kv;
    p.split_writes = 3 * pairs <= device_cus() ? 2 : (2 * pairs <= device_cus() ? 1 : 0);
  }
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (g_prof.on && !ws.use_scratch) {
    std::tie(ev0, ev1) = g_prof.acquire();
    if (!ev0) return fail(OSCAR_EHIP, "hipEventCreate failed");
  }
  return hip_status(launch_decode(p, (hipStream_t)stream, ev0, ev1, p.arg_tables ? &tabs : nullptr), "decode launch");
}

oscar_status oscar_decode_step(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                               const void* k_new, const void* v_new, const int32_t* step_slots, const void* q,
                               int32_t batch, const int32_t* int2_bt, int32_t max_int2_pages,
                               const int32_t* bf16_bt, int32_t max_bf16_pages, const int32_t* ctx_lens,
                               int32_t splits_int2, int32_t splits_bf16, float* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (batch > 0 && (!k_new || !v_new || !step_slots)) return fail(OSCAR_EINVAL, "NULL step input");
  if (!aligned(k_new, 2) || !aligned(v_new, 2) || !aligned(step_slots, 4))
    return fail(OSCAR_EINVAL, "step inputs misaligned");
  const StepWrites w{k_new, v_new, step_slots, false};
  return decode_common(shape, layer, cache, q, batch, int2_bt, max_int2_pages, bf16_bt, max_bf16_pages, ctx_lens,
                       splits_int2, splits_bf16, out, DecodeWorkspace{workspace, workspace_bytes, false}, stream,
                       false, &w);
}

oscar_status oscar_decode_step_host_tables(const oscar_shape* shape, const oscar_layer* layer,
                                           const oscar_cache* cache, const void* k_new, const void* v_new,
                                           const int32_t* step_slots, const void* q, int32_t batch,
                                           const int32_t* int2_bt, int32_t max_int2_pages, const int32_t* bf16_bt,
                                           int32_t max_bf16_pages, const int32_t* ctx_lens, int32_t splits_int2,
                                           int32_t splits_bf16, float* out, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (batch > kArgBatch)
    return fail(OSCAR_EINVAL, "batch %d > %d: the step tables of oscar_decode_step_host_tables travel in the "
                              "launch arguments; use oscar_decode_step with device tables",
                batch, kArgBatch);
  if (batch > 0 && (!k_new || !v_new || !step_slots || !ctx_lens)) return fail(OSCAR_EINVAL, "NULL step input");
  if (!aligned(k_new, 2) || !aligned(v_new, 2)) return fail(OSCAR_EINVAL, "step inputs misaligned");
  const StepWrites w{k_new, v_new, step_slots, true};
  return decode_common(shape, layer, cache, q, batch, int2_bt, max_int2_pages, bf16_bt, max_bf16_pages, ctx_lens,
                       splits_int2, splits_bf16, out, DecodeWorkspace{workspace, workspace_bytes, false}, stream,
                       false, &w);
}


oscar_status oscar_decode_attn(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                               const void* q, int32_t batch, const int32_t* int2_bt, int32_t max_int2_pages,
                               const int32_t* bf16_bt, int32_t max_bf16_pages, const int32_t* ctx_lens,
                               int32_t splits_int2, int32_t splits_bf16, float* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return decode_common(shape, layer, cache, q, batch, int2_bt, max_int2_pages, bf16_bt, max_bf16_pages, ctx_lens,
                       splits_int2, splits_bf16, out, DecodeWorkspace{workspace, workspace_bytes, false}, stream,
                       false);
}

oscar_status oscar_decode_attn_noalloc(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                                       const void* q, int32_t batch, const int32_t* int2_bt, int32_t max_int2_pages,
                                       const int32_t* bf16_bt, int32_t max_bf16_pages, const int32_t* ctx_lens,
                                       int32_t splits_int2, int32_t splits_bf16, float* out, void* stream) {
  return decode_common(shape, layer, cache, q, batch, int2_bt, max_int2_pages, bf16_bt, max_bf16_pages, ctx_lens,
                       splits_int2, splits_bf16, out, DecodeWorkspace{nullptr, 0, true}, stream, false);
}

size_t oscar_decode_noalloc_max_workspace_bytes(void) { return kDecodeScratchBytes; }

// Chunked prefill: queries per launch so that the kernel heads (queries x
// model heads, at most 64: the prologue's capacity) fill at most 16 tiles of
// 16 (head, group) rows; tiles per launch rounded up to 4, 8 or 16 wavefronts.
static int prefill_block(const oscar_shape* shape) {
  const int g = shape->n_q_heads / shape->n_kv_heads;
  return std::max(1, std::min(256 / (g * ng_of(shape)), 64 / g));
}
static int prefill_tiles(const oscar_shape* shape, int queries) {
  const int g = shape->n_q_heads / shape->n_kv_heads;
  const int tiles = (queries * g * ng_of(shape) + 15) / 16;
  return tiles <= 4 ? 4 : (tiles <= 8 ? 8 : 16);
}
static int32_t prefill_auto_splits(const oscar_shape* shape, int32_t batch, int32_t max_int2_pages, int tiles) {
  // Items run in rounds of `cap` items: at 64-channel groups an item is
  // `tiles` wavefronts (4 per SIMD), at 32-channel groups tiles / 4 wide
  // wavefronts (four tiles each, 2 per SIMD).  A pass is long, so a part-empty
  // last round costs its whole share: take the fewest splits whose last round
  // is at least 15/16 full, else the count that fills it best (28 x 8 pairs on
  // 256 compute units, G = 32: 9 splits fill 2016 of 4 x 512).
  const int64_t pairs = (int64_t)batch * shape->n_kv_heads;
  const int per_cu = ng_of(shape) == 4 ? 4 * 2 * 4 : 4 * 4;  // tile slots per compute unit
  const int64_t cap = std::max<int64_t>(1, (int64_t)device_cus() * per_cu / tiles);
  const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(kAutoMaxSplits, max_int2_pages / 32));
  int64_t best = 1;
  double best_fill = 0.0;
  for (int64_t sp = 1; sp <= smax; ++sp) {
    const int64_t n = pairs * sp, rounds = (n + cap - 1) / cap;
    const double fill = (double)n / (double)(rounds * cap);
    if (fill >= 15.0 / 16.0) return (int32_t)sp;
    if (fill > best_fill + 1e-12) {
      best = sp;
      best_fill = fill;
    }
  }
  return (int32_t)best;
}

int32_t oscar_prefill_auto_splits(const oscar_shape* shape, int32_t batch, int32_t max_int2_pages, int32_t chunk) {
  if (check_shape(shape) != OSCAR_OK || batch < 1 || chunk < 1) return 1;
  return prefill_auto_splits(shape, batch, max_int2_pages, prefill_tiles(shape, std::min(chunk, prefill_block(shape))));
}

size_t oscar_prefill_workspace_bytes(const oscar_shape* shape, int32_t batch, int32_t chunk, int32_t splits_int2,
                                     int32_t splits_bf16) {
  if (check_shape(shape) != OSCAR_OK || batch < 0 || chunk < 1 || splits_int2 < 0 || splits_bf16 < 0) return 0;
  const int qn = std::min<int>(chunk, prefill_block(shape));
  const int g = shape->n_q_heads / shape->n_kv_heads;
  const int si = splits_int2 == 0 ? kAutoMaxSplits : splits_int2;
  const int sb = splits_bf16 == 0 ? 1 : splits_bf16;
  return decode_workspace_bytes(batch, shape->n_kv_heads * qn * g, shape->n_kv_heads, prefill_tiles(shape, qn),
                                si + sb);
}

oscar_status oscar_prefill_attn(const oscar_shape* shape, const oscar_layer* layer, const oscar_cache* cache,
                                const void* q, int32_t batch, int32_t chunk, const int32_t* int2_bt,
                                int32_t max_int2_pages, const int32_t* bf16_bt, int32_t max_bf16_pages,
                                const int32_t* ctx_lens, int32_t splits_int2, int32_t splits_bf16, float* out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  oscar_status st = check_shape(shape);
  if (st) return st;
  if (batch < 0 || chunk < 1) return fail(OSCAR_EINVAL, "batch < 0 or chunk < 1");
  if (batch == 0) return ok();
  if (!q || !ctx_lens || !out || !workspace) return fail(OSCAR_EINVAL, "NULL argument");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(workspace, 256))
    return fail(OSCAR_EINVAL, "q/out must be 16-byte and workspace 256-byte aligned");
  if ((st = check_layer(layer, shape)) || (st = check_cache(cache, true, true))) return st;
  if (!int2_bt || max_int2_pages < 1 || !bf16_bt || max_bf16_pages < 1)
    return fail(OSCAR_EINVAL, "block tables missing");
  if (splits_int2 < 0 || splits_bf16 < 0 || splits_int2 > 4096 || splits_bf16 > 4096)
    return fail(OSCAR_EINVAL, "splits out of range");
  const size_t need = oscar_prefill_workspace_bytes(shape, batch, chunk, splits_int2, splits_bf16);
  if (workspace_bytes < need) return fail(OSCAR_EINVAL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  const int g = shape->n_q_heads / shape->n_kv_heads;
  const int block = prefill_block(shape);
  for (int c0 = 0; c0 < chunk; c0 += block) {
    const int qn = std::min(block, chunk - c0);
    DecodeParams p{};
    p.int2_pages = (const uint8_t*)cache->int2_pages;
    p.n_int2_pages = cache->n_int2_pages;
    p.bf16_pages = (const uint8_t*)cache->bf16_pages;
    p.n_bf16_pages = cache->n_bf16_pages;
    p.q = (const uint16_t*)q;
    p.r_k = layer->r_k;
    p.r_v = layer->r_v;
    p.int2_bt = int2_bt;
    p.max_int2_pages = max_int2_pages;
    p.bf16_bt = bf16_bt;
    p.max_bf16_pages = max_bf16_pages;
    p.ctx_lens = ctx_lens;
    p.batch = batch;
    p.n_kv = shape->n_kv_heads;
    p.g_real = g;
    p.q_heads = shape->n_q_heads;
    p.chunk = chunk;
    p.chunk0 = c0;
    p.g = qn * g;
    p.n_q = p.n_kv * p.g;
    p.ng = ng_of(shape);
    p.ct = prefill_tiles(shape, qn);
    p.mb = mb_of(shape);
    p.sink = shape->sink;
    p.recent = shape->recent;
    p.splits_int2 = splits_int2 ? splits_int2 : prefill_auto_splits(shape, batch, max_int2_pages, p.ct);
    p.splits_bf16 = splits_bf16 ? splits_bf16 : 1;
    p.bf16_in_combine = 0;
    const double smax = 2.0 * (double)layer->tau_v / 3.0;
    p.p_scale_exp = 0.f;
    if (std::isfinite(smax) && smax > 0)
      p.p_scale_exp = (float)std::clamp((int)std::floor(std::log2(32768.0 / smax)) - 1, -60, 60);
    decode_workspace_carve(p, workspace);
    p.out = out;
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    if (g_prof.on) {
      std::tie(ev0, ev1) = g_prof.acquire();
      if (!ev0) return fail(OSCAR_EHIP, "hipEventCreate failed");
    }
    if ((st = hip_status(launch_prefill(p, (hipStream_t)stream, ev0, ev1), "prefill launch"))) return st;
  }
  return ok();
}

oscar_status oscar_profile_enable(int32_t on) {
  g_prof.on = on != 0;  // launches recorded so far stay readable
  return ok();
}

oscar_status oscar_profile_read_each(float* ms_each, int64_t cap, double* main_ms, int64_t* launches) {
  if (!main_ms || !launches || cap < 0 || (cap > 0 && !ms_each)) return fail(OSCAR_EINVAL, "bad argument");
  double total = 0.0;
  int64_t i = 0;
  oscar_status st = OSCAR_OK;
  for (size_t k = 0; k < g_prof.used; ++k) {
    const auto& pr = g_prof.pool[k];
    float ms = 0.f;
    if (st == OSCAR_OK &&
        (hipEventSynchronize(pr.second) != hipSuccess || hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess))
      st = fail(OSCAR_EHIP, "event timing failed");
    total += ms;
    if (i < cap) ms_each[i] = ms;
    ++i;
  }
  *launches = (int64_t)g_prof.used;
  g_prof.used = 0;  // the pairs are reused by the next launches
  *main_ms = total;
  return st ? st : ok();
}

oscar_status oscar_profile_read(double* main_ms, int64_t* launches) {
  return oscar_profile_read_each(nullptr, 0, main_ms, launches);
}

oscar_status oscar_decode_attn_bf16_baseline(const oscar_shape* shape, const oscar_cache* cache, const void* q,
                                             int32_t batch, const int32_t* bf16_bt, int32_t max_bf16_pages,
                                             const int32_t* ctx_lens, int32_t splits, float* out, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  return decode_common(shape, nullptr, cache, q, batch, nullptr, 0, bf16_bt, max_bf16_pages, ctx_lens, 0, splits,
                       out, DecodeWorkspace{workspace, workspace_bytes, false}, stream, true);
}

}  // extern "C"
