// Host side of libqwm: argument checks, block layouts, the calibration step
// (host fp64), and the launches of the HIP kernels.  The public contract is
// include/qwm.h.
#include "qwm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "qwm_internal.h"

#define QWM_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local hipError_t g_last_hip = hipSuccess;
thread_local std::string g_msg;
// device uint32[4] that appends add their path counts to (null: none)
uint32_t* g_path_counters = nullptr;

inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

int hip_fail(hipError_t e) {
  g_last_hip = e;
  return QWM_ERR_HIP;
}

int esize(const qwm_config* c) { return c->io_dtype == QWM_F32 ? 4 : 2; }
int rpitch(int r) { return r == 0 ? 0 : (r <= 8 ? 8 : (r <= 16 ? 16 : 32)); }
// rows of the fp16 U^T block of the bf16 attention (one or two 16-row MFMA k-steps)
int ut_rows(int r) { return r > 16 ? 32 : 16; }

int check_config(const qwm_config* c) {
  if (!c) return QWM_ERR_INVALID_ARG;
  if (c->abi_version != QWM_ABI_VERSION || c->reserved != 0) return QWM_ERR_INVALID_ARG;
  if (c->num_heads < 1 || c->frame_tokens < 1 || c->max_frames < 1) return QWM_ERR_INVALID_ARG;
  if (c->num_centroids_k < 1 || c->num_centroids_v < 1) return QWM_ERR_INVALID_ARG;
  if (c->top_candidates < 0 || c->rank < 0 || c->rank > c->head_dim) return QWM_ERR_INVALID_ARG;
  if (c->io_dtype != QWM_BF16 && c->io_dtype != QWM_F32) return QWM_ERR_INVALID_ARG;
  if (c->flags & ~(QWM_UNIFORM_SENS | QWM_NO_RANGE_TERM | QWM_EXACT_ERROR | QWM_FULL_QUADRATIC))
    return QWM_ERR_INVALID_ARG;
  if (c->group_channels != 16) return QWM_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return QWM_ERR_UNSUPPORTED;
  const int t = c->group_tokens;
  if (t != 1 && t != 2 && t != 4 && t != 8 && t != 16 && t != 32) return QWM_ERR_UNSUPPORTED;
  if (c->num_centroids_k > 512 || c->num_centroids_v > 512) return QWM_ERR_UNSUPPORTED;
  if (c->top_candidates > 8 || c->rank > 32) return QWM_ERR_UNSUPPORTED;
  const int64_t cap = (int64_t)c->frame_tokens * c->max_frames;
  if (cap > (int64_t)1 << 30) return QWM_ERR_UNSUPPORTED;
  // codebook + start values must fit in LDS (160 KiB per workgroup)
  const int cmax = std::max(c->num_centroids_k, c->num_centroids_v);
  if (qwm::append_lds_bytes(qwm::append_cpad(cmax), c->head_dim, c->io_dtype == QWM_F32, rpitch(c->rank), 8) >
      160 * 1024)
    return QWM_ERR_UNSUPPORTED;
  return QWM_OK;
}

void fill_layout(const qwm_config* c, qwm_layout_info* L) {
  std::memset(L, 0, sizeof(*L));
  const uint64_t H = c->num_heads, D = c->head_dim, r = c->rank, ng = D / 16;
  const uint64_t es = esize(c);
  const uint64_t ck = c->num_centroids_k, cv = c->num_centroids_v;
  const uint64_t tpf = ceil_div(c->frame_tokens, c->group_tokens);
  L->token_capacity = (uint64_t)c->frame_tokens * c->max_frames;
  L->tile_capacity = tpf * c->max_frames;
  L->idx_k_bytes = ck <= 256 ? 1 : 2;
  L->idx_v_bytes = cv <= 256 ? 1 : 2;
  uint64_t o = 0;
  auto put = [&](uint64_t& field, uint64_t bytes) { field = o; o = align256(o + bytes); };
  put(L->mu_k, H * ck * D * es);
  put(L->mu_v, H * cv * D * es);
  put(L->sens, H * D * 4);
  put(L->u, H * D * r * 4);
  put(L->u64, H * D * rpitch((int)r) * 8);
  put(L->sgroup, H * ng * 8);
  put(L->norm_kw, H * ck * 4);
  put(L->norm_k, H * ck * 4);
  put(L->norm_v, H * cv * 4);
  put(L->head_max, H * 4 * 4);
  put(L->mu_k16, H * ck * D * 2);
  put(L->mu_v16, H * cv * D * 2);
  put(L->ut16, H * ut_rows((int)r) * D * 2);
  put(L->moment, (c->flags & QWM_FULL_QUADRATIC) ? H * D * D * 8 : 0);
  L->calib_bytes = o;
  o = 0;
  const uint64_t N = L->token_capacity, P = L->tile_capacity;
  put(L->idx_k, H * N * L->idx_k_bytes);
  put(L->codes_k, H * N * ng * 4);
  put(L->params_k, H * P * ng * 4);
  put(L->coef, H * N * r);
  put(L->coef_scale, r ? H * N * 2 : 0);
  put(L->idx_v, H * N * L->idx_v_bytes);
  put(L->codes_v, H * N * ng * 4);
  put(L->params_v, H * P * ng * 4);
  L->cache_bytes = o;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_act(const qwm_config* c, const void* ptr, int64_t n, const qwm_strides* st) {
  if (!st) return QWM_ERR_INVALID_ARG;
  if (n < 0) return QWM_ERR_INVALID_ARG;
  if (n == 0) return QWM_OK;
  if (!ptr || !aligned16(ptr)) return QWM_ERR_INVALID_ARG;
  if (st->token < c->head_dim || st->head < 0) return QWM_ERR_INVALID_ARG;
  if ((st->token * esize(c)) % 16 != 0 || (st->head * esize(c)) % 16 != 0) return QWM_ERR_INVALID_ARG;
  if (c->num_heads > 1 && st->head == 0) return QWM_ERR_INVALID_ARG;
  return QWM_OK;
}

// ---------------------------------------------------------------- rounding
float round_bf16(double x) {
  if (x == 0.0 || !std::isfinite(x)) return (float)x;
  int e;
  const double m = std::frexp(x, &e);             // x = m 2^e, 0.5 <= |m| < 1
  const double r = std::nearbyint(std::ldexp(m, 8));  // 8 significant bits, ties to even
  return (float)std::ldexp(r, e - 8);
}

// ---------------------------------------------------------------- calibration
struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    s += 0x9E3779B97F4A7C15ull;
    uint64_t z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

// Lloyd's algorithm (fp64, direct-form distances, ties to the lowest index,
// empty clusters keep their centre), Forgy start from a partial
// Fisher-Yates shuffle driven by SplitMix64.
void kmeans(const float* x, int n, int d, int C, int iters, uint64_t seed, std::vector<double>& mu) {
  std::vector<int> perm(n);
  for (int i = 0; i < n; ++i) perm[i] = i;
  SplitMix64 rng{seed};
  for (int i = 0; i < C; ++i) {
    const int j = i + (int)(rng.next() % (uint64_t)(n - i));
    std::swap(perm[i], perm[j]);
  }
  mu.assign((size_t)C * d, 0.0);
  for (int c = 0; c < C; ++c)
    for (int j = 0; j < d; ++j) mu[(size_t)c * d + j] = x[(size_t)perm[c] * d + j];
  std::vector<int> assign(n);
  std::vector<double> sum((size_t)C * d);
  std::vector<int> cnt(C);
  for (int it = 0; it < iters; ++it) {
    for (int t = 0; t < n; ++t) {
      const float* xt = x + (size_t)t * d;
      double best = INFINITY;
      int bc = 0;
      for (int c = 0; c < C; ++c) {
        const double* m = &mu[(size_t)c * d];
        double acc = 0.0;
        for (int j = 0; j < d; ++j) {
          const double df = (double)xt[j] - m[j];
          acc += df * df;
        }
        if (acc < best) { best = acc; bc = c; }
      }
      assign[t] = bc;
    }
    std::fill(sum.begin(), sum.end(), 0.0);
    std::fill(cnt.begin(), cnt.end(), 0);
    for (int t = 0; t < n; ++t) {
      const int c = assign[t];
      cnt[c]++;
      for (int j = 0; j < d; ++j) sum[(size_t)c * d + j] += x[(size_t)t * d + j];
    }
    for (int c = 0; c < C; ++c)
      if (cnt[c] > 0)
        for (int j = 0; j < d; ++j) mu[(size_t)c * d + j] = sum[(size_t)c * d + j] / cnt[c];
  }
}

// Cyclic Jacobi eigen-decomposition of a symmetric d x d matrix (fp64).
// Returns eigenvalues in w and eigenvectors as columns of v.
void jacobi_eigen(std::vector<double> a, int d, std::vector<double>& w, std::vector<double>& v) {
  v.assign((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) v[(size_t)i * d + i] = 1.0;
  auto A = [&](int i, int j) -> double& { return a[(size_t)i * d + j]; };
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0, tot = 0.0;
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        tot += A(i, j) * A(i, j);
        if (i != j) off += A(i, j) * A(i, j);
      }
    if (off <= 1e-30 * tot) break;
    for (int p = 0; p < d - 1; ++p)
      for (int q = p + 1; q < d; ++q) {
        const double apq = A(p, q);
        if (std::fabs(apq) < 1e-300) continue;
        const double theta = (A(q, q) - A(p, p)) / (2.0 * apq);
        const double t = (theta >= 0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < d; ++k) {  // columns p, q
          const double akp = A(k, p), akq = A(k, q);
          A(k, p) = c * akp - s * akq;
          A(k, q) = s * akp + c * akq;
        }
        for (int k = 0; k < d; ++k) {  // rows p, q
          const double apk = A(p, k), aqk = A(q, k);
          A(p, k) = c * apk - s * aqk;
          A(q, k) = s * apk + c * aqk;
        }
        for (int k = 0; k < d; ++k) {
          const double vkp = v[(size_t)k * d + p], vkq = v[(size_t)k * d + q];
          v[(size_t)k * d + p] = c * vkp - s * vkq;
          v[(size_t)k * d + q] = s * vkp + c * vkq;
        }
      }
  }
  w.resize(d);
  for (int i = 0; i < d; ++i) w[i] = A(i, i);
}

// Query second moment M = (1/n) sum q q^T of one head (fp64, symmetric)
void second_moment(const float* qh, int64_t n_q, int d, double* m) {
  std::fill(m, m + (size_t)d * d, 0.0);
  for (int64_t t = 0; t < n_q; ++t) {
    const float* q = qh + (size_t)t * d;
    for (int i = 0; i < d; ++i) {
      const double qi = q[i];
      for (int j = 0; j <= i; ++j) m[(size_t)i * d + j] += qi * (double)q[j];
    }
  }
  for (int i = 0; i < d; ++i)
    for (int j = 0; j <= i; ++j) {
      m[(size_t)i * d + j] /= (double)n_q;
      m[(size_t)j * d + i] = m[(size_t)i * d + j];
    }
}

void calibrate_head(const qwm_config* c, const float* qh, int64_t n_q, const float* kh, const float* vh,
                    int64_t n_kv, uint64_t seed, int iters, int h, float* mu_k, float* mu_v, float* sens,
                    float* u, double* energy) {
  const int d = c->head_dim, r = c->rank;
  std::vector<double> m((size_t)d * d);
  second_moment(qh, n_q, d, m.data());
  double trace = 0.0;
  for (int i = 0; i < d; ++i) {
    sens[(size_t)h * d + i] = (float)m[(size_t)i * d + i];
    trace += m[(size_t)i * d + i];
  }
  std::vector<double> w, v;
  jacobi_eigen(m, d, w, v);
  std::vector<int> order(d);
  for (int i = 0; i < d; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return w[a] > w[b]; });
  double top = 0.0;
  for (int k = 0; k < r; ++k) {
    const int col = order[k];
    top += w[col];
    int jmax = 0;
    for (int j = 1; j < d; ++j)
      if (std::fabs(v[(size_t)j * d + col]) > std::fabs(v[(size_t)jmax * d + col])) jmax = j;
    const double sgn = v[(size_t)jmax * d + col] < 0 ? -1.0 : 1.0;
    for (int j = 0; j < d; ++j) u[((size_t)h * d + j) * r + k] = (float)(sgn * v[(size_t)j * d + col]);
  }
  if (energy) energy[h] = r > 0 ? top / trace : 0.0;
  std::vector<double> mu;
  const bool f32 = c->io_dtype == QWM_F32;
  kmeans(kh, (int)n_kv, d, c->num_centroids_k, iters, seed + 2 * (uint64_t)h, mu);
  for (size_t i = 0; i < mu.size(); ++i)
    mu_k[(size_t)h * c->num_centroids_k * d + i] = f32 ? (float)mu[i] : round_bf16(mu[i]);
  kmeans(vh, (int)n_kv, d, c->num_centroids_v, iters, seed + 2 * (uint64_t)h + 1, mu);
  for (size_t i = 0; i < mu.size(); ++i)
    mu_v[(size_t)h * c->num_centroids_v * d + i] = f32 ? (float)mu[i] : round_bf16(mu[i]);
}

uint16_t f32_to_bf16_bits(float x) {  // x is bf16-exact
  uint32_t b;
  std::memcpy(&b, &x, 4);
  return (uint16_t)(b >> 16);
}

float bf16_bits_to_f32(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &b, 4);
  return f;
}

int choose_splits(const qwm_config* c, int64_t n_k, int64_t n_q) {
  const int64_t blocks = ((n_q + 127) / 128) * c->num_heads;
  int64_t splits = 1;
  const int64_t target = 1024;  // workgroups to fill 256 CUs several times
  if (blocks < target) splits = (target + blocks - 1) / blocks;
  const int64_t max_by_keys = std::max<int64_t>(1, n_k / 512);  // >= 8 key tiles per split
  splits = std::min<int64_t>(std::min<int64_t>(splits, max_by_keys), 64);
  return (int)std::max<int64_t>(1, splits);
}

}  // namespace

// ====================================================================== API

QWM_API int32_t qwm_abi_version(void) { return QWM_ABI_VERSION; }

QWM_API const char* qwm_status_string(int status) {
  switch (status) {
    case QWM_OK: return "ok";
    case QWM_ERR_INVALID_ARG: return "invalid argument";
    case QWM_ERR_UNSUPPORTED: return "unsupported configuration";
    case QWM_ERR_ALIGN: return "append is not a whole number of frames";
    case QWM_ERR_CAPACITY: return "capacity exceeded";
    case QWM_ERR_STATE: return "cache state mismatch";
    case QWM_ERR_HIP:
      g_msg = std::string("HIP error: ") + hipGetErrorString(g_last_hip);
      return g_msg.c_str();
    default: return "unknown status";
  }
}

QWM_API int qwm_layout(const qwm_config* cfg, qwm_layout_info* out) {
  const int st = check_config(cfg);
  if (st) return st;
  if (!out) return QWM_ERR_INVALID_ARG;
  fill_layout(cfg, out);
  return QWM_OK;
}

QWM_API int qwm_footprint(const qwm_config* cfg, int64_t n_tokens, uint64_t* stored, uint64_t* resident,
                          uint64_t* original) {
  const int st = check_config(cfg);
  if (st) return st;
  if (!stored || !original || n_tokens < 0 || n_tokens % cfg->frame_tokens) return QWM_ERR_INVALID_ARG;
  qwm_layout_info L;
  fill_layout(cfg, &L);
  const uint64_t H = cfg->num_heads, D = cfg->head_dim, r = cfg->rank, ng = D / 16, n = n_tokens;
  const uint64_t es = esize(cfg);
  const uint64_t tiles = (n / cfg->frame_tokens) * (uint64_t)ceil_div(cfg->frame_tokens, cfg->group_tokens);
  const uint64_t cache_part = H * n * (L.idx_k_bytes + L.idx_v_bytes) + 2 * H * n * ng * 4 + 2 * H * tiles * ng * 4 +
                              (r ? H * n * r + 2 * H * n : 0);
  *stored = cache_part + H * (uint64_t)(cfg->num_centroids_k + cfg->num_centroids_v) * D * es + H * D * r * 4 + H * D * 4;
  if (resident) *resident = cache_part + L.calib_bytes;
  *original = 2 * n * H * D * es;
  return QWM_OK;
}

QWM_API int qwm_calibrate_host(const qwm_config* cfg, const float* q_hist, int64_t n_q, const float* k_hist,
                               const float* v_hist, int64_t n_kv, uint64_t seed, int32_t iters, float* mu_k,
                               float* mu_v, float* sens, float* u, double* energy) {
  const int st = check_config(cfg);
  if (st) return st;
  if (!q_hist || !k_hist || !v_hist || !mu_k || !mu_v || !sens || (!u && cfg->rank > 0)) return QWM_ERR_INVALID_ARG;
  if (n_q < 1 || n_kv < std::max(cfg->num_centroids_k, cfg->num_centroids_v) || iters < 0) return QWM_ERR_INVALID_ARG;
  const int H = cfg->num_heads, d = cfg->head_dim;
  const unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  const int nthreads = (int)std::min<unsigned>(hw, (unsigned)H);
  std::vector<std::thread> pool;
  for (int w = 0; w < nthreads; ++w)
    pool.emplace_back([&, w] {
      for (int h = w; h < H; h += nthreads)
        calibrate_head(cfg, q_hist + (size_t)h * n_q * d, n_q, k_hist + (size_t)h * n_kv * d,
                       v_hist + (size_t)h * n_kv * d, n_kv, seed, iters, h, mu_k, mu_v, sens, u, energy);
    });
  for (auto& t : pool) t.join();
  return QWM_OK;
}

QWM_API int qwm_calib_import(const qwm_config* cfg, void* calib, const float* mu_k, const float* mu_v,
                             const float* sens, const float* u, void* stream) {
  const int st = check_config(cfg);
  if (st) return st;
  if (!calib || !mu_k || !mu_v || !sens || (!u && cfg->rank > 0)) return QWM_ERR_INVALID_ARG;
  qwm_layout_info L;
  fill_layout(cfg, &L);
  const int H = cfg->num_heads, d = cfg->head_dim, r = cfg->rank, ng = d / 16, rp = rpitch(r);
  const int ck = cfg->num_centroids_k, cv = cfg->num_centroids_v;
  const bool f32 = cfg->io_dtype == QWM_F32;
  std::vector<unsigned char> blk(L.calib_bytes, 0);
  auto put_mu = [&](uint64_t off, const float* src, size_t count) {
    if (f32) std::memcpy(&blk[off], src, count * 4);
    else {
      uint16_t* dst = reinterpret_cast<uint16_t*>(&blk[off]);
      for (size_t i = 0; i < count; ++i) dst[i] = f32_to_bf16_bits(src[i]);
    }
  };
  put_mu(L.mu_k, mu_k, (size_t)H * ck * d);
  put_mu(L.mu_v, mu_v, (size_t)H * cv * d);
  std::memcpy(&blk[L.sens], sens, (size_t)H * d * 4);
  if (r) std::memcpy(&blk[L.u], u, (size_t)H * d * r * 4);
  double* u64 = reinterpret_cast<double*>(&blk[L.u64]);
  double* sg = reinterpret_cast<double*>(&blk[L.sgroup]);
  float* nkw = reinterpret_cast<float*>(&blk[L.norm_kw]);
  float* nk = reinterpret_cast<float*>(&blk[L.norm_k]);
  float* nv = reinterpret_cast<float*>(&blk[L.norm_v]);
  float* hm = reinterpret_cast<float*>(&blk[L.head_max]);
  // stored values as the kernels see them (bf16 rounding is exact for bf16-valued input)
  auto stored = [&](const float* src, size_t i) { return f32 ? (double)src[i] : (double)bf16_bits_to_f32(f32_to_bf16_bits(src[i])); };
  for (int h = 0; h < H; ++h) {
    for (int j = 0; j < d; ++j)
      for (int i = 0; i < rp; ++i)
        u64[((size_t)h * d + j) * rp + i] = i < r ? (double)u[((size_t)h * d + j) * r + i] : 0.0;
    for (int g = 0; g < ng; ++g) {
      double s = 0.0;
      for (int j = 0; j < 16; ++j) s += (double)sens[(size_t)h * d + 16 * g + j];
      sg[(size_t)h * ng + g] = s;
    }
    double mw = 0, mu1 = 0, mv = 0;
    for (int c = 0; c < ck; ++c) {
      double a = 0, b = 0;
      for (int j = 0; j < d; ++j) {
        const double x = stored(mu_k, ((size_t)h * ck + c) * d + j);
        a += (double)sens[(size_t)h * d + j] * x * x;
        b += x * x;
      }
      nkw[(size_t)h * ck + c] = (float)(a / 2);
      nk[(size_t)h * ck + c] = (float)(b / 2);
      mw = std::max(mw, std::sqrt(a));
      mu1 = std::max(mu1, std::sqrt(b));
    }
    for (int c = 0; c < cv; ++c) {
      double b = 0;
      for (int j = 0; j < d; ++j) {
        const double x = stored(mu_v, ((size_t)h * cv + c) * d + j);
        b += x * x;
      }
      nv[(size_t)h * cv + c] = (float)(b / 2);
      mv = std::max(mv, std::sqrt(b));
    }
    // slightly inflated so the kernel's error bound stays an upper bound
    hm[h * 4 + 0] = (float)(mw * (1 + 1e-6));
    hm[h * 4 + 1] = (float)(mu1 * (1 + 1e-6));
    hm[h * 4 + 2] = (float)(mv * (1 + 1e-6));
    hm[h * 4 + 3] = 0.f;
  }
  // fp16 copies for the bf16 attention path, channels of each 16-group in
  // paired order: position 2j <- channel j, position 2j+1 <- channel j+8
  auto paired = [](int pos) { return (pos & ~15) + (pos & 15) / 2 + 8 * (pos & 1); };
  auto f16 = [](double x) { return __builtin_bit_cast(uint16_t, (_Float16)(float)x); };
  uint16_t* mk16 = reinterpret_cast<uint16_t*>(&blk[L.mu_k16]);
  uint16_t* mv16 = reinterpret_cast<uint16_t*>(&blk[L.mu_v16]);
  uint16_t* ut16 = reinterpret_cast<uint16_t*>(&blk[L.ut16]);
  for (size_t row = 0; row < (size_t)H * ck; ++row)
    for (int j = 0; j < d; ++j) mk16[row * d + j] = f16(stored(mu_k, row * d + paired(j)));
  for (size_t row = 0; row < (size_t)H * cv; ++row)
    for (int j = 0; j < d; ++j) mv16[row * d + j] = f16(stored(mu_v, row * d + paired(j)));
  const int utr = ut_rows(r);
  for (int h = 0; h < H; ++h)
    for (int c = 0; c < utr; ++c)
      for (int j = 0; j < d; ++j)
        ut16[((size_t)h * utr + c) * d + j] = c < r ? f16(u[((size_t)h * d + paired(j)) * r + c]) : 0;
  // Blocking copy after draining the caller's stream: the block is complete
  // in device memory when this call returns.
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  // the moment block (last) is not part of this import
  e = hipMemcpy(calib, blk.data(), (size_t)L.moment, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e);
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e);
  return QWM_OK;
}

QWM_API int qwm_calib_import_moment(const qwm_config* cfg, void* calib, const double* m, void* stream) {
  const int st = check_config(cfg);
  if (st) return st;
  if (!calib || !m || !(cfg->flags & QWM_FULL_QUADRATIC)) return QWM_ERR_INVALID_ARG;
  qwm_layout_info L;
  fill_layout(cfg, &L);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  const size_t bytes = (size_t)cfg->num_heads * cfg->head_dim * cfg->head_dim * 8;
  e = hipMemcpy(static_cast<unsigned char*>(calib) + L.moment, m, bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e);
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e);
  return QWM_OK;
}

QWM_API int qwm_calibrate(const qwm_config* cfg, void* calib, const void* q_hist, int64_t n_q,
                          const qwm_strides* st_q, const void* k_hist, const void* v_hist, int64_t n_kv,
                          const qwm_strides* st_kv, uint64_t seed, int32_t iters, double* energy, void* stream) {
  int st = check_config(cfg);
  if (st) return st;
  if (!calib || n_q < 1 || n_kv < 1) return QWM_ERR_INVALID_ARG;
  if ((st = check_act(cfg, q_hist, n_q, st_q)) || (st = check_act(cfg, k_hist, n_kv, st_kv)) ||
      (st = check_act(cfg, v_hist, n_kv, st_kv)))
    return st;
  if (n_kv < std::max(cfg->num_centroids_k, cfg->num_centroids_v) || iters < 0) return QWM_ERR_INVALID_ARG;
  const int H = cfg->num_heads, d = cfg->head_dim, es = esize(cfg);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the inputs are produced on the caller's stream: drain it, then copy with
  // blocking copies (complete on return)
  {
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e);
  }
  // Device -> host through a pinned staging buffer (blocking 2D copies, one per
  // head), then widened to fp32.
  auto fetch = [&](const void* src, int64_t n, const qwm_strides* sd, std::vector<float>& dst) -> int {
    const size_t bytes = (size_t)H * n * d * es;
    void* stage = nullptr;
    hipError_t e = hipHostMalloc(&stage, bytes, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e);
    unsigned char* raw = static_cast<unsigned char*>(stage);
    for (int h = 0; h < H && e == hipSuccess; ++h)
      e = hipMemcpy2D(raw + (size_t)h * n * d * es, (size_t)d * es,
                      static_cast<const unsigned char*>(src) + (size_t)h * sd->head * es, (size_t)sd->token * es,
                      (size_t)d * es, (size_t)n, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      hipHostFree(stage);
      return hip_fail(e);
    }
    dst.resize((size_t)H * n * d);
    if (es == 4) std::memcpy(dst.data(), raw, bytes);
    else {
      const uint16_t* b = reinterpret_cast<const uint16_t*>(raw);
      for (size_t i = 0; i < dst.size(); ++i) dst[i] = bf16_bits_to_f32(b[i]);
    }
    e = hipHostFree(stage);
    if (e != hipSuccess) return hip_fail(e);
    return QWM_OK;
  };
  std::vector<float> q, k, v;
  if ((st = fetch(q_hist, n_q, st_q, q)) || (st = fetch(k_hist, n_kv, st_kv, k)) || (st = fetch(v_hist, n_kv, st_kv, v)))
    return st;
  std::vector<float> mk((size_t)H * cfg->num_centroids_k * d), mv((size_t)H * cfg->num_centroids_v * d);
  std::vector<float> sens((size_t)H * d), u((size_t)H * d * std::max(cfg->rank, 1));
  st = qwm_calibrate_host(cfg, q.data(), n_q, k.data(), v.data(), n_kv, seed, iters, mk.data(), mv.data(),
                          sens.data(), u.data(), energy);
  if (st) return st;
  st = qwm_calib_import(cfg, calib, mk.data(), mv.data(), sens.data(), u.data(), stream);
  if (st || !(cfg->flags & QWM_FULL_QUADRATIC)) return st;
  std::vector<double> m((size_t)H * d * d);
  for (int h = 0; h < H; ++h) second_moment(q.data() + (size_t)h * n_q * d, n_q, d, m.data() + (size_t)h * d * d);
  return qwm_calib_import_moment(cfg, calib, m.data(), stream);
}

QWM_API int qwm_append_path_counters(void* counters) {
  if (counters && ((uintptr_t)counters & 3u)) return QWM_ERR_INVALID_ARG;
  g_path_counters = static_cast<uint32_t*>(counters);
  return QWM_OK;
}

QWM_API int qwm_cache_init(const qwm_config* cfg, const void* calib, void* base, qwm_cache* cache) {
  const int st = check_config(cfg);
  if (st) return st;
  if (!calib || !base || !cache || !aligned16(base) || !aligned16(calib)) return QWM_ERR_INVALID_ARG;
  cache->base = base;
  cache->calib = calib;
  cache->n_k = 0;
  cache->n_v = 0;
  cache->abi_version = QWM_ABI_VERSION;
  cache->reserved = 0;
  return QWM_OK;
}

namespace {

// Checks one append and fills its kernel parameters (n_new > 0 on success
// with QWM_OK; *empty set when there is nothing to do).
int fill_append(const qwm_config* cfg, const qwm_cache* cache, const void* x, int64_t n_new, const qwm_strides* st,
                bool key, qwm::AppendParams& p, bool* empty) {
  *empty = false;
  int s = check_config(cfg);
  if (s) return s;
  if (!cache || !cache->base || !cache->calib || cache->abi_version != QWM_ABI_VERSION) return QWM_ERR_INVALID_ARG;
  if ((s = check_act(cfg, x, n_new, st))) return s;
  if (n_new % cfg->frame_tokens) return QWM_ERR_ALIGN;
  qwm_layout_info L;
  fill_layout(cfg, &L);
  const int64_t n0 = key ? cache->n_k : cache->n_v;
  if (n0 < 0 || n0 % cfg->frame_tokens) return QWM_ERR_STATE;
  if (n0 + n_new > (int64_t)L.token_capacity) return QWM_ERR_CAPACITY;
  if (n_new == 0) {
    *empty = true;
    return QWM_OK;
  }
  const int F = cfg->frame_tokens;
  unsigned char* cb = static_cast<unsigned char*>(cache->base);
  const unsigned char* kb = static_cast<const unsigned char*>(cache->calib);
  p = qwm::AppendParams{};
  p.x = x;
  p.head_stride = st->head;
  p.token_stride = st->token;
  p.n_new = (int)n_new;
  p.frame0 = (int)(n0 / F);
  p.F = F;
  p.T = cfg->group_tokens;
  p.tpf = ceil_div(F, cfg->group_tokens);
  p.segs_per_frame = ceil_div(F, qwm::kSegTokens);
  p.total_segs = (int)(n_new / F) * p.segs_per_frame;
  p.Ncap = (int64_t)L.token_capacity;
  p.Pcap = (int64_t)L.tile_capacity;
  p.tok0 = n0;
  if (key) {
    p.C = cfg->num_centroids_k;
    p.uniform = (cfg->flags & QWM_UNIFORM_SENS) ? 1 : 0;
    p.use_range = (cfg->flags & QWM_NO_RANGE_TERM) || cfg->top_candidates <= 1 ? 0 : 1;
    p.Kc = p.use_range ? cfg->top_candidates : 1;
    // stage-2 score: the full form with s = 1 is the diagonal form with s = 1
    p.s2mode = (cfg->flags & QWM_FULL_QUADRATIC) ? (p.uniform ? 1 : 2) : (cfg->flags & QWM_EXACT_ERROR) ? 1 : 0;
    p.moment = reinterpret_cast<const double*>(kb + L.moment);
    p.r = cfg->rank;
    p.mu = kb + L.mu_k;
    p.norm_half = reinterpret_cast<const float*>(kb + (p.uniform ? L.norm_k : L.norm_kw));
    p.head_max_slot = p.uniform ? 1 : 0;
    p.idx = cb + L.idx_k;
    p.idx_bytes = (int)L.idx_k_bytes;
    p.codes = reinterpret_cast<uint32_t*>(cb + L.codes_k);
    p.params = reinterpret_cast<uint32_t*>(cb + L.params_k);
    p.coef = reinterpret_cast<int8_t*>(cb + L.coef);
    p.coef_scale = reinterpret_cast<uint16_t*>(cb + L.coef_scale);
  } else {
    p.C = cfg->num_centroids_v;
    p.uniform = 1;
    p.use_range = 0;
    p.Kc = 1;
    p.r = 0;
    p.mu = kb + L.mu_v;
    p.norm_half = reinterpret_cast<const float*>(kb + L.norm_v);
    p.head_max_slot = 2;
    p.idx = cb + L.idx_v;
    p.idx_bytes = (int)L.idx_v_bytes;
    p.codes = reinterpret_cast<uint32_t*>(cb + L.codes_v);
    p.params = reinterpret_cast<uint32_t*>(cb + L.params_v);
  }
  p.Cpad = qwm::append_cpad(p.C);
  p.sens = reinterpret_cast<const float*>(kb + L.sens);
  p.u64 = reinterpret_cast<const double*>(kb + L.u64);
  p.rp = rpitch(cfg->rank);
  p.sgroup = reinterpret_cast<const double*>(kb + L.sgroup);
  p.head_max = reinterpret_cast<const float*>(kb + L.head_max);
  p.counters = g_path_counters;
  return QWM_OK;
}

int append(const qwm_config* cfg, qwm_cache* cache, const void* x, int64_t n_new, const qwm_strides* st, void* stream,
           bool key) {
  qwm::AppendParams p;
  bool empty;
  int s = fill_append(cfg, cache, x, n_new, st, key, p, &empty);
  if (s || empty) return s;
  hipError_t e = qwm::launch_append(p, cfg->num_heads, cfg->head_dim, cfg->io_dtype == QWM_F32, key,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  if (key) cache->n_k += n_new;
  else cache->n_v += n_new;
  return QWM_OK;
}

int fill_attn(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q, const qwm_strides* st_q,
              float scale, qwm::AttnParams& p) {
  int s = check_config(cfg);
  if (s) return s;
  if (!cache || !cache->base || !cache->calib || cache->abi_version != QWM_ABI_VERSION) return QWM_ERR_INVALID_ARG;
  if ((s = check_act(cfg, q, n_q, st_q))) return s;
  if (cache->n_k != cache->n_v) return QWM_ERR_STATE;
  qwm_layout_info L;
  fill_layout(cfg, &L);
  if (cache->n_k < 0 || cache->n_k > (int64_t)L.token_capacity) return QWM_ERR_STATE;
  const unsigned char* cb = static_cast<const unsigned char*>(cache->base);
  const unsigned char* kb = static_cast<const unsigned char*>(cache->calib);
  p = qwm::AttnParams{};
  p.q = q;
  p.q_head_stride = st_q->head;
  p.q_token_stride = st_q->token;
  p.n_q = (int)n_q;
  p.n_k = (int)cache->n_k;
  p.F = cfg->frame_tokens;
  p.T = cfg->group_tokens;
  p.tpf = ceil_div(cfg->frame_tokens, cfg->group_tokens);
  p.r = cfg->rank;
  p.rp = rpitch(cfg->rank);
  const float sc = scale > 0.f ? scale : 1.f / std::sqrt((float)cfg->head_dim);
  p.scale = sc;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.Ncap = (int64_t)L.token_capacity;
  p.Pcap = (int64_t)L.tile_capacity;
  p.C_k = cfg->num_centroids_k;
  p.C_v = cfg->num_centroids_v;
  p.mu_k = kb + L.mu_k;
  p.mu_v = kb + L.mu_v;
  p.u = reinterpret_cast<const float*>(kb + L.u);
  p.idx_k = cb + L.idx_k;
  p.idx_k_bytes = (int)L.idx_k_bytes;
  p.codes_k = reinterpret_cast<const uint32_t*>(cb + L.codes_k);
  p.params_k = reinterpret_cast<const uint32_t*>(cb + L.params_k);
  p.coef = reinterpret_cast<const int8_t*>(cb + L.coef);
  p.coef_scale = reinterpret_cast<const uint16_t*>(cb + L.coef_scale);
  p.idx_v = cb + L.idx_v;
  p.idx_v_bytes = (int)L.idx_v_bytes;
  p.codes_v = reinterpret_cast<const uint32_t*>(cb + L.codes_v);
  p.params_v = reinterpret_cast<const uint32_t*>(cb + L.params_v);
  p.mu_k16 = reinterpret_cast<const uint16_t*>(kb + L.mu_k16);
  p.mu_v16 = reinterpret_cast<const uint16_t*>(kb + L.mu_v16);
  p.ut16 = reinterpret_cast<const uint16_t*>(kb + L.ut16);
  // key / F = (key + umulhi(key, lo)) >> s with M = 2^32 + lo = ceil(2^(32+s) / F),
  // s = ceil(log2 F): exact for every key below 2^32 (keys stay below 2^30)
  int sF = 0;
  while ((1ll << sF) < cfg->frame_tokens) ++sF;
  const uint64_t M = ((1ull << (32 + sF)) + (uint64_t)cfg->frame_tokens - 1) / (uint64_t)cfg->frame_tokens;
  p.divF_lo = (uint32_t)(M - (1ull << 32));
  p.divF_s = sF;
  int lt = 0;
  while ((1 << lt) < cfg->group_tokens) ++lt;
  p.log2T = lt;
  p.splits = 1;
  p.keys_per_split = std::max(p.n_k, 1);
  return QWM_OK;
}

}  // namespace

QWM_API int qwm_quantize_append_k(const qwm_config* cfg, qwm_cache* cache, const void* k_new, int64_t n_new,
                                  const qwm_strides* st, void* stream) {
  return append(cfg, cache, k_new, n_new, st, stream, true);
}

QWM_API int qwm_quantize_append_v(const qwm_config* cfg, qwm_cache* cache, const void* v_new, int64_t n_new,
                                  const qwm_strides* st, void* stream) {
  return append(cfg, cache, v_new, n_new, st, stream, false);
}

QWM_API int qwm_quantize_append_kv(const qwm_config* cfg, qwm_cache* cache, const void* k_new, const void* v_new,
                                   int64_t n_new, const qwm_strides* st_k, const qwm_strides* st_v, void* stream) {
  if (!cache) return QWM_ERR_INVALID_ARG;
  if (cache->n_k != cache->n_v) return QWM_ERR_STATE;
  qwm::AppendParams pk, pv;
  bool empty_k, empty_v;
  int s = fill_append(cfg, cache, k_new, n_new, st_k, true, pk, &empty_k);
  if (s) return s;
  if ((s = fill_append(cfg, cache, v_new, n_new, st_v, false, pv, &empty_v))) return s;
  if (empty_k) return QWM_OK;
  hipError_t e = qwm::launch_append_kv(pk, pv, cfg->num_heads, cfg->head_dim, cfg->io_dtype == QWM_F32,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  cache->n_k += n_new;
  cache->n_v += n_new;
  return QWM_OK;
}

// Partial-result workspace of the bf16 attention (stream-K): two slots of
// kAttnBf16Queries rows per workgroup, O in fp16 then the fp32 lse values.
size_t bf16_partial_bytes(const qwm_config* cfg) {
  const size_t rows = 2 * (size_t)qwm::kAttnBf16MaxWorkgroups * qwm::kAttnBf16Queries;
  return align256(rows * (size_t)cfg->head_dim * 2) + rows * 4;
}

QWM_API size_t qwm_attention_workspace_size(const qwm_config* cfg, int64_t n_tokens, int64_t n_q) {
  if (check_config(cfg) || n_tokens < 0 || n_q < 0) return 0;
  if (cfg->io_dtype == QWM_BF16) return (n_tokens > 0 && n_q > 0) ? bf16_partial_bytes(cfg) : 0;
  const int splits = choose_splits(cfg, n_tokens, n_q);
  if (splits <= 1) return 0;
  return (size_t)splits * cfg->num_heads * n_q * ((size_t)cfg->head_dim * 4 + 4) + 256;
}

// bf16 activations: stream-K partials when the workspace holds them, else one
// whole (head, query block) per workgroup
int run_attention_bf16(const qwm_config* cfg, qwm::AttnParams& p, void* workspace, size_t ws_bytes, void* stream,
                       const qwm::PartTable* parts = nullptr) {
  if (p.n_k + p.n_loc > 0 && ws_bytes >= bf16_partial_bytes(cfg)) {
    const size_t rows = 2 * (size_t)qwm::kAttnBf16MaxWorkgroups * qwm::kAttnBf16Queries;
    p.part_o = static_cast<float*>(workspace);  // holds fp16 rows on this path
    p.part_ml = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) +
                                         align256(rows * (size_t)cfg->head_dim * 2));
  }
  hipError_t e = parts ? qwm::launch_attention_bf16(p, cfg->num_heads, cfg->head_dim, static_cast<hipStream_t>(stream), parts)
                       : qwm::launch_attention(p, cfg->num_heads, cfg->head_dim, false, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return QWM_OK;
}

QWM_API int qwm_attention_timed(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q,
                                const qwm_strides* st_q, float scale, void* out, const qwm_strides* st_out,
                                float* lse, void* workspace, size_t ws_bytes, void* stream, void* ev_kernel_begin,
                                void* ev_kernel_end) {
  qwm::AttnParams p;
  int s = fill_attn(cfg, cache, q, n_q, st_q, scale, p);
  if (s) return s;
  p.ev_begin = ev_kernel_begin;
  p.ev_end = ev_kernel_end;
  if ((s = check_act(cfg, out, n_q, st_out))) return s;
  if (n_q == 0) return QWM_OK;
  if (lse && !aligned16(lse)) return QWM_ERR_INVALID_ARG;
  if (ws_bytes > 0 && (!workspace || !aligned16(workspace))) return QWM_ERR_INVALID_ARG;
  p.out = out;
  p.o_head_stride = st_out->head;
  p.o_token_stride = st_out->token;
  p.lse = lse;
  if (cfg->io_dtype == QWM_BF16) return run_attention_bf16(cfg, p, workspace, ws_bytes, stream);
  int splits = choose_splits(cfg, p.n_k, n_q);
  const size_t per_split = (size_t)cfg->num_heads * n_q * ((size_t)cfg->head_dim * 4 + 4);
  while (splits > 1 && (size_t)splits * per_split + 256 > ws_bytes) --splits;
  if (splits > 1) {
    int kps = ceil_div(p.n_k, splits);
    kps = ceil_div(kps, 64) * 64;
    splits = ceil_div(p.n_k, kps);
    p.splits = splits;
    p.keys_per_split = kps;
    p.part_o = static_cast<float*>(workspace);
    const size_t obytes = (size_t)splits * cfg->num_heads * n_q * cfg->head_dim * 4;
    p.part_ml = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + ((obytes + 255) & ~size_t(255)));
  }
  hipError_t e = qwm::launch_attention(p, cfg->num_heads, cfg->head_dim, cfg->io_dtype == QWM_F32,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return QWM_OK;
}

namespace {

// One compressed cache as a part of the multi-part attention kernel.
void fill_part(const qwm_cache* c, qwm::CachePart& cp) {
  cp.cache = static_cast<const unsigned char*>(c->base);
  cp.calib = static_cast<const unsigned char*>(c->calib);
  cp.n_k = (int)c->n_k;
  cp.tile0 = 0;
}

// Attention of one query chunk over the compressed caches of successive
// epochs (oldest first) and optionally the chunk's own keys and values, in one
// softmax (bf16 activations).
int attention_parts(const qwm_config* cfg, const qwm_cache* caches, int32_t n_caches, const void* q, int64_t n_q,
                    const qwm_strides* st_q, const void* k_loc, const void* v_loc, int64_t n_loc,
                    const qwm_strides* st_k, const qwm_strides* st_v, float scale, void* out,
                    const qwm_strides* st_out, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  if (!caches || n_caches < 1) return QWM_ERR_INVALID_ARG;
  qwm::AttnParams p;
  int s = fill_attn(cfg, &caches[0], q, n_q, st_q, scale, p);
  if (s) return s;
  if (n_caches > qwm::kMaxParts) return QWM_ERR_UNSUPPORTED;
  qwm_layout_info L;
  fill_layout(cfg, &L);
  int64_t total = 0;
  for (int e = 0; e < n_caches; ++e) {
    const qwm_cache* c = &caches[e];
    if (!c->base || !c->calib || c->abi_version != QWM_ABI_VERSION) return QWM_ERR_INVALID_ARG;
    if (c->n_k != c->n_v || c->n_k < 0 || c->n_k > (int64_t)L.token_capacity) return QWM_ERR_STATE;
    total += c->n_k;
  }
  if (cfg->io_dtype != QWM_BF16) return QWM_ERR_UNSUPPORTED;
  if ((s = check_act(cfg, k_loc, n_loc, st_k)) || (s = check_act(cfg, v_loc, n_loc, st_v))) return s;
  if (n_loc > ((int64_t)1 << 30) || total > ((int64_t)1 << 30)) return QWM_ERR_UNSUPPORTED;
  if ((s = check_act(cfg, out, n_q, st_out))) return s;
  if (n_q == 0) return QWM_OK;
  if (lse && !aligned16(lse)) return QWM_ERR_INVALID_ARG;
  if (ws_bytes > 0 && (!workspace || !aligned16(workspace))) return QWM_ERR_INVALID_ARG;
  qwm::PartTable tbl{};
  tbl.n_parts = n_caches;
  for (int e = 0; e < n_caches; ++e) fill_part(&caches[e], tbl.part[e]);
  tbl.idx_k = (int64_t)L.idx_k;
  tbl.idx_v = (int64_t)L.idx_v;
  tbl.codes_k = (int64_t)L.codes_k;
  tbl.codes_v = (int64_t)L.codes_v;
  tbl.params_k = (int64_t)L.params_k;
  tbl.params_v = (int64_t)L.params_v;
  tbl.coef = (int64_t)L.coef;
  tbl.coef_scale = (int64_t)L.coef_scale;
  tbl.mu_k16 = (int64_t)L.mu_k16;
  tbl.mu_v16 = (int64_t)L.mu_v16;
  tbl.ut16 = (int64_t)L.ut16;
  p.n_k = (int)total;
  p.out = out;
  p.o_head_stride = st_out->head;
  p.o_token_stride = st_out->token;
  p.lse = lse;
  p.n_loc = (int)n_loc;
  if (n_loc > 0) {
    p.k_loc = k_loc;
    p.v_loc = v_loc;
    p.kl_head_stride = st_k->head;
    p.kl_token_stride = st_k->token;
    p.vl_head_stride = st_v->head;
    p.vl_token_stride = st_v->token;
  }
  // one cache and no local keys: the single-cache kernel
  return run_attention_bf16(cfg, p, workspace, ws_bytes, stream, (n_caches == 1 && n_loc == 0) ? nullptr : &tbl);
}

}  // namespace

QWM_API int qwm_attention_local(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q,
                                const qwm_strides* st_q, const void* k_loc, const void* v_loc, int64_t n_loc,
                                const qwm_strides* st_k, const qwm_strides* st_v, float scale, void* out,
                                const qwm_strides* st_out, float* lse, void* workspace, size_t ws_bytes,
                                void* stream) {
  return attention_parts(cfg, cache, 1, q, n_q, st_q, k_loc, v_loc, n_loc, st_k, st_v, scale, out, st_out, lse,
                         workspace, ws_bytes, stream);
}

QWM_API int qwm_attention_epochs(const qwm_config* cfg, const qwm_cache* caches, int32_t n_caches, const void* q,
                                 int64_t n_q, const qwm_strides* st_q, const void* k_loc, const void* v_loc,
                                 int64_t n_loc, const qwm_strides* st_k, const qwm_strides* st_v, float scale,
                                 void* out, const qwm_strides* st_out, float* lse, void* workspace, size_t ws_bytes,
                                 void* stream) {
  return attention_parts(cfg, caches, n_caches, q, n_q, st_q, k_loc, v_loc, n_loc, st_k, st_v, scale, out, st_out,
                         lse, workspace, ws_bytes, stream);
}

// ------------------------------------------------- allocation-free attention
// The partial results of qwm_attention_noalloc live in this file-scope device
// array (each GPU the library runs on holds its own copy until the process
// ends).  In host code `scratch` names a host-side stand-in, not device
// memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[QWM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call on each device, with that device current).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return QWM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!ptr) return QWM_ERR_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return QWM_OK;
}
}  // namespace

QWM_API int qwm_attention_noalloc(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q,
                                  const qwm_strides* st_q, float scale, void* out, const qwm_strides* st_out,
                                  float* lse, void* stream) {
  int s = check_config(cfg);
  if (s) return s;
  // the stream-K partial results of bf16 activations must fit in the array
  // (fp32 activations split their key range only as far as it holds them)
  if (cfg->io_dtype == QWM_BF16 && bf16_partial_bytes(cfg) > (size_t)QWM_NOALLOC_SCRATCH_BYTES)
    return QWM_ERR_CAPACITY;
  void* ptr = nullptr;
  if ((s = scratch_address(&ptr))) return s;
  return qwm_attention_timed(cfg, cache, q, n_q, st_q, scale, out, st_out, lse, ptr,
                             (size_t)QWM_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr);
}

QWM_API int qwm_attention(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q,
                          const qwm_strides* st_q, float scale, void* out, const qwm_strides* st_out, float* lse,
                          void* workspace, size_t ws_bytes, void* stream) {
  return qwm_attention_timed(cfg, cache, q, n_q, st_q, scale, out, st_out, lse, workspace, ws_bytes, stream, nullptr,
                             nullptr);
}

QWM_API int qwm_attention_logits(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q,
                                 const qwm_strides* st_q, float scale, float* logits, void* stream) {
  qwm::AttnParams p;
  int s = fill_attn(cfg, cache, q, n_q, st_q, scale, p);
  if (s) return s;
  if (!logits && n_q > 0 && cache->n_k > 0) return QWM_ERR_INVALID_ARG;
  if (n_q == 0 || cache->n_k == 0) return QWM_OK;
  // the debug variant of the attention kernel that the activations' dtype
  // selects (the bf16 kernel, or the fp32 one): the same tile rebuild and
  // S = Q' K~^T, exporting the scaled logits instead of the attention output
  p.logits = logits;
  p.out = nullptr;
  hipError_t e = qwm::launch_attention(p, cfg->num_heads, cfg->head_dim, cfg->io_dtype == QWM_F32,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return QWM_OK;
}

QWM_API int qwm_top1(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q,
                     const qwm_strides* st_q, int32_t* top1, void* stream) {
  qwm::AttnParams p;
  int s = fill_attn(cfg, cache, q, n_q, st_q, 0.f, p);
  if (s) return s;
  if (n_q == 0) return QWM_OK;
  if (!top1 || cache->n_k == 0) return QWM_ERR_INVALID_ARG;
  p.top1 = top1;
  hipError_t e = qwm::launch_attention(p, cfg->num_heads, cfg->head_dim, cfg->io_dtype == QWM_F32,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return QWM_OK;
}

QWM_API int qwm_dense_top1(const qwm_config* cfg, const void* q, int64_t n_q, const qwm_strides* st_q, const void* k,
                           int64_t n_k, const qwm_strides* st_k, int32_t* top1, void* stream) {
  int s = check_config(cfg);
  if (s) return s;
  if ((s = check_act(cfg, q, n_q, st_q)) || (s = check_act(cfg, k, n_k, st_k))) return s;
  if (n_q == 0) return QWM_OK;
  if (!top1 || n_k == 0) return QWM_ERR_INVALID_ARG;
  hipError_t e = qwm::launch_dense_top1(q, st_q->head, st_q->token, (int)n_q, k, st_k->head, st_k->token, (int)n_k,
                                        cfg->num_heads, cfg->head_dim, cfg->io_dtype == QWM_F32, top1,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return QWM_OK;
}
