// Host side of the TurboQuant KV-cache library: the Lloyd-Max solver, the
// seeded parameter draw, the record layout, context management, argument
// validation and error reporting.  Kernels live in tq_quantize.hip and
// tq_decode.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "tq_api.h"
#include "tq_internal.h"

namespace tq {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

// ---------------------------------------------------------------------------
// Lloyd-Max codebook of one coordinate U of a uniform point on S^(d-1).
// Hub, technical principle steps 1-2: after the random rotation each
// coordinate follows a Beta-type law and the method precomputes optimal
// scalar codebooks for it.  U has density f(u) = (1-u^2)^m / B on [-1, 1] with
// m = (d-3)/2.  Cell masses use the exact reduction formula
//   J_m(a,b) = int_a^b (1-u^2)^m du
//            = [u (1-u^2)^m]_a^b / (2m+1) + 2m/(2m+1) J_{m-1}(a,b),
// started from J_{1/2} = [(u sqrt(1-u^2) + asin u)/2] (half-integer m, even d)
// or J_0 = b - a (integer m); the recursion only ever multiplies earlier
// errors by 2m/(2m+1) < 1.  Cell first moments are closed-form:
//   int_a^b u (1-u^2)^m du = ((1-a^2)^(m+1) - (1-b^2)^(m+1)) / (2(m+1)).
// ---------------------------------------------------------------------------
namespace {

double pow_1mu2(double u, double e) {
  double w = 1.0 - u * u;
  if (w <= 0.0) return 0.0;
  return std::pow(w, e);
}

double J(double a, double b, int twice_m) {
  // twice_m = 2m = d - 3
  double acc;
  int start;
  if (twice_m % 2 == 1) {
    auto F = [](double u) { return 0.5 * (u * std::sqrt(std::max(0.0, 1.0 - u * u)) + std::asin(u)); };
    acc = F(b) - F(a);
    start = 3;  // 2m = 3, 5, ...
  } else {
    acc = b - a;
    start = 2;
  }
  for (int tm = start; tm <= twice_m; tm += 2) {
    double m = 0.5 * tm;
    double T = b * pow_1mu2(b, m) - a * pow_1mu2(a, m);
    acc = T / (2.0 * m + 1.0) + (2.0 * m / (2.0 * m + 1.0)) * acc;
  }
  return acc;
}

double first_moment(double a, double b, int twice_m) {
  double mp1 = 0.5 * twice_m + 1.0;
  return (pow_1mu2(a, mp1) - pow_1mu2(b, mp1)) / (2.0 * mp1);
}

}  // namespace

}  // namespace tq

using namespace tq;

namespace {
// Lloyd's conditions t_j = (c_j + c_{j+1}) / 2, with c_k the conditional mean
// of cell k = (t_{k-1}, t_k], solved by Newton's method on the L - 1
// thresholds.  Lloyd's iteration contracts by only ~1 - O(1/L^2) per step,
// so with many levels (more than 4 bits) it is run a little and this
// finishes the fixed point.  A cell's mean moves with its edges as
// dc_k/dt_k = f(t_k)(t_k - c_k)/P_k and dc_k/dt_{k-1} = f(t_{k-1})(c_k - t_{k-1})/P_k,
// so the Jacobian is tridiagonal (Thomas algorithm); steps are halved until
// the thresholds stay ordered in (-1, 1) and the residual drops, and the
// iterate is kept odd-symmetric.  c: centroids in, centroids out.
void newton_refine(int d, std::vector<double>& c) {
  const int L = (int)c.size(), n = L - 1, tm = d - 3;
  const double m = 0.5 * tm;
  std::vector<double> t(n), P(L), cc(L), F(n), tn(n), Pn(L), ccn(L), Fn(n);
  std::vector<double> a(n), b(n), cu(n), delta(n);
  for (int k = 0; k < n; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
  // cell masses and the density without the normaliser B (it cancels in
  // the means and in f / P)
  auto eval = [&](const std::vector<double>& tt, std::vector<double>& PP, std::vector<double>& CC, std::vector<double>& FF) {
    double fmax = 0.0;
    for (int k = 0; k < L; ++k) {
      const double lo = k == 0 ? -1.0 : tt[k - 1], hi = k == L - 1 ? 1.0 : tt[k];
      PP[k] = J(lo, hi, tm);
      CC[k] = first_moment(lo, hi, tm) / PP[k];
    }
    for (int j = 0; j < n; ++j) {
      FF[j] = tt[j] - 0.5 * (CC[j] + CC[j + 1]);
      fmax = std::max(fmax, std::fabs(FF[j]));
    }
    return fmax;
  };
  double f0 = eval(t, P, cc, F);
  for (int it = 0; it < 200; ++it) {
    double cmax = 0.0;
    for (int k = 0; k < L; ++k) cmax = std::max(cmax, std::fabs(cc[k]));
    if (f0 <= 1e-15 * cmax) break;
    for (int j = 0; j < n; ++j) {
      const double fj = pow_1mu2(t[j], m);  // (1 - t^2)^m, the density times B
      const double up = fj * (t[j] - cc[j]) / P[j];          // dc_j / dt_j
      const double lo = fj * (cc[j + 1] - t[j]) / P[j + 1];  // dc_{j+1} / dt_j
      b[j] = 1.0 - 0.5 * (up + lo);
      if (j + 1 < n) a[j + 1] = -0.5 * lo;  // dF_{j+1} / dt_j
      if (j > 0) cu[j - 1] = -0.5 * up;     // dF_{j-1} / dt_j
    }
    // tridiagonal solve (Thomas): a sub-, b main, cu super-diagonal
    std::vector<double> cp(n), dp(n);
    cp[0] = n > 1 ? cu[0] / b[0] : 0.0;
    dp[0] = -F[0] / b[0];
    for (int j = 1; j < n; ++j) {
      const double den = b[j] - a[j] * cp[j - 1];
      cp[j] = j + 1 < n ? cu[j] / den : 0.0;
      dp[j] = (-F[j] - a[j] * dp[j - 1]) / den;
    }
    delta[n - 1] = dp[n - 1];
    for (int j = n - 2; j >= 0; --j) delta[j] = dp[j] - cp[j] * delta[j + 1];
    double lam = 1.0, fn = 0.0;
    bool ok = false;
    while (lam >= 1e-12) {
      for (int j = 0; j < n; ++j) tn[j] = t[j] + lam * delta[j];
      for (int j = 0; j < n / 2; ++j) {
        const double s = 0.5 * (tn[j] - tn[n - 1 - j]);
        tn[j] = s;
        tn[n - 1 - j] = -s;
      }
      if (n % 2) tn[n / 2] = 0.0;
      bool ordered = tn[0] > -1.0 && tn[n - 1] < 1.0;
      for (int j = 1; j < n && ordered; ++j) ordered = tn[j] > tn[j - 1];
      if (ordered) {
        fn = eval(tn, Pn, ccn, Fn);
        if (fn < f0 || lam < 1e-6) {
          ok = true;
          break;
        }
      }
      lam *= 0.5;
    }
    if (!ok) break;
    t.swap(tn);
    P.swap(Pn);
    cc.swap(ccn);
    F.swap(Fn);
    f0 = fn;
  }
  for (int k = 0; k < L; ++k) c[k] = 0.5 * (cc[k] - cc[L - 1 - k]);
}
}  // namespace

extern "C" int tq_lloyd_max(int32_t d, int32_t bits, double* centroids, double* thresholds) {
  if (d < 4 || (d & 1) || bits < 1 || bits > 8 || !centroids || !thresholds) {
    set_error("tq_lloyd_max: need even head_dim >= 4, bits in 1..8 and non-NULL outputs");
    return TQ_EINVAL;
  }
  const int L = 1 << bits;
  const int tm = d - 3;
  // Start from levels spread evenly over +-2/sqrt(d) (where the density is
  // far from underflow); the law is log-concave, so Lloyd's iteration has a
  // single fixed point and converges to it from any ordered start.
  std::vector<double> c(L), t(L - 1), cn(L), lo(L), hi(L);
  for (int k = 0; k < L; ++k) c[k] = (2.0 * k + 1.0 - L) / L * 2.0 / std::sqrt((double)d);
  // with more than four levels Lloyd's iteration is run only to bring the
  // codebook near the fixed point, which newton_refine then solves (the
  // plain iteration would take seconds at 3-4 bits and never finish at 8)
  const int lloyd_iters = bits <= 1 ? 100000 : 200;
  for (int it = 0; it < lloyd_iters; ++it) {
    for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
    for (int k = 0; k < L; ++k) {
      double a = k == 0 ? -1.0 : t[k - 1];
      double b = k == L - 1 ? 1.0 : t[k];
      cn[k] = first_moment(a, b, tm) / J(a, b, tm);
    }
    // the density is even: keep the iterate exactly odd-symmetric
    double delta = 0.0, cmax = 0.0;
    for (int k = 0; k < L; ++k) {
      double s = 0.5 * (cn[k] - cn[L - 1 - k]);
      delta = std::max(delta, std::fabs(s - c[k]));
      cmax = std::max(cmax, std::fabs(s));
      lo[k] = s;
    }
    c = lo;
    if (delta <= 1e-15 * cmax) break;
  }
  if (bits > 1) newton_refine(d, c);
  for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
  std::memcpy(centroids, c.data(), sizeof(double) * L);
  std::memcpy(thresholds, t.data(), sizeof(double) * (L - 1));
  return TQ_OK;
}

// ---------------------------------------------------------------------------
// Uniform codebook (Roadmap §4.3, the "tq4u" mode: equally spaced centroids,
// dequantised as idx * step + c0).  The page fixes the spacing rule only as
// "linear"; the step taken here is the one of least mean squared error for
// the same rotated-coordinate law: centroids c_k = a_k step with
// a_k = k - (L-1)/2 (c0 = -(L-1) step / 2), thresholds at the midpoints.  With
// cells moving with the step, the midpoint thresholds make the boundary terms
// of dD/dstep vanish, so the optimum is the root of
//   F(step) = sum_k a_k (M1_k - a_k step M0_k),
// M0_k, M1_k the mass and first moment of cell k.  F > 0 for small steps and
// < 0 for large ones; the root is bracketed and found by bisection to the
// last bit.
// ---------------------------------------------------------------------------
extern "C" int tq_uniform_codebook(int32_t d, int32_t bits, double* centroids, double* thresholds) {
  if (d < 4 || (d & 1) || bits < 1 || bits > 8 || !centroids || !thresholds) {
    set_error("tq_uniform_codebook: need even head_dim >= 4, bits in 1..8 and non-NULL outputs");
    return TQ_EINVAL;
  }
  const int L = 1 << bits;
  const int tm = d - 3;
  auto F = [&](double step) {
    double acc = 0.0;
    for (int k = 0; k < L; ++k) {
      const double ak = k - 0.5 * (L - 1);
      // cell k = (midpoint below, midpoint above), cut to the support [-1, 1]
      const double a = k == 0 ? -1.0 : std::min(1.0, std::max(-1.0, (ak - 0.5) * step));
      const double b = k == L - 1 ? 1.0 : std::min(1.0, std::max(-1.0, (ak + 0.5) * step));
      acc += ak * (first_moment(a, b, tm) - ak * step * J(a, b, tm));
    }
    return acc;
  };
  double lo = 1e-4 / std::sqrt((double)d), hi = 8.0 / std::sqrt((double)d);
  if (!(F(lo) > 0.0) || !(F(hi) < 0.0)) {
    set_error("tq_uniform_codebook: no sign change of the stationarity condition for d %d bits %d", d, bits);
    return TQ_EINVAL;
  }
  for (int it = 0; it < 200 && hi - lo > 0.0; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    (F(mid) > 0.0 ? lo : hi) = mid;
  }
  const double step = 0.5 * (lo + hi);
  for (int k = 0; k < L; ++k) centroids[k] = (k - 0.5 * (L - 1)) * step;
  for (int k = 0; k + 1 < L; ++k) thresholds[k] = 0.5 * (centroids[k] + centroids[k + 1]);
  return TQ_OK;
}

// ---------------------------------------------------------------------------
// Seeded draw of D1, D2 and S (splitmix64 counter stream).
// ---------------------------------------------------------------------------
namespace {
uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}
uint64_t stream_at(uint64_t seed, uint64_t i) { return splitmix64(seed ^ (0x9E3779B97F4A7C15ull * (i + 1))); }
}  // namespace

extern "C" int tq_draw_params(uint64_t seed, int32_t d, int8_t* signs, float* S) {
  if (d <= 0 || d > 4096) {
    set_error("tq_draw_params: head_dim out of range");
    return TQ_EINVAL;
  }
  if (signs)
    for (int i = 0; i < 2 * d; ++i) signs[i] = (stream_at(seed, i) >> 63) ? int8_t(-1) : int8_t(1);
  if (S) {
    const double two_pi = 6.283185307179586476925286766559;
    uint64_t base = 2ull * d;
    for (int64_t m = 0; m < (int64_t)d * d / 2; ++m) {
      double u1 = ((stream_at(seed, base + 2 * m) >> 11) + 1) * 0x1.0p-53;
      double u2 = (stream_at(seed, base + 2 * m + 1) >> 11) * 0x1.0p-53;
      double r = std::sqrt(-2.0 * std::log(u1));
      S[2 * m] = (float)(r * std::cos(two_pi * u2));
      S[2 * m + 1] = (float)(r * std::sin(two_pi * u2));
    }
  }
  return TQ_OK;
}

// ---------------------------------------------------------------------------
// Paged record layout (iThome: block table + paged KV cache; the byte layout
// is this library's own: 16-slot records, each region 16-byte aligned).
// ---------------------------------------------------------------------------
Layout tq::make_layout(int d, int kb, int vb, bool qjl) {
  Layout l;
  int64_t o = 0;
  l.kcodes = o; o += 16 * (kb * d / 8);
  l.kqjl = o;   o += qjl ? 16 * (d / 8) : 0;
  l.kmeta = o;  o += 16 * (qjl ? 4 : 2);
  l.vcodes = o; o += (vb * d / 8) * 16;
  l.vmeta = o;  o += (d / 32) * 16 * 4;
  l.bytes = o;
  return l;
}

namespace {
int check_preset(const tq_preset* p) {
  if (!p) {
    set_error("preset is NULL");
    return TQ_EINVAL;
  }
  const bool mse = (p->flags & TQ_PRESET_MSE_ONLY) != 0;
  const bool kb_ok = (p->k_bits >= 2 && p->k_bits <= 4) || (p->k_bits == 8 && mse);
  if ((p->head_dim != 128 && p->head_dim != 256) || !kb_ok || (p->v_bits != 2 && p->v_bits != 4) ||
      p->v_group != 32 || p->block_size != 16 ||
      (p->flags & ~(TQ_PRESET_MSE_ONLY | TQ_PRESET_UNIFORM | TQ_PRESET_ROTATE_V)) != 0) {
    set_error("unsupported preset: head_dim %d k_bits %d v_bits %d v_group %d block_size %d flags %d "
              "(supported: head_dim 128|256, k_bits 2..4, or 8 with TQ_PRESET_MSE_ONLY, v_bits 2|4, v_group 32, "
              "block_size 16, flags: an or of TQ_PRESET_MSE_ONLY, TQ_PRESET_UNIFORM, TQ_PRESET_ROTATE_V)",
              p->head_dim, p->k_bits, p->v_bits, p->v_group, p->block_size, p->flags);
    return TQ_EUNSUPPORTED;
  }
  return TQ_OK;
}

uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}
float f16_bits_to_f32(uint16_t b) {
  _Float16 h;
  std::memcpy(&h, &b, 2);
  return (float)h;
}
uint16_t f32_to_bf16_bits(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return (uint16_t)u;
}
float bf16_bits_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
}  // namespace

extern "C" int tq_record_layout(const tq_preset* p, tq_layout* out) {
  int rc = check_preset(p);
  if (rc) return rc;
  if (!out) {
    set_error("tq_record_layout: out is NULL");
    return TQ_EINVAL;
  }
  Layout l = make_layout(p->head_dim, p->k_bits, p->v_bits, (p->flags & TQ_PRESET_MSE_ONLY) == 0);
  out->kcodes = l.kcodes;
  out->kqjl = l.kqjl;
  out->kmeta = l.kmeta;
  out->vcodes = l.vcodes;
  out->vmeta = l.vmeta;
  out->record_bytes = l.bytes;
  return TQ_OK;
}

// ---------------------------------------------------------------------------
// Context
// ---------------------------------------------------------------------------
extern "C" int tq_codebook_init(const tq_preset* p, const int8_t* signs, const float* S, tq_ctx** out) {
  int rc = check_preset(p);
  if (rc) return rc;
  if (!out) {
    set_error("tq_codebook_init: out is NULL");
    return TQ_EINVAL;
  }
  *out = nullptr;
  const int d = p->head_dim, kb = p->k_bits, vb = p->v_bits, L = 1 << kb;
  if (signs) {
    for (int i = 0; i < 2 * d; ++i)
      if (signs[i] != 1 && signs[i] != -1) {
        set_error("tq_codebook_init: signs[%d] = %d is not +-1", i, (int)signs[i]);
        return TQ_EINVAL;
      }
  }
  if (S) {
    for (int64_t i = 0; i < (int64_t)d * d; ++i)
      if (!std::isfinite(S[i]) || std::fabs(S[i]) >= 2048.0f) {
        set_error("tq_codebook_init: S[%lld] is not a finite value below 2048 in magnitude", (long long)i);
        return TQ_EINVAL;
      }
  }
  tq_ctx* c = new (std::nothrow) tq_ctx();
  if (!c) {
    set_error("tq_codebook_init: out of host memory");
    return TQ_ENOMEM;
  }
  c->preset = *p;
  c->d = d;
  c->kb = kb;
  c->vb = vb;
  c->qjl = (p->flags & TQ_PRESET_MSE_ONLY) == 0;
  c->rotv = (p->flags & TQ_PRESET_ROTATE_V) != 0;
  c->lay = make_layout(d, kb, vb, c->qjl);
  c->c64.resize(L);
  c->t64.resize(L - 1);
  if (p->flags & TQ_PRESET_UNIFORM)
    tq_uniform_codebook(d, kb, c->c64.data(), c->t64.data());
  else
    tq_lloyd_max(d, kb, c->c64.data(), c->t64.data());
  c->c32.resize(L);
  c->t32.resize(L - 1);
  for (int k = 0; k < L; ++k) c->c32[k] = (float)c->c64[k];
  for (int k = 0; k + 1 < L; ++k) c->t32[k] = (float)c->t64[k];
  c->signs.resize(2 * d);
  c->S.resize((size_t)d * d);
  if (signs)
    std::memcpy(c->signs.data(), signs, 2 * d);
  else
    tq_draw_params(p->seed, d, c->signs.data(), nullptr);
  if (S)
    std::memcpy(c->S.data(), S, sizeof(float) * d * d);
  else
    tq_draw_params(p->seed, d, nullptr, c->S.data());

  // ---- host images of the device tables
  std::vector<float> sg1(d), sg2(d);
  for (int i = 0; i < d; ++i) {
    sg1[i] = (float)c->signs[i];
    sg2[i] = (float)c->signs[d + i];
  }
  const int NT = d / 16, KT = d / 32;
  std::vector<uint16_t> tiles((size_t)NT * KT * 2 * 64 * 8), tiles_d2(tiles.size());
  const float sscale = std::ldexp(1.0f, kSScaleLog2);
  for (int nt = 0; nt < NT; ++nt)
    for (int kt = 0; kt < KT; ++kt)
      for (int l = 0; l < 64; ++l)
        for (int e = 0; e < 8; ++e) {
          int row = 16 * nt + (l % 16);
          int col = 32 * kt + 8 * (l / 16) + e;
          float v = c->S[(size_t)row * d + col] * sscale;
          uint16_t h = f32_to_f16_bits(v);
          uint16_t lo = f32_to_f16_bits(v - f16_bits_to_f32(h));
          size_t base = (((size_t)nt * KT + kt) * 2) * 64 * 8;
          tiles[base + (size_t)l * 8 + e] = h;
          tiles[base + 64 * 8 + (size_t)l * 8 + e] = lo;
          const uint16_t flip = sg2[col] < 0.f ? 0x8000u : 0u;  // fp16 sign bit
          tiles_d2[base + (size_t)l * 8 + e] = h ^ flip;
          tiles_d2[base + 64 * 8 + (size_t)l * 8 + e] = lo ^ flip;
        }
  // the same S diag(D2) tiles with the k index permuted the way the
  // head_dim-128 store kernel holds its residual (d = 128 only)
  std::vector<uint16_t> tiles_perm(d == 128 ? tiles.size() : 0);
  if (d == 128)
    for (int nt = 0; nt < NT; ++nt)
      for (int kt = 0; kt < KT; ++kt)
        for (int l = 0; l < 64; ++l)
          for (int e = 0; e < 8; ++e) {
            int row = 16 * nt + (l % 16);
            int col = 32 * kt + 16 * (e / 4) + 4 * (l / 16) + e % 4;
            float v = c->S[(size_t)row * d + col] * sscale;
            uint16_t h = f32_to_f16_bits(v);
            uint16_t lo = f32_to_f16_bits(v - f16_bits_to_f32(h));
            const uint16_t flip = sg2[col] < 0.f ? 0x8000u : 0u;
            size_t base = (((size_t)nt * KT + kt) * 2) * 64 * 8;
            tiles_perm[base + (size_t)l * 8 + e] = h ^ flip;
            tiles_perm[base + 64 * 8 + (size_t)l * 8 + e] = lo ^ flip;
          }
  // two-code pair tables (2-4-bit keys; 8-bit keys would need 65,536 pairs)
  const int P = kb <= 4 ? 1 << (2 * kb) : 0;
  std::vector<uint32_t> pair((size_t)P * 2);
  for (int idx = 0; idx < P; ++idx) {
    int a = idx & (L - 1), b = idx >> kb;
    uint16_t ha = f32_to_bf16_bits(c->c32[a]), hb = f32_to_bf16_bits(c->c32[b]);
    uint16_t la = f32_to_bf16_bits(c->c32[a] - bf16_bits_to_f32(ha));
    uint16_t lb = f32_to_bf16_bits(c->c32[b] - bf16_bits_to_f32(hb));
    pair[2 * idx] = (uint32_t)ha | ((uint32_t)hb << 16);
    pair[2 * idx + 1] = (uint32_t)la | ((uint32_t)lb << 16);
  }
  std::vector<uint32_t> pair16((size_t)P * 2);
  for (int idx = 0; idx < P; ++idx) {
    int a = idx & (L - 1), b = idx >> kb;
    uint16_t ha = f32_to_f16_bits(c->c32[a]), hb = f32_to_f16_bits(c->c32[b]);
    uint16_t la = f32_to_f16_bits(c->c32[a] - f16_bits_to_f32(ha));
    uint16_t lb = f32_to_f16_bits(c->c32[b] - f16_bits_to_f32(hb));
    pair16[2 * idx] = (uint32_t)ha | ((uint32_t)hb << 16);
    pair16[2 * idx + 1] = (uint32_t)la | ((uint32_t)lb << 16);
  }

  // one-code table (the 8-bit decode): entry a = bf16 hi | bf16 lo << 16 of c[a]
  std::vector<uint32_t> code1((size_t)L);
  for (int a = 0; a < L; ++a) {
    const uint16_t h = f32_to_bf16_bits(c->c32[a]);
    const uint16_t l = f32_to_bf16_bits(c->c32[a] - bf16_bits_to_f32(h));
    code1[a] = (uint32_t)h | ((uint32_t)l << 16);
  }

  // ---- one device allocation, 256-byte aligned pieces
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t o_c = 0, o_t = up(o_c + 4 * L), o_s1 = up(o_t + 4 * L), o_s2 = up(o_s1 + 4 * d), o_S = up(o_s2 + 4 * d),
         o_tiles = up(o_S + 4 * (size_t)d * d), o_tiles2 = up(o_tiles + 2 * tiles.size()),
         o_pair = up(o_tiles2 + 2 * tiles_d2.size()), o_pair16 = up(o_pair + 4 * pair.size()),
         o_perm = up(o_pair16 + 4 * pair16.size()), o_code1 = up(o_perm + 2 * tiles_perm.size()),
         total = up(o_code1 + 4 * code1.size());
  if (hipGetDevice(&c->device) != hipSuccess) {
    set_error("tq_codebook_init: no HIP device");
    delete c;
    return TQ_EHIP;
  }
  if (hipMalloc(&c->dev_block, total) != hipSuccess) {
    set_error("tq_codebook_init: hipMalloc of %zu bytes failed", total);
    delete c;
    return TQ_ENOMEM;
  }
  char* base = (char*)c->dev_block;
  std::vector<char> img(total, 0);
  std::memcpy(img.data() + o_c, c->c32.data(), 4 * L);
  std::memcpy(img.data() + o_t, c->t32.data(), 4 * (L - 1));
  std::memcpy(img.data() + o_s1, sg1.data(), 4 * d);
  std::memcpy(img.data() + o_s2, sg2.data(), 4 * d);
  std::memcpy(img.data() + o_S, c->S.data(), 4 * (size_t)d * d);
  std::memcpy(img.data() + o_tiles, tiles.data(), 2 * tiles.size());
  std::memcpy(img.data() + o_tiles2, tiles_d2.data(), 2 * tiles_d2.size());
  std::memcpy(img.data() + o_pair, pair.data(), 4 * pair.size());
  std::memcpy(img.data() + o_pair16, pair16.data(), 4 * pair16.size());
  if (!tiles_perm.empty()) std::memcpy(img.data() + o_perm, tiles_perm.data(), 2 * tiles_perm.size());
  std::memcpy(img.data() + o_code1, code1.data(), 4 * code1.size());
  if (hipMemcpy(base, img.data(), total, hipMemcpyHostToDevice) != hipSuccess) {
    set_error("tq_codebook_init: upload failed");
    (void)hipFree(c->dev_block);
    delete c;
    return TQ_EHIP;
  }
  c->dev.centroids = (const float*)(base + o_c);
  c->dev.thresholds = (const float*)(base + o_t);
  c->dev.signs1 = (const float*)(base + o_s1);
  c->dev.signs2 = (const float*)(base + o_s2);
  c->dev.S = (const float*)(base + o_S);
  c->dev.s_tiles = (const uint16_t*)(base + o_tiles);
  c->dev.s_tiles_d2 = (const uint16_t*)(base + o_tiles2);
  c->dev.pair_lut = (const uint32_t*)(base + o_pair);
  c->dev.pair_lut_f16 = (const uint32_t*)(base + o_pair16);
  c->dev.s_tiles_perm_d2 = tiles_perm.empty() ? nullptr : (const uint16_t*)(base + o_perm);
  c->dev.code_lut = (const uint32_t*)(base + o_code1);
  // equally spaced codebook: c_k = (k - (L-1)/2) step, so c[1] - c[0] is the step
  c->dev.uni_step = (p->flags & TQ_PRESET_UNIFORM) ? (float)(c->c64[1] - c->c64[0]) : 0.f;
  *out = c;
  return TQ_OK;
}

extern "C" int tq_ctx_destroy(tq_ctx* c) {
  if (!c) return TQ_OK;
  int rc = TQ_OK;
  if (c->dev_block) {
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(c->device);
    if (hipFree(c->dev_block) != hipSuccess) {
      set_error("tq_ctx_destroy: hipFree failed");
      rc = TQ_EHIP;
    }
    (void)hipSetDevice(prev);
  }
  delete c;
  return rc;
}

extern "C" int tq_ctx_tables(const tq_ctx* c, float* centroids, float* thresholds, int8_t* signs, float* S) {
  if (!c) {
    set_error("tq_ctx_tables: ctx is NULL");
    return TQ_EINVAL;
  }
  if (centroids) std::memcpy(centroids, c->c32.data(), 4 * c->c32.size());
  if (thresholds) std::memcpy(thresholds, c->t32.data(), 4 * c->t32.size());
  if (signs) std::memcpy(signs, c->signs.data(), c->signs.size());
  if (S) std::memcpy(S, c->S.data(), 4 * c->S.size());
  return TQ_OK;
}

extern "C" int tq_ctx_preset(const tq_ctx* c, tq_preset* out) {
  if (!c || !out) {
    set_error("tq_ctx_preset: NULL argument");
    return TQ_EINVAL;
  }
  *out = c->preset;
  return TQ_OK;
}

extern "C" int tq_fold_output_projection(int32_t d, const int8_t* signs, const float* w_o, int64_t rows,
                                         int32_t num_q_heads, float* out) {
  if (d < 2 || d > 4096 || (d & (d - 1)) || !signs || !w_o || !out || rows < 0 || num_q_heads <= 0) {
    set_error("tq_fold_output_projection: need head_dim a power of two in 2..4096, non-NULL arrays, rows >= 0 "
              "and num_q_heads > 0");
    return TQ_EINVAL;
  }
  for (int i = 0; i < 2 * d; ++i)
    if (signs[i] != 1 && signs[i] != -1) {
      set_error("tq_fold_output_projection: signs[%d] = %d is not +-1", i, (int)signs[i]);
      return TQ_EINVAL;
    }
  const double inv_sqrt_d = 1.0 / std::sqrt((double)d);
  std::vector<double> y(d);
  for (int64_t r = 0; r < rows; ++r)
    for (int h = 0; h < num_q_heads; ++h) {
      const size_t base = (size_t)r * num_q_heads * d + (size_t)h * d;
      // row block w times Pi^-1 = (Pi w^T)^T: D1, Hadamard butterflies, D2
      for (int j = 0; j < d; ++j) y[j] = (double)w_o[base + j] * (double)signs[j];
      for (int hs = 1; hs < d; hs <<= 1)
        for (int j = 0; j < d; ++j)
          if ((j & hs) == 0) {
            const double a = y[j], b = y[j + hs];
            y[j] = a + b;
            y[j + hs] = a - b;
          }
      for (int j = 0; j < d; ++j) out[base + j] = (float)(y[j] * inv_sqrt_d * (double)signs[d + j]);
    }
  return TQ_OK;
}

extern "C" size_t tq_block_bytes(const tq_ctx* c) { return c ? (size_t)c->lay.bytes : 0; }

extern "C" const char* tq_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------------------
// Quantise / store
// ---------------------------------------------------------------------------
extern "C" int tq_quantize_store(const tq_ctx* c, const void* k, const void* v, int32_t in_dtype, int64_t num_tokens,
                                 int32_t num_kv_heads, const int32_t* slot_mapping, void* pool, int64_t num_blocks,
                                 void* stream) {
  if (!c) {
    set_error("tq_quantize_store: ctx is NULL");
    return TQ_EINVAL;
  }
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) {
    set_error("tq_quantize_store: num_tokens %lld num_kv_heads %d num_blocks %lld out of range",
              (long long)num_tokens, num_kv_heads, (long long)num_blocks);
    return TQ_EINVAL;
  }
  if (in_dtype != TQ_DTYPE_BF16 && in_dtype != TQ_DTYPE_F32) {
    set_error("tq_quantize_store: in_dtype %d is neither TQ_DTYPE_BF16 nor TQ_DTYPE_F32", in_dtype);
    return TQ_EINVAL;
  }
  if (num_tokens == 0) return TQ_OK;
  if (!k || !v || !slot_mapping || !pool) {
    set_error("tq_quantize_store: NULL device pointer");
    return TQ_EINVAL;
  }
  if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)pool) & 15) {
    set_error("tq_quantize_store: k, v and pool must be 16-byte aligned");
    return TQ_EINVAL;
  }
  if (num_tokens * num_kv_heads > (int64_t)1 << 40) {
    set_error("tq_quantize_store: too many token-heads");
    return TQ_EINVAL;
  }
  hipError_t e = launch_quantize(c, k, v, in_dtype, num_tokens, num_kv_heads, slot_mapping, pool, num_blocks,
                                 (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("tq_quantize_store: launch failed: %s", hipGetErrorString(e));
    return TQ_EHIP;
  }
  return TQ_OK;
}

// ---------------------------------------------------------------------------
// Decode
// ---------------------------------------------------------------------------
namespace {
int check_decode_shape(const tq_decode_args* a) {
  if (!a) {
    set_error("decode args are NULL");
    return TQ_EINVAL;
  }
  if (a->num_presets < 1 || a->num_presets > 2 || !a->ctx[0] || (a->num_presets == 2 && !a->ctx[1])) {
    set_error("decode: num_presets must be 1 or 2 with a context per preset");
    return TQ_EINVAL;
  }
  const int d = a->ctx[0]->d;
  if (a->num_presets == 2 && a->ctx[1]->d != d) {
    set_error("decode: both presets must share head_dim");
    return TQ_EINVAL;
  }
  if (a->batch < 0 || a->batch > 8192 || a->num_q_heads <= 0 || a->num_kv_heads <= 0 ||
      a->num_q_heads % a->num_kv_heads) {
    set_error("decode: batch %d, num_q_heads %d, num_kv_heads %d invalid", a->batch, a->num_q_heads,
              a->num_kv_heads);
    return TQ_EINVAL;
  }
  for (int i = 0; i < a->num_presets; ++i) {
    if ((int64_t)a->num_kv_heads * a->ctx[i]->lay.bytes >= ((int64_t)1 << 31)) {
      set_error("decode: num_kv_heads %d x %d-byte records per block exceeds 2^31 bytes", a->num_kv_heads,
                (int)a->ctx[i]->lay.bytes);
      return TQ_EUNSUPPORTED;
    }
  }
  int G = a->num_q_heads / a->num_kv_heads;
  if (G > 8) {
    set_error("decode: query heads per KV head %d > 8 is not supported", G);
    return TQ_EUNSUPPORTED;
  }
  if (a->chunk_tokens < 32 || a->chunk_tokens % 32 || a->chunk_tokens > 8192) {
    set_error("decode: chunk_tokens %d must be a multiple of 32 in [32, 8192]", a->chunk_tokens);
    return TQ_EINVAL;
  }
  if (a->max_seq_len < 0 || a->max_blocks_per_seq < 0 || (int64_t)a->max_seq_len > 16ll * a->max_blocks_per_seq) {
    set_error("decode: max_seq_len %d exceeds 16 * max_blocks_per_seq %d", a->max_seq_len, a->max_blocks_per_seq);
    return TQ_EINVAL;
  }
  if ((int64_t)(a->max_seq_len + a->chunk_tokens - 1) / a->chunk_tokens + 1 > 1024) {
    set_error("decode: max_seq_len %d / chunk_tokens %d gives more than 1023 splits per sequence", a->max_seq_len,
              a->chunk_tokens);
    return TQ_EINVAL;
  }
  if ((a->recent_k == nullptr) != (a->recent_v == nullptr) || (a->recent_k == nullptr) != (a->recent_lens == nullptr)) {
    set_error("decode: recent_k, recent_v and recent_lens must be all set or all NULL");
    return TQ_EINVAL;
  }
  if (a->flags & ~(int32_t)TQ_DECODE_DETERMINISTIC) {
    set_error("decode: unknown flags 0x%x", (unsigned)a->flags);
    return TQ_EINVAL;
  }
  if (a->recent_k && (a->recent_window <= 0 || a->recent_window > 4096)) {
    set_error("decode: recent_window %d out of range 1..4096", a->recent_window);
    return TQ_EINVAL;
  }
  return TQ_OK;
}
}  // namespace

DecodePlan tq::plan_decode(const tq_decode_args* a) {
  DecodePlan p{};
  p.d = a->ctx[0]->d;
  p.G = a->num_q_heads / a->num_kv_heads;
  p.chunk = a->chunk_tokens;
  p.num_splits_max = (a->max_seq_len + a->chunk_tokens - 1) / a->chunk_tokens + (a->recent_k ? 1 : 0);
  if (p.num_splits_max < 1) p.num_splits_max = 1;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t nq = (size_t)a->batch * a->num_q_heads;
  p.off_part = 0;
  p.bytes = up(p.off_part + 4 * nq * (size_t)p.num_splits_max * (p.d + 2));
  return p;
}

extern "C" size_t tq_decode_workspace_bytes(const tq_decode_args* a) {
  if (check_decode_shape(a)) return 0;
  return plan_decode(a).bytes;
}

// Shared by tq_decode_attention and tq_decode_attention_noalloc; with
// noalloc the workspace fields are ignored and the library's static scratch
// array takes their place.
static int decode_entry(const tq_decode_args* a, void* stream, bool noalloc) {
  const char* who = noalloc ? "tq_decode_attention_noalloc" : "tq_decode_attention";
  int rc = check_decode_shape(a);
  if (rc) return rc;
  if (a->batch == 0) return TQ_OK;
  if (!a->q || !a->block_tables || !a->seq_lens || !a->out || !a->pool[0] || (a->num_presets == 2 && !a->pool[1])) {
    set_error("%s: NULL device pointer", who);
    return TQ_EINVAL;
  }
  if (a->q_dtype != TQ_DTYPE_BF16 && a->q_dtype != TQ_DTYPE_F32) {
    set_error("%s: q_dtype %d invalid", who, a->q_dtype);
    return TQ_EINVAL;
  }
  if (((uintptr_t)a->pool[0] | (uintptr_t)a->pool[1] | (uintptr_t)a->q) & 15) {
    set_error("%s: q and pools must be 16-byte aligned", who);
    return TQ_EINVAL;
  }
  if (a->scores_out && a->scores_stride < a->max_seq_len + (a->recent_k ? a->recent_window : 0)) {
    set_error("%s: scores_stride %d too small", who, a->scores_stride);
    return TQ_EINVAL;
  }
  DecodePlan plan = plan_decode(a);
  tq_decode_args args = *a;
  if (noalloc) {
    if (plan.bytes > TQ_NOALLOC_SCRATCH_BYTES) {
      set_error("%s: the split partials need %zu bytes, above the %zu-byte static scratch", who, plan.bytes,
                (size_t)TQ_NOALLOC_SCRATCH_BYTES);
      return TQ_EINVAL;
    }
    void* p = nullptr;
    hipError_t e = noalloc_scratch(&p);
    if (e != hipSuccess) {
      set_error("%s: hipGetSymbolAddress of the scratch array failed: %s", who, hipGetErrorString(e));
      return TQ_EHIP;
    }
    args.workspace = p;
    args.workspace_bytes = TQ_NOALLOC_SCRATCH_BYTES;
  } else if (!a->workspace || a->workspace_bytes < plan.bytes || ((uintptr_t)a->workspace & 255)) {
    set_error("decode: workspace must be 256-byte aligned and hold %zu bytes (got %zu)", plan.bytes,
              a->workspace_bytes);
    return TQ_EINVAL;
  }
  if (check_decode_launch(&args, plan) != hipSuccess) return TQ_EINVAL;  // message set by the check
  hipError_t e = launch_decode(&args, plan, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", who, hipGetErrorString(e));
    return TQ_EHIP;
  }
  return TQ_OK;
}

extern "C" int tq_decode_attention(const tq_decode_args* a, void* stream) { return decode_entry(a, stream, false); }

extern "C" int tq_decode_attention_noalloc(const tq_decode_args* a, void* stream) {
  return decode_entry(a, stream, true);
}

// ---------------------------------------------------------------------------
// Extend
// ---------------------------------------------------------------------------
extern "C" int tq_extend_attention(const tq_extend_args* a, void* stream) {
  if (!a || !a->ctx) {
    set_error("tq_extend_attention: NULL arguments or context");
    return TQ_EINVAL;
  }
  if (a->batch < 0 || a->num_q_heads <= 0 || a->num_kv_heads <= 0 || a->num_q_heads % a->num_kv_heads ||
      a->max_chunk < 0 || a->max_prefix_len < 0 || a->max_blocks_per_seq < 0 ||
      (int64_t)a->max_prefix_len > 16ll * a->max_blocks_per_seq || a->pool_blocks < 0) {
    set_error("tq_extend_attention: batch %d, heads %d / %d, max_chunk %d, max_prefix_len %d, max_blocks %d invalid",
              a->batch, a->num_q_heads, a->num_kv_heads, a->max_chunk, a->max_prefix_len, a->max_blocks_per_seq);
    return TQ_EINVAL;
  }
  const int G = a->num_q_heads / a->num_kv_heads;
  if (a->ctx->d != 128 || (G != 1 && G != 2 && G != 4 && G != 8) || a->ctx->kb > 4) {
    set_error("tq_extend_attention: head_dim %d, %d query heads per KV head, %d-bit keys is not supported "
              "(head_dim 128, G in {1, 2, 4, 8}, 2-4-bit keys)", a->ctx->d, G, a->ctx->kb);
    return TQ_EUNSUPPORTED;
  }
  if (a->batch == 0 || a->max_chunk == 0) return TQ_OK;
  if (!a->q || !a->k || !a->v || !a->cu_chunk || !a->prefix_lens || !a->out ||
      (a->max_prefix_len > 0 && (!a->pool || !a->block_tables))) {
    set_error("tq_extend_attention: NULL device pointer");
    return TQ_EINVAL;
  }
  if (((uintptr_t)a->q | (uintptr_t)a->k | (uintptr_t)a->v | (uintptr_t)a->pool) & 15) {
    set_error("tq_extend_attention: q, k, v and pool must be 16-byte aligned");
    return TQ_EINVAL;
  }
  hipError_t e = launch_extend(a, (hipStream_t)stream);
  if (e != hipSuccess) {
    set_error("tq_extend_attention: launch failed: %s", hipGetErrorString(e));
    return TQ_EHIP;
  }
  return TQ_OK;
}
