// Host-side construction of the random-feature matrix Omega [H, m, d] (fp64 -> fp32).
//
// Performer paper, section 2.4 and appendix B.2: orthogonal random features are
// built per d x d block with Gram-Schmidt; blocks are stacked for m > d.
// Appendix F.4: each orthogonal row keeps the N(0, I_d) marginal, i.e. a
// uniform direction with an independent chi(d) length.
//
// The bit-level recipe is fixed so that results are reproducible across
// processes and machines with the same C library:
//   stream key  K(seed,h,b,s) = mix(seed ^ mix(h*2^40 + b*2^8 + s))
//   draw i      x_i = mix(K + (i+1)*0x9E3779B97F4A7C15)      (SplitMix64, counter form)
//   uniform     u_i = ((x_i >> 12) + 0.5) * 2^-52            in (0, 1)
//   Gaussians   Box-Muller on (u_2p, u_2p+1): r = sqrt(-2 log u), angle 2*pi*u'
//   block       G (stream 0) d x d row-major; modified Gram-Schmidt over rows,
//               left-to-right fp64 sums, exact division by the norm;
//               lengths = row norms of a second Gaussian d x d matrix (stream 1)
//   rounding    fp64 -> fp32 round-to-nearest-even.
// This file must be compiled without floating-point contraction and without
// fast-math so that every operation rounds exactly once in binary64.
#include <cmath>
#include <cstdint>
#include <vector>

namespace favor_host {

static inline uint64_t splitmix_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t key_of(uint64_t seed, uint64_t head, uint64_t block, uint64_t stream) {
  const uint64_t tag = (head << 40) + (block << 8) + stream;
  return splitmix_mix(seed ^ splitmix_mix(tag));
}

static inline double unit_open(uint64_t key, uint64_t i) {
  const uint64_t x = splitmix_mix(key + (i + 1) * 0x9E3779B97F4A7C15ull);
  return (static_cast<double>(x >> 12) + 0.5) * 0x1p-52;
}

// n standard normals of one stream, pairs (r cos t, r sin t).
static void normals(uint64_t key, int n, std::vector<double>& out) {
  out.resize(static_cast<size_t>(n) + 1);
  const double two_pi = 6.283185307179586;
  for (int p = 0; 2 * p < n; ++p) {
    const double u1 = unit_open(key, 2ull * p);
    const double u2 = unit_open(key, 2ull * p + 1);
    const double r = std::sqrt(-2.0 * std::log(u1));
    const double t = two_pi * u2;
    out[2 * p] = r * std::cos(t);
    out[2 * p + 1] = r * std::sin(t);
  }
  out.resize(n);
}

// One d x d block of rows (fp64), row-major into `rows`.
static void block_rows(uint64_t seed, int head, int block, int d, int mode, std::vector<double>& rows) {
  std::vector<double> g;
  normals(key_of(seed, head, block, 0), d * d, g);
  rows.assign(static_cast<size_t>(d) * d, 0.0);
  if (mode == 1) {  // iid Gaussian rows
    rows = g;
    return;
  }
  // modified Gram-Schmidt: project each new row against the finished ones, in order
  std::vector<double> v(d);
  for (int i = 0; i < d; ++i) {
    for (int t = 0; t < d; ++t) v[t] = g[i * d + t];
    for (int j = 0; j < i; ++j) {
      const double* qj = &rows[static_cast<size_t>(j) * d];
      double c = 0.0;
      for (int t = 0; t < d; ++t) c += v[t] * qj[t];
      for (int t = 0; t < d; ++t) v[t] = v[t] - c * qj[t];
    }
    double s = 0.0;
    for (int t = 0; t < d; ++t) s += v[t] * v[t];
    const double nrm = std::sqrt(s);
    for (int t = 0; t < d; ++t) rows[static_cast<size_t>(i) * d + t] = v[t] / nrm;
  }
  if (mode == 2) {  // every row on the sphere of radius sqrt(d)
    const double len = std::sqrt(static_cast<double>(d));
    for (auto& x : rows) x = len * x;
    return;
  }
  std::vector<double> nv;
  normals(key_of(seed, head, block, 1), d * d, nv);
  for (int i = 0; i < d; ++i) {
    double s = 0.0;
    for (int t = 0; t < d; ++t) s += nv[i * d + t] * nv[i * d + t];
    const double len = std::sqrt(s);
    for (int t = 0; t < d; ++t) rows[static_cast<size_t>(i) * d + t] = len * rows[static_cast<size_t>(i) * d + t];
  }
}

void make_omega(uint64_t seed, int H, int m, int d, int mode, float* out) {
  if (mode == 3 || mode == 4) {
    // hyperbolic positive features (3): the m/2 rows of the orthogonal chi(d) mode, then their
    // negatives; trigonometric pairs (4): the same rows twice, for the sine and the cosine
    // features of each vector (m is even)
    const float sign = mode == 3 ? -1.f : 1.f;
    const int half = m / 2;
    std::vector<float> base(static_cast<size_t>(H) * half * d);
    make_omega(seed, H, half, d, 0, base.data());
    for (int h = 0; h < H; ++h)
      for (int r = 0; r < half; ++r)
        for (int t = 0; t < d; ++t) {
          const float x = base[(static_cast<size_t>(h) * half + r) * d + t];
          out[(static_cast<size_t>(h) * m + r) * d + t] = x;
          out[(static_cast<size_t>(h) * m + half + r) * d + t] = sign * x;
        }
    return;
  }
  const int nblocks = (m + d - 1) / d;
  std::vector<double> rows;
  for (int h = 0; h < H; ++h) {
    int r = 0;
    for (int b = 0; b < nblocks && r < m; ++b) {
      block_rows(seed, h, b, d, mode, rows);
      for (int i = 0; i < d && r < m; ++i, ++r) {
        float* dst = out + (static_cast<size_t>(h) * m + r) * d;
        for (int t = 0; t < d; ++t) dst[t] = static_cast<float>(rows[static_cast<size_t>(i) * d + t]);
      }
    }
  }
}

}  // namespace favor_host
