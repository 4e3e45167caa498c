// Host-side weight packer of libsvdq (CPU only): smoothing vector, rank-r
// truncated SVD of the smoothed weight, residual, per-group int4 quantization
// and nibble packing.  Contract: include/svdq.h.
//
// Method (mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen durch
// Nunchaku 4-Bit-Quantisierung", section "Nunchaku und SVDQuant"; ai2day.live,
// "AI-Bildmodelle auf normalen GPUs ausführen", section "Was ist Nunchaku Lite
// und was macht es genau?"): activation outliers are moved into the weights
// (W' = W diag(lambda)), the dominant part of W' is kept as a 16-bit rank-r
// product, the remainder is quantized to 4 bits.  The rank (32 in the example
// config) and the group size come from the quantization config shown in the
// section "Native Ladefunktion in Diffusers".
//
// The SVD is randomized subspace iteration (Halko, Martinsson, Tropp, "Finding
// structure with randomness", SIAM Review 2011, algorithm 4.4) with
// oversampling, followed by one-sided Jacobi (Hestenes) on the small projected
// matrix.  No LAPACK.  Every output element is produced by one thread in a fixed
// order, so results do not depend on the thread count.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

#include "svdq.h"

svdq_status svdq_internal_fail(svdq_status s, const char* msg);
svdq_status svdq_internal_ok();

namespace {

double bf16_to_double(uint16_t h) {
  const uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

// bfloat16 nearest-even of a finite double, rounded once from the double value.
uint16_t double_to_bf16(double v) {
  uint64_t b;
  std::memcpy(&b, &v, 8);
  const uint16_t sign = static_cast<uint16_t>((b >> 63) << 15);
  const double a = std::fabs(v);
  if (a == 0.0) return sign;
  if (a < 0x1p-126) {  // bf16 subnormal range: quantum 2^-133 (128 -> smallest normal)
    return sign | static_cast<uint16_t>(std::nearbyint(a * 0x1p133));
  }
  const uint64_t ab = b & 0x7FFFFFFFFFFFFFFFull;
  int e = static_cast<int>(ab >> 52);
  const uint64_t m = (ab & ((1ull << 52) - 1)) | (1ull << 52);
  uint64_t q = m >> 45;
  const uint64_t rem = m & ((1ull << 45) - 1);
  const uint64_t half = 1ull << 44;
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (q == 256) {
    q = 128;
    ++e;
  }
  const int eb = e - 1023 + 127;
  if (eb >= 255) return sign | 0x7F80;
  return sign | static_cast<uint16_t>(eb << 7) | static_cast<uint16_t>(q & 0x7F);
}

int thread_count() {
  int t = static_cast<int>(std::thread::hardware_concurrency());
  if (const char* env = std::getenv("SVDQ_PACK_THREADS")) t = std::atoi(env);
  return std::max(1, std::min(t, 64));
}

template <class F>
void parallel_for(int64_t n, F f) {
  const int T = static_cast<int>(std::min<int64_t>(thread_count(), n));
  if (T <= 1) {
    f(int64_t{0}, n);
    return;
  }
  std::vector<std::thread> th;
  th.reserve(T);
  for (int t = 0; t < T; ++t) {
    const int64_t a = n * t / T, b = n * (t + 1) / T;
    th.emplace_back([=] { f(a, b); });
  }
  for (auto& x : th) x.join();
}

uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

// standard normal sample number `idx` of stream `seed` (Box-Muller on two hashed uniforms)
double gauss(uint64_t seed, uint64_t idx) {
  const uint64_t h1 = splitmix64(seed * 0x632BE59BD9B4E019ull + 2 * idx);
  const uint64_t h2 = splitmix64(seed * 0x632BE59BD9B4E019ull + 2 * idx + 1);
  const double u1 = (static_cast<double>(h1 >> 11) + 0.5) * 0x1p-53;
  const double u2 = static_cast<double>(h2 >> 11) * 0x1p-53;
  return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
}

// Y[n, :] = A[n, :] @ X  (A: N x K row-major, X: K x l row-major, Y: N x l)
void mul_a(const std::vector<double>& A, int64_t N, int64_t K, const std::vector<double>& X, int l,
           std::vector<double>& Y) {
  Y.assign(static_cast<size_t>(N) * l, 0.0);
  parallel_for(N, [&](int64_t n0, int64_t n1) {
    std::vector<double> acc(l);
    for (int64_t n = n0; n < n1; ++n) {
      std::fill(acc.begin(), acc.end(), 0.0);
      const double* a = &A[static_cast<size_t>(n) * K];
      for (int64_t k = 0; k < K; ++k) {
        const double av = a[k];
        const double* x = &X[static_cast<size_t>(k) * l];
        for (int c = 0; c < l; ++c) acc[c] += av * x[c];
      }
      std::copy(acc.begin(), acc.end(), &Y[static_cast<size_t>(n) * l]);
    }
  });
}

// Z[k, :] = sum_n A[n, k] * Q[n, :]   (Z = A^T Q, K x l)
void mul_at(const std::vector<double>& A, int64_t N, int64_t K, const std::vector<double>& Q, int l,
            std::vector<double>& Z) {
  Z.assign(static_cast<size_t>(K) * l, 0.0);
  constexpr int64_t kBlock = 64;
  const int64_t nblk = (K + kBlock - 1) / kBlock;
  parallel_for(nblk, [&](int64_t b0, int64_t b1) {
    for (int64_t b = b0; b < b1; ++b) {
      const int64_t k0 = b * kBlock, k1 = std::min(K, k0 + kBlock);
      for (int64_t n = 0; n < N; ++n) {
        const double* a = &A[static_cast<size_t>(n) * K];
        const double* q = &Q[static_cast<size_t>(n) * l];
        for (int64_t k = k0; k < k1; ++k) {
          const double av = a[k];
          double* z = &Z[static_cast<size_t>(k) * l];
          for (int c = 0; c < l; ++c) z[c] += av * q[c];
        }
      }
    }
  });
}

// Orthonormalise the columns of a rows x l row-major matrix (classical
// Gram-Schmidt applied twice).  Columns that vanish are set to zero.
void orthonormalize(std::vector<double>& Y, int64_t rows, int l) {
  std::vector<double> col(rows), proj(l);
  for (int c = 0; c < l; ++c) {
    for (int64_t n = 0; n < rows; ++n) col[n] = Y[static_cast<size_t>(n) * l + c];
    double norm0 = 0.0;
    for (int64_t n = 0; n < rows; ++n) norm0 += col[n] * col[n];
    norm0 = std::sqrt(norm0);
    for (int pass = 0; pass < 2; ++pass) {
      for (int j = 0; j < c; ++j) {
        double d = 0.0;
        for (int64_t n = 0; n < rows; ++n) d += Y[static_cast<size_t>(n) * l + j] * col[n];
        proj[j] = d;
      }
      for (int j = 0; j < c; ++j)
        for (int64_t n = 0; n < rows; ++n) col[n] -= proj[j] * Y[static_cast<size_t>(n) * l + j];
    }
    double norm = 0.0;
    for (int64_t n = 0; n < rows; ++n) norm += col[n] * col[n];
    norm = std::sqrt(norm);
    const double inv = (norm > 1e-13 * norm0 && norm > 0.0) ? 1.0 / norm : 0.0;
    for (int64_t n = 0; n < rows; ++n) Y[static_cast<size_t>(n) * l + c] = col[n] * inv;
  }
}

// One-sided Jacobi on the columns of Mt (l columns of length K, stored
// column-major as Mt[c * K + k]); accumulates the rotations in J (l x l,
// row-major, J[j * l + c]).
void one_sided_jacobi(std::vector<double>& Mt, int64_t K, int l, std::vector<double>& J) {
  J.assign(static_cast<size_t>(l) * l, 0.0);
  for (int c = 0; c < l; ++c) J[static_cast<size_t>(c) * l + c] = 1.0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    bool rotated = false;
    for (int p = 0; p < l - 1; ++p) {
      for (int q = p + 1; q < l; ++q) {
        double* x = &Mt[static_cast<size_t>(p) * K];
        double* y = &Mt[static_cast<size_t>(q) * K];
        double alpha = 0.0, beta = 0.0, gamma = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          alpha += x[k] * x[k];
          beta += y[k] * y[k];
          gamma += x[k] * y[k];
        }
        if (gamma == 0.0 || std::fabs(gamma) <= 1e-15 * std::sqrt(alpha * beta)) continue;
        rotated = true;
        const double zeta = (beta - alpha) / (2.0 * gamma);
        const double t = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        const double cs = 1.0 / std::sqrt(1.0 + t * t);
        const double sn = cs * t;
        for (int64_t k = 0; k < K; ++k) {
          const double xv = x[k], yv = y[k];
          x[k] = cs * xv - sn * yv;
          y[k] = sn * xv + cs * yv;
        }
        for (int j = 0; j < l; ++j) {
          double* jr = &J[static_cast<size_t>(j) * l];
          const double a = jr[p], b = jr[q];
          jr[p] = cs * a - sn * b;
          jr[q] = sn * a + cs * b;
        }
      }
    }
    if (!rotated) break;
  }
}

}  // namespace

extern "C" {

svdq_status svdq_smooth_from_absmax(const float* x_absmax, const uint16_t* w, int64_t N, int64_t K,
                                    float* smooth) {
  if (!x_absmax || !w || !smooth) return svdq_internal_fail(SVDQ_STATUS_INVALID_VALUE, "null pointer");
  if (N <= 0 || K <= 0) return svdq_internal_fail(SVDQ_STATUS_INVALID_VALUE, "N and K must be positive");
  const double eps = 1e-5;
  std::vector<double> wmax(static_cast<size_t>(K), 0.0);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k)
      wmax[k] = std::max(wmax[k], std::fabs(bf16_to_double(w[static_cast<size_t>(n) * K + k])));
  for (int64_t k = 0; k < K; ++k) {
    const double a = std::max(static_cast<double>(x_absmax[k]), eps);
    const double b = std::max(wmax[k], eps);
    smooth[k] = static_cast<float>(std::sqrt(a / b));
  }
  return svdq_internal_ok();
}

}  // extern "C"

namespace {

// E2M1 code of t (|t| < 8 after the block scaling): nearest value, a midpoint
// to the even code, above 6 saturating, zero without a sign
uint8_t fp4_code(double t) {
  const double m = std::fabs(t);
  const int c = (m > 0.25) + (m >= 0.75) + (m > 1.25) + (m >= 1.75) + (m > 2.5) + (m >= 3.5) + (m > 5.0);
  return static_cast<uint8_t>(c | ((t < 0 && c != 0) ? 8 : 0));
}

svdq_status pack_impl(const uint16_t* w, const float* smooth, int64_t N, int64_t K, int64_t r,
                      int64_t group_size, uint64_t seed, uint8_t* w_codes, uint16_t* w_scales,
                      uint16_t* lora_down, uint16_t* lora_up, bool fp4) {
  if (!w || !smooth || !w_codes || !w_scales) return svdq_internal_fail(SVDQ_STATUS_INVALID_VALUE, "null pointer");
  if (N <= 0 || K <= 0 || r < 0 || group_size <= 0)
    return svdq_internal_fail(SVDQ_STATUS_INVALID_VALUE, "bad dimensions");
  if (group_size != 64) return svdq_internal_fail(SVDQ_STATUS_NOT_SUPPORTED, "group_size must be 64");
  if (K % 64 != 0) return svdq_internal_fail(SVDQ_STATUS_NOT_SUPPORTED, "K must be a multiple of 64");
  if (r > 128 || r > std::min(N, K)) return svdq_internal_fail(SVDQ_STATUS_NOT_SUPPORTED, "rank too large");
  if (r > 0 && (!lora_down || !lora_up))
    return svdq_internal_fail(SVDQ_STATUS_INVALID_VALUE, "r > 0 needs lora_down and lora_up");

  // W' = W diag(lambda), exact in double (8 + 24 significant bits)
  std::vector<double> A(static_cast<size_t>(N) * K);
  parallel_for(N, [&](int64_t n0, int64_t n1) {
    for (int64_t n = n0; n < n1; ++n)
      for (int64_t k = 0; k < K; ++k)
        A[static_cast<size_t>(n) * K + k] =
            bf16_to_double(w[static_cast<size_t>(n) * K + k]) * static_cast<double>(smooth[k]);
  });

  std::vector<double> up_d(static_cast<size_t>(N) * r), down_d(static_cast<size_t>(r) * K);
  if (r > 0) {
    const int l = static_cast<int>(std::min<int64_t>(r + 16, std::min(N, K)));
    const int power_iters = 8;  // residual within ~1e-4 of Eckart-Young even on a flat spectrum
    std::vector<double> Omega(static_cast<size_t>(K) * l), Y, Z;
    parallel_for(K, [&](int64_t k0, int64_t k1) {
      for (int64_t k = k0; k < k1; ++k)
        for (int c = 0; c < l; ++c)
          Omega[static_cast<size_t>(k) * l + c] = gauss(seed, static_cast<uint64_t>(k) * l + c);
    });
    mul_a(A, N, K, Omega, l, Y);
    orthonormalize(Y, N, l);
    for (int it = 0; it < power_iters; ++it) {
      mul_at(A, N, K, Y, l, Z);
      orthonormalize(Z, K, l);
      mul_a(A, N, K, Z, l, Y);
      orthonormalize(Y, N, l);
    }
    // B^T = A^T Q (K x l); SVD of B^T by one-sided Jacobi: B^T J = V S
    mul_at(A, N, K, Y, l, Z);
    std::vector<double> Mt(static_cast<size_t>(l) * K);
    for (int64_t k = 0; k < K; ++k)
      for (int c = 0; c < l; ++c) Mt[static_cast<size_t>(c) * K + k] = Z[static_cast<size_t>(k) * l + c];
    std::vector<double> J;
    one_sided_jacobi(Mt, K, l, J);
    std::vector<double> sigma(l);
    for (int c = 0; c < l; ++c) {
      double s = 0.0;
      for (int64_t k = 0; k < K; ++k) s += Mt[static_cast<size_t>(c) * K + k] * Mt[static_cast<size_t>(c) * K + k];
      sigma[c] = std::sqrt(s);
    }
    std::vector<int> order(l);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return sigma[a] > sigma[b]; });
    // A ~= (Q J) S V^T: lora_up = (Q J)[:, c] sqrt(s_c); lora_down = sqrt(s_c) V[:, c]^T
    for (int i = 0; i < r; ++i) {
      const int c = order[i];
      const double s = sigma[c];
      const double root = std::sqrt(s);
      const double inv = s > 0 ? 1.0 / s : 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double v = Mt[static_cast<size_t>(c) * K + k] * inv;
        const uint16_t h = double_to_bf16(root * v);
        lora_down[static_cast<size_t>(i) * K + k] = h;
        down_d[static_cast<size_t>(i) * K + k] = bf16_to_double(h);
      }
    }
    parallel_for(N, [&](int64_t n0, int64_t n1) {
      for (int64_t n = n0; n < n1; ++n) {
        const double* q = &Y[static_cast<size_t>(n) * l];
        for (int i = 0; i < r; ++i) {
          const int c = order[i];
          double u = 0.0;
          for (int j = 0; j < l; ++j) u += q[j] * J[static_cast<size_t>(j) * l + c];
          const uint16_t h = double_to_bf16(u * std::sqrt(sigma[c]));
          lora_up[static_cast<size_t>(n) * r + i] = h;
          up_d[static_cast<size_t>(n) * r + i] = bf16_to_double(h);
        }
      }
    });
  }

  // residual against the rounded factors, then per-group symmetric int4 or
  // MXFP4 per 32-block
  const int64_t G = K / 64;
  parallel_for(N, [&](int64_t n0, int64_t n1) {
    std::vector<double> R(static_cast<size_t>(K));
    for (int64_t n = n0; n < n1; ++n) {
      const double* a = &A[static_cast<size_t>(n) * K];
      for (int64_t k = 0; k < K; ++k) {
        double lowrank = 0.0;
        for (int64_t i = 0; i < r; ++i)
          lowrank += up_d[static_cast<size_t>(n) * r + i] * down_d[static_cast<size_t>(i) * K + k];
        R[k] = a[k] - lowrank;
      }
      if (fp4) {
        // MXFP4 (OCP Microscaling v1.0): e = floor(log2 amax) - 2 in [-127, 127]
        // (-127 for a zero block), elements R / 2^e to E2M1
        uint8_t* sc = reinterpret_cast<uint8_t*>(w_scales) + static_cast<size_t>(n) * (K / 32);
        for (int64_t b = 0; b < K / 32; ++b) {
          const double* seg = &R[static_cast<size_t>(b) * 32];
          double amax = 0.0;
          for (int e = 0; e < 32; ++e) amax = std::max(amax, std::fabs(seg[e]));
          int e = -127;
          if (amax > 0) {
            int x = 0;
            (void)std::frexp(amax, &x);
            e = std::max(-127, std::min(127, x - 1 - 2));
          }
          sc[b] = static_cast<uint8_t>(e + 127);
          uint8_t* out = &w_codes[static_cast<size_t>(n) * (K / 2) + b * 16];
          for (int i = 0; i < 32; i += 2)
            out[i / 2] = static_cast<uint8_t>(fp4_code(std::ldexp(seg[i], -e)) |
                                              (fp4_code(std::ldexp(seg[i + 1], -e)) << 4));
        }
        continue;
      }
      for (int64_t g = 0; g < G; ++g) {
        const double* seg = &R[static_cast<size_t>(g) * 64];
        double amax = 0.0;
        for (int e = 0; e < 64; ++e) amax = std::max(amax, std::fabs(seg[e]));
        const uint16_t sb = double_to_bf16(amax / 7.0);
        w_scales[static_cast<size_t>(n) * G + g] = sb;
        const double s = bf16_to_double(sb);
        uint8_t* out = &w_codes[static_cast<size_t>(n) * (K / 2) + g * 32];
        // storage order: rows with bit 3 set hold the two 8-byte halves of every
        // 16-byte granule exchanged (byte j of the row at j ^ 8)
        const int flip = (n & 8) ? 8 : 0;
        for (int e = 0; e < 64; e += 2) {
          int q0 = 0, q1 = 0;
          if (s > 0) {
            q0 = static_cast<int>(std::nearbyint(seg[e] / s));
            q1 = static_cast<int>(std::nearbyint(seg[e + 1] / s));
            q0 = std::max(-7, std::min(7, q0));
            q1 = std::max(-7, std::min(7, q1));
          }
          out[(e / 2) ^ flip] = static_cast<uint8_t>((q0 & 0xF) | ((q1 & 0xF) << 4));
        }
      }
    }
  });
  return svdq_internal_ok();
}

}  // namespace

extern "C" {

svdq_status svdq_pack_weights(const uint16_t* w, const float* smooth, int64_t N, int64_t K, int64_t r,
                              int64_t group_size, uint64_t seed, uint8_t* w_codes, uint16_t* w_scales,
                              uint16_t* lora_down, uint16_t* lora_up) {
  return pack_impl(w, smooth, N, K, r, group_size, seed, w_codes, w_scales, lora_down, lora_up, false);
}

svdq_status svdq_pack_weights_fp4(const uint16_t* w, const float* smooth, int64_t N, int64_t K, int64_t r,
                                  uint64_t seed, uint8_t* w_codes, uint8_t* w_scales, uint16_t* lora_down,
                                  uint16_t* lora_up) {
  if (K > 0 && K % 128 != 0) return svdq_internal_fail(SVDQ_STATUS_NOT_SUPPORTED, "K must be a multiple of 128");
  return pack_impl(w, smooth, N, K, r, 64, seed, w_codes, reinterpret_cast<uint16_t*>(w_scales), lora_down,
                   lora_up, true);
}


// AWQ W4A16 packer (Lin et al., 2023, "AWQ: Activation-aware Weight
// Quantization"): s = clamp(mean|x|^alpha, 1e-4) / sqrt(max s * min s) for
// alpha = i / n_grid, i = 0..n_grid-1; the alpha whose quantized layer has the
// least mean squared output error on the calibration rows wins (the first on
// ties); W * s is then quantized per 64-wide group to unsigned 4-bit codes with
// Delta = bf16(max(max - min, 1e-5) / 15) and z = clamp(rint(-min / Delta), 0, 15).
// The scheme is the one the Nunchaku Lite integration uses for its modulation
// projections (mind-verse.de, "Effiziente Optimierung von Diffusionsmodellen
// durch Nunchaku 4-Bit-Quantisierung", section "Nunchaku Lite: Nahtlose
// Integration in Diffusers").
svdq_status svdq_awq_pack_weights(const uint16_t* w, const uint16_t* x_calib, int64_t Mc, int64_t N,
                                  int64_t K, int64_t group_size, int n_grid, float* smooth,
                                  uint8_t* w_codes, uint16_t* w_scales, uint8_t* w_zeros, float* alpha_out) {
  if (!w || !x_calib || !smooth || !w_codes || !w_scales || !w_zeros)
    return svdq_internal_fail(SVDQ_STATUS_INVALID_VALUE, "null pointer");
  if (Mc <= 0 || N <= 0 || K <= 0 || n_grid <= 0 || n_grid > 1000)
    return svdq_internal_fail(SVDQ_STATUS_INVALID_VALUE, "bad dimensions or grid");
  if (group_size != 64) return svdq_internal_fail(SVDQ_STATUS_NOT_SUPPORTED, "group_size must be 64");
  if (K % 64 != 0) return svdq_internal_fail(SVDQ_STATUS_NOT_SUPPORTED, "K must be a multiple of 64");
  const int64_t G = K / 64;
  std::vector<double> x(static_cast<size_t>(Mc * K)), wd(static_cast<size_t>(N * K));
  for (int64_t i = 0; i < Mc * K; ++i) x[i] = bf16_to_double(x_calib[i]);
  for (int64_t i = 0; i < N * K; ++i) wd[i] = bf16_to_double(w[i]);
  std::vector<double> sx(static_cast<size_t>(K), 0.0);
  for (int64_t m = 0; m < Mc; ++m)
    for (int64_t k = 0; k < K; ++k) sx[k] += std::fabs(x[m * K + k]);
  for (int64_t k = 0; k < K; ++k) sx[k] /= static_cast<double>(Mc);

  auto scales_for = [&](double alpha, std::vector<float>& s32) {
    std::vector<double> s(static_cast<size_t>(K));
    for (int64_t k = 0; k < K; ++k) s[k] = std::max(std::pow(sx[k], alpha), 1e-4);
    const double mx = *std::max_element(s.begin(), s.end());
    const double mn = *std::min_element(s.begin(), s.end());
    const double nrm = std::sqrt(mx * mn);
    for (int64_t k = 0; k < K; ++k) s32[k] = static_cast<float>(s[k] / nrm);
  };
  // quantizes row n of W * s; fills codes q (0..15), Delta bits, z
  auto quant_row = [&](int64_t n, const std::vector<float>& s32, uint8_t* q, uint16_t* dbits, uint8_t* z) {
    for (int64_t g = 0; g < G; ++g) {
      double mx = -INFINITY, mn = INFINITY;
      double v[64];
      for (int j = 0; j < 64; ++j) {
        const int64_t k = g * 64 + j;
        v[j] = wd[n * K + k] * static_cast<double>(s32[k]);
        mx = std::max(mx, v[j]);
        mn = std::min(mn, v[j]);
      }
      const uint16_t db = double_to_bf16(std::max(mx - mn, 1e-5) / 15.0);
      const double d = bf16_to_double(db);
      const double zz = std::min(std::max(std::nearbyint(-mn / d), 0.0), 15.0);
      for (int j = 0; j < 64; ++j)
        q[g * 64 + j] = static_cast<uint8_t>(std::min(std::max(std::nearbyint(v[j] / d) + zz, 0.0), 15.0));
      dbits[g] = db;
      z[g] = static_cast<uint8_t>(zz);
    }
  };
  // mean squared output error over the calibration rows; each thread sums its
  // rows of W in order, the per-row sums are added in row order
  auto loss_for = [&](const std::vector<float>& s32) {
    std::vector<double> row_err(static_cast<size_t>(N), 0.0);
    parallel_for(N, [&](int64_t a, int64_t b) {
      std::vector<uint8_t> q(static_cast<size_t>(K)), z(static_cast<size_t>(G));
      std::vector<uint16_t> db(static_cast<size_t>(G));
      std::vector<double> diff(static_cast<size_t>(K));
      for (int64_t n = a; n < b; ++n) {
        quant_row(n, s32, q.data(), db.data(), z.data());
        for (int64_t k = 0; k < K; ++k) {
          const int64_t g = k / 64;
          const double weff = ((double)q[k] - (double)z[g]) * bf16_to_double(db[g]) / (double)s32[k];
          diff[k] = wd[n * K + k] - weff;
        }
        double e = 0.0;
        for (int64_t m = 0; m < Mc; ++m) {
          const double* xr = &x[m * K];
          double acc[4] = {0.0, 0.0, 0.0, 0.0};
          int64_t k = 0;
          for (; k + 4 <= K; k += 4)
            for (int j = 0; j < 4; ++j) acc[j] += xr[k + j] * diff[k + j];
          double dot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
          for (; k < K; ++k) dot += xr[k] * diff[k];
          e += dot * dot;
        }
        row_err[n] = e;
      }
    });
    double tot = 0.0;
    for (int64_t n = 0; n < N; ++n) tot += row_err[n];
    return tot / static_cast<double>(Mc * N);
  };

  std::vector<float> s32(static_cast<size_t>(K)), best(static_cast<size_t>(K));
  double best_loss = INFINITY, best_alpha = 0.0;
  for (int i = 0; i < n_grid; ++i) {
    const double alpha = static_cast<double>(i) / n_grid;
    scales_for(alpha, s32);
    const double l = loss_for(s32);
    if (l < best_loss) {
      best_loss = l;
      best_alpha = alpha;
      best = s32;
    }
  }
  parallel_for(N, [&](int64_t a, int64_t b) {
    std::vector<uint8_t> q(static_cast<size_t>(K));
    for (int64_t n = a; n < b; ++n) {
      quant_row(n, best, q.data(), w_scales + n * G, w_zeros + n * G);
      for (int64_t i = 0; i < K / 2; ++i)
        w_codes[n * (K / 2) + i] = static_cast<uint8_t>(q[2 * i] | (q[2 * i + 1] << 4));
    }
  });
  std::memcpy(smooth, best.data(), sizeof(float) * static_cast<size_t>(K));
  if (alpha_out) *alpha_out = static_cast<float>(best_alpha);
  return svdq_internal_ok();
}

}  // extern "C"
