// Device building blocks for the gfx950 kernels: compile-time twiddles, an in-register FFT
// whose output permutation is resolved at compile time, and the forward / inverse real-layout
// transforms of one head vector held by one lane.
//
// The rotation is SRFT(x) = pack(F diag(s) x) with F the unitary DFT ("When Quantization Is
// Free", technical summary, Methodology 1).  The write kernel the explainer describes runs
// log2(d/2) radix-2 Stockham stages and then unpacks the Hermitian half-spectrum (Methodology
// 2).  Here the same d/2-point complex FFT is done with radix-4 stages (fewer VALU operations)
// fully unrolled in registers, so the Stockham/bit-reversal reordering costs nothing: every
// register index is a compile-time constant.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace kvqd {

// ------------------------------------------------------------------------------------------
// compile-time helpers
// ------------------------------------------------------------------------------------------
template <int B, int E, typename F>
__host__ __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(std::forward<F>(f));
  }
}

constexpr double csqrt(double v) {  // Newton iteration, v > 0
  double x = v > 1.0 ? v : 1.0;
  for (int i = 0; i < 64; ++i) x = 0.5 * (x + v / x);
  return x;
}

constexpr double kPi = 3.14159265358979323846264338327950288;

constexpr double taylor_sin(double x) {  // |x| <= pi/4
  double term = x, sum = x;
  for (int n = 1; n < 16; ++n) {
    term *= -x * x / double((2 * n) * (2 * n + 1));
    sum += term;
  }
  return sum;
}

constexpr double taylor_cos(double x) {  // |x| <= pi/4
  double term = 1.0, sum = 1.0;
  for (int n = 1; n < 16; ++n) {
    term *= -x * x / double((2 * n - 1) * (2 * n));
    sum += term;
  }
  return sum;
}

struct CosSin {
  double c, s;
};

// cos and sin of 2*pi*m/n for a power-of-two n >= 4, by exact octant reduction.
constexpr CosSin cos_sin_turn(long m, long n) {
  m = ((m % n) + n) % n;
  if (2 * m > n) {  // theta = 2pi - phi
    CosSin r = cos_sin_turn(n - m, n);
    return {r.c, -r.s};
  }
  if (4 * m > n) {  // theta = pi - phi
    CosSin r = cos_sin_turn(n / 2 - m, n);
    return {-r.c, r.s};
  }
  if (8 * m > n) {  // theta = pi/2 - phi
    CosSin r = cos_sin_turn(n / 4 - m, n);
    return {r.s, r.c};
  }
  const double x = 2.0 * kPi * double(m) / double(n);
  return {taylor_cos(x), taylor_sin(x)};
}

template <int N, int E>
struct Twiddle {
  static constexpr CosSin v = cos_sin_turn(E, N);
  static constexpr float c = float(v.c);
  static constexpr float s = float(v.s);
};

// (re, im) *= exp(-2 pi i E / N) (forward) or exp(+2 pi i E / N) (inverse).
template <int N, int E, bool INV>
__host__ __device__ __forceinline__ void twiddle(float& re, float& im) {
  constexpr int e = ((E % N) + N) % N;
  if constexpr (e == 0) {
    return;
  } else if constexpr (2 * e == N) {
    re = -re;
    im = -im;
  } else if constexpr (4 * e == N || 4 * e == 3 * N) {
    // forward, e = N/4: multiply by -i; inverse: by +i.  e = 3N/4 is the opposite.
    constexpr bool minus_i = (4 * e == N) != INV;
    const float t = re;
    if constexpr (minus_i) {
      re = im;
      im = -t;
    } else {
      re = -im;
      im = t;
    }
  } else {
    constexpr float c = Twiddle<N, e>::c;
    constexpr float s = Twiddle<N, e>::s;
    const float r0 = re, i0 = im;
    if constexpr (!INV) {  // (r + i m)(c - i s)
      re = r0 * c + i0 * s;
      im = i0 * c - r0 * s;
    } else {  // (r + i m)(c + i s)
      re = r0 * c - i0 * s;
      im = i0 * c + r0 * s;
    }
  }
}

// ------------------------------------------------------------------------------------------
// In-register decimation-in-frequency FFT of M complex values (M a power of two >= 4).
// Radix-4 stages while the block is >= 4 points, then one radix-2 stage if needed.
// Input in natural order; output bin k ends up in register dif_pos<M>(k).
// ------------------------------------------------------------------------------------------
constexpr int dif_radix(int nb) { return nb >= 4 ? 4 : 2; }

constexpr int dif_pos(int k, int nb) {
  return nb == 1 ? 0 : (k % dif_radix(nb)) * (nb / dif_radix(nb)) + dif_pos(k / dif_radix(nb), nb / dif_radix(nb));
}

template <int M, int NB, bool INV>
__host__ __device__ __forceinline__ void dif_stage(float (&re)[M], float (&im)[M]) {
  if constexpr (NB >= 2) {
    constexpr int R = dif_radix(NB);
    constexpr int H = NB / R;  // span
    static_for<0, M / NB>([&](auto BLK) {
      constexpr int b = decltype(BLK)::value * NB;
      static_for<0, H>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if constexpr (R == 4) {
          const float x0r = re[b + j], x0i = im[b + j];
          const float x1r = re[b + j + H], x1i = im[b + j + H];
          const float x2r = re[b + j + 2 * H], x2i = im[b + j + 2 * H];
          const float x3r = re[b + j + 3 * H], x3i = im[b + j + 3 * H];
          const float t0r = x0r + x2r, t0i = x0i + x2i;
          const float t1r = x0r - x2r, t1i = x0i - x2i;
          const float t2r = x1r + x3r, t2i = x1i + x3i;
          float t3r = x1r - x3r, t3i = x1i - x3i;
          {  // t3 *= -i (forward) or +i (inverse)
            const float t = t3r;
            if constexpr (!INV) {
              t3r = t3i;
              t3i = -t;
            } else {
              t3r = -t3i;
              t3i = t;
            }
          }
          re[b + j] = t0r + t2r;
          im[b + j] = t0i + t2i;
          float y1r = t1r + t3r, y1i = t1i + t3i;
          float y2r = t0r - t2r, y2i = t0i - t2i;
          float y3r = t1r - t3r, y3i = t1i - t3i;
          twiddle<NB, j, INV>(y1r, y1i);
          twiddle<NB, 2 * j, INV>(y2r, y2i);
          twiddle<NB, 3 * j, INV>(y3r, y3i);
          re[b + j + H] = y1r;
          im[b + j + H] = y1i;
          re[b + j + 2 * H] = y2r;
          im[b + j + 2 * H] = y2i;
          re[b + j + 3 * H] = y3r;
          im[b + j + 3 * H] = y3i;
        } else {
          const float x0r = re[b + j], x0i = im[b + j];
          const float x1r = re[b + j + H], x1i = im[b + j + H];
          re[b + j] = x0r + x1r;
          im[b + j] = x0i + x1i;
          float dr = x0r - x1r, di = x0i - x1i;
          twiddle<NB, j, INV>(dr, di);
          re[b + j + H] = dr;
          im[b + j + H] = di;
        }
      });
    });
    dif_stage<M, NB / R, INV>(re, im);
  }
}

template <int M, bool INV>
__host__ __device__ __forceinline__ void fft_dif(float (&re)[M], float (&im)[M]) {
  dif_stage<M, M, INV>(re, im);
}

// ------------------------------------------------------------------------------------------
// Forward real transform of one vector (one lane).
//   in : y[n], n < D, the sign-flipped input
//   out: r[c] with the unitary packed slot c equal to r[c] * fwd_norm<D>(c)
// Layout of slots: c=0 Re X0, c=1 Re X_{D/2}, c=2k sqrt2 Re Xk, c=2k+1 sqrt2 Im Xk.
// The D-point real DFT is computed as a D/2-point complex FFT of z[n] = y[2n] + i y[2n+1]
// followed by the Hermitian unpack X_k = E_k + W^k O_k with E, O the even/odd spectra.
// ------------------------------------------------------------------------------------------
template <int D>
__host__ __device__ constexpr float fwd_norm(int c) {
  // raw slots carry: Xfull for c < 2, 2*Xfull for pairs, Xfull for k = D/4 (c = D/2, D/2+1)
  return c < 2 ? float(1.0 / csqrt(double(D)))
               : (c == D / 2 || c == D / 2 + 1) ? float(csqrt(2.0 / double(D)))
                                                : float(1.0 / csqrt(2.0 * double(D)));
}

template <int D>
__host__ __device__ __forceinline__ void real_fwd_raw(const float (&y)[D], float (&r)[D]) {
  constexpr int M = D / 2;
  float zr[M], zi[M];
  static_for<0, M>([&](auto N) {
    constexpr int n = decltype(N)::value;
    zr[n] = y[2 * n];
    zi[n] = y[2 * n + 1];
  });
  fft_dif<M, false>(zr, zi);
  {
    constexpr int p0 = dif_pos(0, M);
    r[0] = zr[p0] + zi[p0];  // Xfull[0]
    r[1] = zr[p0] - zi[p0];  // Xfull[M]
  }
  static_for<1, M / 2>([&](auto K) {
    constexpr int k = decltype(K)::value;
    constexpr int pa = dif_pos(k, M), pb = dif_pos(M - k, M);
    const float ar = zr[pa], ai = zi[pa], br = zr[pb], bi = zi[pb];
    const float er = ar + br, ei = ai - bi;  // 2E = a + conj(b)
    float orr = ai + bi, oi = br - ar;       // 2O = -i (a - conj(b))
    twiddle<D, k, false>(orr, oi);           // 2 W^k O
    r[2 * k] = er + orr;                     // 2 X_k
    r[2 * k + 1] = ei + oi;
    r[2 * (M - k)] = er - orr;               // 2 X_{M-k} = conj(2E - 2W^k O)
    r[2 * (M - k) + 1] = oi - ei;
  });
  {
    constexpr int ph = dif_pos(M / 2, M);  // X_{M/2} = conj(Z[M/2])
    r[M] = zr[ph];
    r[M + 1] = -zi[ph];
  }
}

// ------------------------------------------------------------------------------------------
// Inverse real transform of one vector (one lane).
//   in : a[c] = unitary packed slots
//   out: y[n] * inv_norm<D>() is the inverse-transformed vector (before the sign flip)
// ------------------------------------------------------------------------------------------
template <int D>
__host__ __device__ constexpr float inv_norm() {
  return float(1.0 / csqrt(2.0 * double(D)));
}

template <int D>
__host__ __device__ __forceinline__ void real_inv_raw(const float (&a)[D], float (&y)[D]) {
  constexpr int M = D / 2;
  constexpr float kSqrt2 = 1.41421356237309504880f;
  float zr[M], zi[M];
  {
    const float a0 = kSqrt2 * a[0], am = kSqrt2 * a[1];  // A[0], A[M] (real)
    zr[0] = a0 + am;
    zi[0] = a0 - am;
  }
  static_for<1, M / 2>([&](auto K) {
    constexpr int k = decltype(K)::value;
    const float ar = a[2 * k], ai = a[2 * k + 1];
    const float br = a[2 * (M - k)], bi = a[2 * (M - k) + 1];
    const float er = ar + br, ei = ai - bi;  // E = A[k] + conj(A[M-k])
    float dr = ar - br, di = ai + bi;        // A[k] - conj(A[M-k])
    twiddle<D, k, true>(dr, di);             // conj(W^k) (.)
    const float pr = -di, pi = dr;           // P = i * conj(W^k) (.)
    zr[k] = er + pr;
    zi[k] = ei + pi;
    zr[M - k] = er - pr;                     // conj(E - P)
    zi[M - k] = pi - ei;
  });
  zr[M / 2] = 2.0f * a[M];  // 2 conj(A[M/2])
  zi[M / 2] = -2.0f * a[M + 1];
  fft_dif<M, true>(zr, zi);
  static_for<0, M>([&](auto N) {
    constexpr int n = decltype(N)::value;
    constexpr int p = dif_pos(n, M);
    y[2 * n] = zr[p];
    y[2 * n + 1] = zi[p];
  });
}

// ------------------------------------------------------------------------------------------
// small helpers
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float half_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(f)));
}

// In-place fast Walsh-Hadamard transform in Sylvester (natural) order, unnormalized:
// y <- H y with H[i][j] = (-1)^popcount(i & j), log2 N stages of add / subtract butterflies.
// The SRHT is d^-1/2 H diag(s) x; H is symmetric and H H = N I, so the same routine inverts it.
template <int N>
__host__ __device__ __forceinline__ void wht(float (&y)[N]) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1) {
#pragma unroll
    for (int i = 0; i < N; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
    }
  }
}

template <int D>
__host__ __device__ constexpr float inv_sqrt_d() {
  return float(1.0 / csqrt(double(D)));
}

// ---- the code decision of the write path (group absmax -> fp16 scale -> rounded codes) ----

// Rounding by the float32 "magic number": for |v| <= 2^22, fma(u, inv, M) with M = 2^23 + off
// rounds u*inv to the nearest integer (ties to even, as M + off is even) and leaves
// off + code in the low mantissa bits.  With off = 8 (int4) / 128 (int8) and codes clamped to
// [-qmax, qmax], byte 0 of the bit pattern is the offset-binary code and nothing above it
// within the byte is set.
template <int BITS>
struct CodeMagic {
  static constexpr float qmax = BITS == 4 ? 7.0f : 127.0f;
  static constexpr float magic = BITS == 4 ? 8388616.0f : 8388736.0f;  // 2^23 + 8 / 2^23 + 128
  static constexpr uint32_t to_twos = BITS == 4 ? 0x88888888u : 0x80808080u;
};

// fp32 a / qmax, correctly rounded (reciprocal product plus one exact residual correction),
// saturated at the fp16 maximum
template <int BITS>
__device__ __forceinline__ float scale_of(float a) {
  constexpr float q = BITS == 4 ? 7.0f : 127.0f;
  constexpr float rq = 1.0f / q;
  const float y = a * rq;
  const float r = fmaf(-y, q, a);
  return fminf(fmaf(r, rq, y), 65504.0f);
}

// Offset-binary code byte (code + 8 or code + 128) of u under the reciprocal scale inv.
template <int BITS>
__device__ __forceinline__ uint32_t code_byte(float u, float inv) {
  using CM = CodeMagic<BITS>;
  float vq = fmaf(u, inv, CM::magic);
  vq = fminf(fmaxf(vq, CM::magic - CM::qmax), CM::magic + CM::qmax);
  return __float_as_uint(vq) & 0xffu;
}

}  // namespace kvqd
