// Write path for gfx950: SRFT rotation + per-channel lambda + group-of-16 absmax quantization
// + packing ("When Quantization Is Free", technical summary, Methodology 2 and 3), its inverse
// (dequantize) and per-channel lambda calibration.
//
// One lane owns one head vector end to end: it loads the fp16 vector, flips signs, runs the
// d/2-point complex FFT and the Hermitian unpack in registers, scales by norm/lambda, takes the
// absmax of each group of 16 channels, rounds to codes and writes packed bytes and fp16 scales.
// A work-group covers up to 256 consecutive tokens of one (sequence, kv head) row, so the sign
// masks and the per-channel factors are staged once in LDS and read as broadcasts.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq_impl {
namespace {

using namespace kvqd;

constexpr int kQuantThreads = 256;

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

// Quantize one group of 16 channels already scaled to u (float32).
// Returns the fp16 scale bits and writes the packed group (8 bytes int4, 16 bytes int8).
template <int BITS>
__device__ __forceinline__ uint32_t quantize_group(const float (&u)[16], uint32_t (&packed)[BITS == 4 ? 2 : 4]) {
  using CM = CodeMagic<BITS>;
  float a = 0.0f;
  static_for<0, 16>([&](auto C) { a = fmaxf(a, fabsf(u[decltype(C)::value])); });
  // scale = fp16(a / qmax), saturated at 65504; division correctly rounded in float32
  const float ratio = fminf(a / CM::qmax, 65504.0f);
  const _Float16 sh = static_cast<_Float16>(ratio);
  const float sf = static_cast<float>(sh);
  const float inv = sf > 0.0f ? 1.0f / sf : 0.0f;
  uint32_t t[16];
  static_for<0, 16>([&](auto C) {
    constexpr int c = decltype(C)::value;
    float v = fmaf(u[c], inv, CM::magic);
    v = fminf(fmaxf(v, CM::magic - CM::qmax), CM::magic + CM::qmax);
    t[c] = __float_as_uint(v);
  });
  if constexpr (BITS == 4) {
    static_for<0, 2>([&](auto W) {
      constexpr int w = decltype(W)::value;
      uint32_t acc = 0;
      static_for<0, 4>([&](auto B) {
        constexpr int b = decltype(B)::value;
        const uint32_t byte = ((t[8 * w + 2 * b + 1] << 4) | t[8 * w + 2 * b]) & 0xffu;
        acc |= byte << (8 * b);
      });
      packed[w] = acc ^ CM::to_twos;
    });
  } else {
    static_for<0, 4>([&](auto W) {
      constexpr int w = decltype(W)::value;
      packed[w] = ((t[4 * w] & 0xffu) | ((t[4 * w + 1] & 0xffu) << 8) | ((t[4 * w + 2] & 0xffu) << 16) |
                   (t[4 * w + 3] << 24)) ^
                  CM::to_twos;
    });
  }
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, sh));
}

// Stage the sign flips of row b as fp16 sign-bit masks (one dword = two channels).
template <int D>
__device__ __forceinline__ void stage_sign_masks(uint32_t* smask, const float* __restrict__ sign) {
  for (int i = threadIdx.x; i < D / 2; i += blockDim.x) {
    smask[i] = (sign[2 * i] < 0.0f ? 0x8000u : 0u) | (sign[2 * i + 1] < 0.0f ? 0x80000000u : 0u);
  }
}

// Load one fp16 vector, flip signs, widen to float.
template <int D>
__device__ __forceinline__ void load_signed_vector(const uint16_t* __restrict__ src, const uint32_t* smask,
                                                   float (&y)[D]) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  static_for<0, D / 8>([&](auto J) {
    constexpr int j = decltype(J)::value;
    const uint4 w = s4[j];
    const uint4 m = reinterpret_cast<const uint4*>(smask)[j];
    const uint32_t w0 = w.x ^ m.x, w1 = w.y ^ m.y, w2 = w.z ^ m.z, w3 = w.w ^ m.w;
    y[8 * j + 0] = half_lo(w0);
    y[8 * j + 1] = half_hi(w0);
    y[8 * j + 2] = half_lo(w1);
    y[8 * j + 3] = half_hi(w1);
    y[8 * j + 4] = half_lo(w2);
    y[8 * j + 5] = half_hi(w2);
    y[8 * j + 6] = half_lo(w3);
    y[8 * j + 7] = half_hi(w3);
  });
}

template <int D, int BITS, bool HAS_LAMBDA>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(
    const uint16_t* __restrict__ x, int n_tok, int kv_heads, int tiles_per_row, int pos, int capacity,
    const float* __restrict__ sign, int64_t sign_bs, const float* __restrict__ lambda, int64_t lambda_bs,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  __shared__ __align__(16) uint32_t smask[D / 2];
  __shared__ __align__(16) float gtab[D];
  const int row = blockIdx.x / tiles_per_row;
  const int tile = blockIdx.x - row * tiles_per_row;
  const int b = row / kv_heads;
  const int h = row - b * kv_heads;
  stage_sign_masks<D>(smask, sign + b * sign_bs);
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float g = fwd_norm<D>(c);
    if constexpr (HAS_LAMBDA) g = g / lambda[b * lambda_bs + int64_t(h) * D + c];
    gtab[c] = g;
  }
  __syncthreads();
  const int t = tile * kQuantThreads + threadIdx.x;
  if (t >= n_tok) return;

  float y[D];
  load_signed_vector<D>(x + (int64_t(row) * n_tok + t) * D, smask, y);
  float r[D];
  real_fwd_raw<D>(y, r);

  constexpr int CB = D * BITS / 8;  // code bytes per vector
  const int64_t slot = int64_t(row) * capacity + pos + t;
  uint8_t* dst = codes + slot * CB;
  uint32_t sbits[D / 16];
  static_for<0, D / 16>([&](auto G) {
    constexpr int g = decltype(G)::value;
    float u[16];
    const float4* gt4 = reinterpret_cast<const float4*>(gtab + 16 * g);
    static_for<0, 4>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      const float4 f = gt4[q];
      u[4 * q + 0] = r[16 * g + 4 * q + 0] * f.x;
      u[4 * q + 1] = r[16 * g + 4 * q + 1] * f.y;
      u[4 * q + 2] = r[16 * g + 4 * q + 2] * f.z;
      u[4 * q + 3] = r[16 * g + 4 * q + 3] * f.w;
    });
    if constexpr (BITS == 4) {
      uint32_t p[2];
      sbits[g] = quantize_group<4>(u, p);
      *reinterpret_cast<uint2*>(dst + 8 * g) = make_uint2(p[0], p[1]);
    } else {
      uint32_t p[4];
      sbits[g] = quantize_group<8>(u, p);
      *reinterpret_cast<uint4*>(dst + 16 * g) = make_uint4(p[0], p[1], p[2], p[3]);
    }
  });
  uint4* sdst = reinterpret_cast<uint4*>(scales + slot * (D / 16));
  static_for<0, D / 128>([&](auto Q) {
    constexpr int q = decltype(Q)::value;
    sdst[q] = make_uint4(sbits[8 * q + 0] | (sbits[8 * q + 1] << 16), sbits[8 * q + 2] | (sbits[8 * q + 3] << 16),
                         sbits[8 * q + 4] | (sbits[8 * q + 5] << 16), sbits[8 * q + 6] | (sbits[8 * q + 7] << 16));
  });
}

// Signed code of channel c from a packed plane row.
template <int BITS>
__device__ __forceinline__ float code_at(const uint8_t* __restrict__ row, int c) {
  if constexpr (BITS == 4) {
    const int byte = row[c >> 1];
    const int nib = (c & 1) ? (byte >> 4) : (byte & 0xf);
    return static_cast<float>((nib ^ 8) - 8);
  } else {
    return static_cast<float>(static_cast<int8_t>(row[c]));
  }
}

template <int D, int BITS, bool HAS_LAMBDA>
__global__ __launch_bounds__(kQuantThreads) void dequantize_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int n_tok, int kv_heads,
    int tiles_per_row, int pos, int capacity, const float* __restrict__ sign, int64_t sign_bs,
    const float* __restrict__ lambda, int64_t lambda_bs, float* __restrict__ out) {
  __shared__ float lam[D];
  __shared__ float sgn[D];
  const int row = blockIdx.x / tiles_per_row;
  const int tile = blockIdx.x - row * tiles_per_row;
  const int b = row / kv_heads;
  const int h = row - b * kv_heads;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    lam[c] = HAS_LAMBDA ? lambda[b * lambda_bs + int64_t(h) * D + c] : 1.0f;
    sgn[c] = (sign[b * sign_bs + c] < 0.0f ? -1.0f : 1.0f) * inv_norm<D>();
  }
  __syncthreads();
  const int t = tile * kQuantThreads + threadIdx.x;
  if (t >= n_tok) return;
  const int64_t slot = int64_t(row) * capacity + pos + t;
  const uint8_t* crow = codes + slot * (D * BITS / 8);
  const uint16_t* srow = scales + slot * (D / 16);
  float a[D];
  static_for<0, D / 16>([&](auto G) {
    constexpr int g = decltype(G)::value;
    const float sc = static_cast<float>(__builtin_bit_cast(_Float16, srow[g]));
    static_for<0, 16>([&](auto C) {
      constexpr int c = 16 * g + decltype(C)::value;
      a[c] = code_at<BITS>(crow, c) * sc * lam[c];
    });
  });
  float y[D];
  real_inv_raw<D>(a, y);
  float4* o4 = reinterpret_cast<float4*>(out + (int64_t(row) * n_tok + t) * D);
  static_for<0, D / 4>([&](auto Q) {
    constexpr int q = decltype(Q)::value;
    o4[q] = make_float4(y[4 * q] * sgn[4 * q], y[4 * q + 1] * sgn[4 * q + 1], y[4 * q + 2] * sgn[4 * q + 2],
                        y[4 * q + 3] * sgn[4 * q + 3]);
  });
}

// lambda[b, h, c] = max over the first n_cal tokens of |SRFT(x)_c|; one work-group per row.
template <int D>
__global__ __launch_bounds__(kQuantThreads) void calibrate_kernel(const uint16_t* __restrict__ x, int n_tok,
                                                                  int n_cal, const float* __restrict__ sign,
                                                                  int64_t sign_bs, int kv_heads,
                                                                  float* __restrict__ lambda) {
  __shared__ __align__(16) uint32_t smask[D / 2];
  __shared__ uint32_t amax[D];
  const int row = blockIdx.x;
  const int b = row / kv_heads;
  stage_sign_masks<D>(smask, sign + b * sign_bs);
  for (int c = threadIdx.x; c < D; c += blockDim.x) amax[c] = 0u;
  __syncthreads();
  for (int t0 = 0; t0 < n_cal; t0 += kQuantThreads) {
    const int t = t0 + threadIdx.x;
    const bool valid = t < n_cal;
    float y[D];
    load_signed_vector<D>(x + (int64_t(row) * n_tok + (valid ? t : 0)) * D, smask, y);
    float r[D];
    real_fwd_raw<D>(y, r);
    static_for<0, D>([&](auto C) {
      constexpr int c = decltype(C)::value;
      // non-negative floats order like their bit patterns
      uint32_t v = valid ? __float_as_uint(fabsf(r[c] * fwd_norm<D>(c))) : 0u;
      for (int off = 32; off > 0; off >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off)));
      if ((threadIdx.x & 63) == 0) atomicMax(&amax[c], v);
    });
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    const float m = __uint_as_float(amax[c]);
    lambda[int64_t(row) * D + c] = m > 0.0f ? m : 1.0f;
  }
}

template <int D, int BITS>
hipError_t quantize_dispatch_lambda(const QuantArgs& a, hipStream_t s) {
  const int rows = a.batch * a.kv_heads;
  const int tiles = (a.n_tok + kQuantThreads - 1) / kQuantThreads;
  const dim3 grid(rows * tiles), block(kQuantThreads);
  auto* x = static_cast<const uint16_t*>(a.x);
  auto* codes = static_cast<uint8_t*>(a.codes);
  auto* scales = static_cast<uint16_t*>(a.scales);
  if (a.lambda)
    hipLaunchKernelGGL((quantize_kernel<D, BITS, true>), grid, block, 0, s, x, a.n_tok, a.kv_heads, tiles, a.pos,
                       a.capacity, a.sign, a.sign_bs, a.lambda, a.lambda_bs, codes, scales);
  else
    hipLaunchKernelGGL((quantize_kernel<D, BITS, false>), grid, block, 0, s, x, a.n_tok, a.kv_heads, tiles, a.pos,
                       a.capacity, a.sign, a.sign_bs, a.lambda, a.lambda_bs, codes, scales);
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t dequantize_dispatch_lambda(const DequantArgs& a, hipStream_t s) {
  const int rows = a.batch * a.kv_heads;
  const int tiles = (a.n_tok + kQuantThreads - 1) / kQuantThreads;
  const dim3 grid(rows * tiles), block(kQuantThreads);
  auto* codes = static_cast<const uint8_t*>(a.codes);
  auto* scales = static_cast<const uint16_t*>(a.scales);
  if (a.lambda)
    hipLaunchKernelGGL((dequantize_kernel<D, BITS, true>), grid, block, 0, s, codes, scales, a.n_tok, a.kv_heads,
                       tiles, a.pos, a.capacity, a.sign, a.sign_bs, a.lambda, a.lambda_bs, a.out);
  else
    hipLaunchKernelGGL((dequantize_kernel<D, BITS, false>), grid, block, 0, s, codes, scales, a.n_tok, a.kv_heads,
                       tiles, a.pos, a.capacity, a.sign, a.sign_bs, a.lambda, a.lambda_bs, a.out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.head_dim == 128) return a.bits == 4 ? quantize_dispatch_lambda<128, 4>(a, s) : quantize_dispatch_lambda<128, 8>(a, s);
  return a.bits == 4 ? quantize_dispatch_lambda<256, 4>(a, s) : quantize_dispatch_lambda<256, 8>(a, s);
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t s) {
  if (a.head_dim == 128)
    return a.bits == 4 ? dequantize_dispatch_lambda<128, 4>(a, s) : dequantize_dispatch_lambda<128, 8>(a, s);
  return a.bits == 4 ? dequantize_dispatch_lambda<256, 4>(a, s) : dequantize_dispatch_lambda<256, 8>(a, s);
}

hipError_t launch_calibrate(const CalibArgs& a, hipStream_t s) {
  const dim3 grid(a.batch * a.kv_heads), block(kQuantThreads);
  auto* x = static_cast<const uint16_t*>(a.x);
  if (a.head_dim == 128)
    hipLaunchKernelGGL((calibrate_kernel<128>), grid, block, 0, s, x, a.n_tok, a.n_cal, a.sign, a.sign_bs,
                       a.kv_heads, a.lambda);
  else
    hipLaunchKernelGGL((calibrate_kernel<256>), grid, block, 0, s, x, a.n_tok, a.n_cal, a.sign, a.sign_bs,
                       a.kv_heads, a.lambda);
  return hipGetLastError();
}

}  // namespace kvq_impl
