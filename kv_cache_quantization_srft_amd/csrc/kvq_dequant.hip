// Off-path kernels of the write path for gfx950: the inverse of the write path (dequantize,
// for inspection and tests) and per-channel lambda calibration ("When Quantization Is Free",
// technical summary, Methodology 2: lambda is learned or calibrated).
//
// One lane owns one head vector end to end: it loads the fp16 vector (or codes), runs the
// d/2-point complex FFT and the Hermitian (un)pack in registers, and scales by lambda.  A
// work-group covers up to 256 consecutive tokens of one (sequence, kv head) row, so the sign
// masks and per-channel factors are staged once in LDS and read as broadcasts.
#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq_impl {
namespace {

using namespace kvqd;

constexpr int kQuantThreads = 256;

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

// pt: one scale per vector (group = head_dim) instead of one per group of 16; lambda may be null
template <int D, int BITS, bool HAD>
__global__ __launch_bounds__(kQuantThreads) void dequantize_kernel(
    const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int n_tok, int kv_heads,
    int tiles_per_row, int pos, int capacity, const float* __restrict__ sign, int64_t sign_bs,
    const float* __restrict__ lambda, int64_t lambda_bs, float* __restrict__ out, int pt) {
  __shared__ float lam[D];
  __shared__ float sgn[D];
  const int row = blockIdx.x / tiles_per_row;
  const int tile = blockIdx.x - row * tiles_per_row;
  const int b = row / kv_heads;
  const int h = row - b * kv_heads;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    lam[c] = lambda ? lambda[b * lambda_bs + int64_t(h) * D + c] : 1.0f;
    sgn[c] = (sign[b * sign_bs + c] < 0.0f ? -1.0f : 1.0f) * (HAD ? inv_sqrt_d<D>() : inv_norm<D>());
  }
  __syncthreads();
  const int t = tile * kQuantThreads + threadIdx.x;
  if (t >= n_tok) return;
  const int64_t slot = int64_t(row) * capacity + pos + t;
  const uint8_t* crow = codes + slot * (D * BITS / 8);
  const uint16_t* srow = scales + slot * (pt ? 1 : D / 16);
  float a[D];
  static_for<0, D / 16>([&](auto G) {
    constexpr int g = decltype(G)::value;
    const float sc = static_cast<float>(__builtin_bit_cast(_Float16, srow[pt ? 0 : g]));
    static_for<0, 16>([&](auto C) {
      constexpr int c = 16 * g + decltype(C)::value;
      a[c] = code_at<BITS>(crow, c) * sc * lam[c];
    });
  });
  float y[D];
  if constexpr (HAD) {
    static_for<0, D>([&](auto C) { y[decltype(C)::value] = a[decltype(C)::value]; });
    wht<D>(y);
  } else {
    real_inv_raw<D>(a, y);
  }
  float4* o4 = reinterpret_cast<float4*>(out + (int64_t(row) * n_tok + t) * D);
  static_for<0, D / 4>([&](auto Q) {
    constexpr int q = decltype(Q)::value;
    o4[q] = make_float4(y[4 * q] * sgn[4 * q], y[4 * q + 1] * sgn[4 * q + 1], y[4 * q + 2] * sgn[4 * q + 2],
                        y[4 * q + 3] * sgn[4 * q + 3]);
  });
}

// lambda[b, h, c] = max over the first n_cal tokens of |SRFT(x)_c|; one work-group per row.
template <int D, bool HAD>
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
    if constexpr (HAD) {
      static_for<0, D>([&](auto C) { r[decltype(C)::value] = y[decltype(C)::value]; });
      wht<D>(r);
    } else {
      real_fwd_raw<D>(y, r);
    }
    static_for<0, D>([&](auto C) {
      constexpr int c = decltype(C)::value;
      // non-negative floats order like their bit patterns
      const float nrm = HAD ? inv_sqrt_d<D>() : fwd_norm<D>(c);
      uint32_t v = valid ? __float_as_uint(fabsf(r[c] * nrm)) : 0u;
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

template <int D, int BITS, bool HAD>
hipError_t dequantize_dispatch(const DequantArgs& a, hipStream_t s) {
  const int rows = a.batch * a.kv_heads;
  const int tiles = (a.n_tok + kQuantThreads - 1) / kQuantThreads;
  const dim3 grid(rows * tiles), block(kQuantThreads);
  hipLaunchKernelGGL((dequantize_kernel<D, BITS, HAD>), grid, block, 0, s, static_cast<const uint8_t*>(a.codes),
                     static_cast<const uint16_t*>(a.scales), a.n_tok, a.kv_heads, tiles, a.pos, a.capacity, a.sign,
                     a.sign_bs, a.lambda, a.lambda_bs, a.out, a.group == a.head_dim ? 1 : 0);
  return hipGetLastError();
}

template <int D, bool HAD>
hipError_t calibrate_dispatch(const CalibArgs& a, hipStream_t s) {
  const dim3 grid(a.batch * a.kv_heads), block(kQuantThreads);
  hipLaunchKernelGGL((calibrate_kernel<D, HAD>), grid, block, 0, s, static_cast<const uint16_t*>(a.x), a.n_tok,
                     a.n_cal, a.sign, a.sign_bs, a.kv_heads, a.lambda);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t s) {
  // group == head_dim: one scale per vector (the per-token comparison mode)
  const bool had = a.transform != 0;
  if (a.head_dim == 128) {
    if (a.bits == 4) return had ? dequantize_dispatch<128, 4, true>(a, s) : dequantize_dispatch<128, 4, false>(a, s);
    return had ? dequantize_dispatch<128, 8, true>(a, s) : dequantize_dispatch<128, 8, false>(a, s);
  }
  if (a.bits == 4) return had ? dequantize_dispatch<256, 4, true>(a, s) : dequantize_dispatch<256, 4, false>(a, s);
  return had ? dequantize_dispatch<256, 8, true>(a, s) : dequantize_dispatch<256, 8, false>(a, s);
}

hipError_t launch_calibrate(const CalibArgs& a, hipStream_t s) {
  const bool had = a.transform != 0;
  if (a.head_dim == 128) return had ? calibrate_dispatch<128, true>(a, s) : calibrate_dispatch<128, false>(a, s);
  return had ? calibrate_dispatch<256, true>(a, s) : calibrate_dispatch<256, false>(a, s);
}

}  // namespace kvq_impl
