// Kernels of the write path that run the rotation as an in-register FFT on the vector ALUs, one
// lane per head vector: the inverse of the write path (dequantize, for inspection and tests),
// per-channel lambda calibration ("When Quantization Is Free", technical summary, Methodology 2:
// lambda is learned or calibrated), and the forward write path itself in that form
// (kvq_quantize_fft: the shape of the pages' fused write kernel, FFT stages plus the Hermitian
// unpack in registers, kept beside kvq_quantize's MFMA form, which it is measured against).
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

// The write path of one vector per lane: u = SRFT(x) / lambda from the in-register FFT, then the
// same decision as kvq_quantize (group absmax, fp16 scale, rounded codes; pt: one scale per
// vector) and the same plane layout.  One work-group per (row, tile of 256 tokens).
template <int D, int BITS, bool HAD>
__global__ __launch_bounds__(kQuantThreads) void quantize_fft_kernel(
    const uint16_t* __restrict__ x, int n_tok, int kv_heads, int tiles_per_row, int pos, int capacity,
    const float* __restrict__ sign, int64_t sign_bs, const float* __restrict__ lambda, int64_t lambda_bs,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales, int pt) {
  constexpr int NG = D / 16, CB = D * BITS / 8;
  __shared__ __align__(16) uint32_t smask[D / 2];
  __shared__ float rl[D];  // normalization of slot c over lambda_c
  const int row = blockIdx.x / tiles_per_row;
  const int tile = blockIdx.x - row * tiles_per_row;
  const int b = row / kv_heads;
  const int h = row - b * kv_heads;
  stage_sign_masks<D>(smask, sign + b * sign_bs);
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    const float nrm = HAD ? inv_sqrt_d<D>() : fwd_norm<D>(c);
    rl[c] = lambda ? nrm / lambda[b * lambda_bs + int64_t(h) * D + c] : nrm;
  }
  __syncthreads();
  const int t = tile * kQuantThreads + threadIdx.x;
  if (t >= n_tok) return;
  float y[D];
  load_signed_vector<D>(x + (int64_t(row) * n_tok + t) * D, smask, y);
  float u[D];
  if constexpr (HAD) {
    static_for<0, D>([&](auto C) { u[decltype(C)::value] = y[decltype(C)::value]; });
    wht<D>(u);
  } else {
    real_fwd_raw<D>(y, u);
  }
  static_for<0, D>([&](auto C) { u[decltype(C)::value] *= rl[decltype(C)::value]; });
  // group absmax (non-negative floats order like their bits), or one maximum per vector
  float amax[NG];
  static_for<0, NG>([&](auto G) {
    constexpr int g = decltype(G)::value;
    uint32_t m = 0u;
    static_for<0, 16>([&](auto C) { m = max(m, __float_as_uint(fabsf(u[16 * g + decltype(C)::value]))); });
    amax[g] = __uint_as_float(m);
  });
  if (pt) {
    float m = 0.0f;
    static_for<0, NG>([&](auto G) { m = fmaxf(m, amax[decltype(G)::value]); });
    static_for<0, NG>([&](auto G) { amax[decltype(G)::value] = m; });
  }
  const int64_t slot = int64_t(row) * capacity + pos + t;
  uint32_t cw[CB / 4];
  uint32_t sw[NG / 2];
  static_for<0, NG>([&](auto G) {
    constexpr int g = decltype(G)::value;
    const _Float16 sh = static_cast<_Float16>(scale_of<BITS>(amax[g]));
    const float sf = static_cast<float>(sh);
    const float inv = sf > 0.0f ? __builtin_amdgcn_rcpf(sf) : 0.0f;
    uint32_t cb[16];
    static_for<0, 16>([&](auto C) { cb[decltype(C)::value] = code_byte<BITS>(u[16 * g + decltype(C)::value], inv); });
    if constexpr (BITS == 4) {
      // two's-complement nibbles, even channel low: 8 bytes per group, 2 dwords
      static_for<0, 2>([&](auto W) {
        constexpr int wd = decltype(W)::value;
        uint32_t v = 0u;
        static_for<0, 4>([&](auto J) {
          constexpr int j = decltype(J)::value;
          const uint32_t byte = ((cb[8 * wd + 2 * j] ^ 8u) & 0xfu) | (((cb[8 * wd + 2 * j + 1] ^ 8u) & 0xfu) << 4);
          v |= byte << (8 * j);
        });
        cw[2 * g + wd] = v;
      });
    } else {
      static_for<0, 4>([&](auto W) {
        constexpr int wd = decltype(W)::value;
        cw[4 * g + wd] = ((cb[4 * wd] ^ 0x80u) | ((cb[4 * wd + 1] ^ 0x80u) << 8) | ((cb[4 * wd + 2] ^ 0x80u) << 16) |
                          ((cb[4 * wd + 3] ^ 0x80u) << 24));
      });
    }
    const uint32_t hb = __builtin_bit_cast(uint16_t, sh);
    if constexpr (g % 2 == 0)
      sw[g / 2] = hb;
    else
      sw[g / 2] |= hb << 16;
  });
  uint4* co = reinterpret_cast<uint4*>(codes + slot * CB);
  static_for<0, CB / 16>([&](auto Q) {
    constexpr int q = decltype(Q)::value;
    co[q] = make_uint4(cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]);
  });
  if (pt) {
    scales[slot] = uint16_t(sw[0] & 0xffffu);
  } else {
    uint4* so = reinterpret_cast<uint4*>(scales + slot * NG);
    static_for<0, NG / 8>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      so[q] = make_uint4(sw[4 * q], sw[4 * q + 1], sw[4 * q + 2], sw[4 * q + 3]);
    });
  }
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

template <int D, int BITS, bool HAD>
hipError_t quantize_fft_dispatch(const QuantArgs& a, hipStream_t s) {
  const int rows = a.batch * a.kv_heads;
  const int tiles = (a.n_tok + kQuantThreads - 1) / kQuantThreads;
  hipLaunchKernelGGL((quantize_fft_kernel<D, BITS, HAD>), dim3(rows * tiles), dim3(kQuantThreads), 0, s,
                     static_cast<const uint16_t*>(a.x), a.n_tok, a.kv_heads, tiles, a.pos, a.capacity, a.sign, a.sign_bs,
                     a.lambda, a.lambda_bs, static_cast<uint8_t*>(a.codes), static_cast<uint16_t*>(a.scales),
                     a.group == a.head_dim ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_fft(const QuantArgs& a, hipStream_t s) {
  const bool had = a.transform != 0;
  if (a.head_dim == 128) {
    if (a.bits == 4) return had ? quantize_fft_dispatch<128, 4, true>(a, s) : quantize_fft_dispatch<128, 4, false>(a, s);
    return had ? quantize_fft_dispatch<128, 8, true>(a, s) : quantize_fft_dispatch<128, 8, false>(a, s);
  }
  if (a.bits == 4) return had ? quantize_fft_dispatch<256, 4, true>(a, s) : quantize_fft_dispatch<256, 4, false>(a, s);
  return had ? quantize_fft_dispatch<256, 8, true>(a, s) : quantize_fft_dispatch<256, 8, false>(a, s);
}

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
