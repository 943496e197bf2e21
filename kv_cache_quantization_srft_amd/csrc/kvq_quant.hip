// Write path for gfx950: SRFT rotation + per-channel lambda + group-of-16 absmax quantization
// + packing ("When Quantization Is Free", technical summary, Methodology 2 and 3), its inverse
// (dequantize) and per-channel lambda calibration.
//
// Two implementations of the same write path:
//  * d = 128: the rotation of 16 vectors at a time is a 128x128 matrix product on MFMA
//    (quantize_mfma_kernel, below), which leaves the VALU free for the absmax, rounding and
//    packing;
//  * d = 256 (and calibration / dequantize): one lane owns one head vector end to end: it loads
//    the fp16 vector, flips signs, runs the d/2-point complex FFT and the Hermitian unpack in
//    registers, scales by norm/lambda, takes the absmax of each group of 16 channels, rounds to
//    codes and writes packed bytes and fp16 scales.  A work-group covers up to 256 consecutive
//    tokens of one (sequence, kv head) row, so the sign masks and per-channel factors are staged
//    once in LDS and read as broadcasts.
#include <algorithm>

#include "kvq_decode_common.h"
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

// ------------------------------------------------------------------------------------------
// d = 128 write path on MFMA.  u = Q (s * x) / lambda for 16 vectors at a time with
// v_mfma_f32_16x16x32_f16: A = the forward table (16 Q as fp16 hi + lo, rows = channels,
// k = input index n), B = the sign-flipped fp16 input (exact), fp32 accumulation.  Wave w owns
// channel blocks 2w and 2w+1 (groups 2w, 2w+1) and keeps their A operands in registers; the
// input tile is shared through LDS.  In the result each lane holds 4 consecutive channels of
// one vector, so a group of 16 channels spans 4 lanes (lane, lane+16, lane+32, lane+48).
// ------------------------------------------------------------------------------------------
namespace mq {

using dec::v8h;
using dec::v4f;

constexpr int kD = 128;
constexpr int kNStep = kD / 32;    // k steps of 32 inputs
constexpr int kVecs = 16;          // vectors per block (MFMA columns)

template <int BITS>
__device__ __forceinline__ float scale_of(float a) {
  // fp32 a / qmax, correctly rounded (reciprocal product plus one exact residual correction)
  constexpr float q = BITS == 4 ? 7.0f : 127.0f;
  constexpr float rq = 1.0f / q;
  const float y = a * rq;
  const float r = fmaf(-y, q, a);
  return fminf(fmaf(r, rq, y), 65504.0f);
}

template <int BITS, bool HAS_LAMBDA>
__global__ __launch_bounds__(256) void quantize_mfma_kernel(const uint16_t* __restrict__ x, int n_tok,
                                                           int kv_heads, int pos, int capacity,
                                                           const float* __restrict__ sign, int64_t sign_bs,
                                                           const float* __restrict__ lambda, int64_t lambda_bs,
                                                           uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                           int64_t n_vec) {
  constexpr int CB = kD * BITS / 8;  // code bytes per vector
  using CM = CodeMagic<BITS>;
  __shared__ __align__(16) uint4 xt[kVecs][16];          // 16 vectors x 256 B, piece p at p ^ v
  __shared__ __align__(16) uint8_t ct[kVecs][CB];        // packed codes
  __shared__ __align__(16) uint16_t st[kVecs][kD / 16];  // scales
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, r4 = lane >> 4;

  // A operands of this wave's two channel blocks (constant for the kernel)
  const dec::MfmaQTable<kD>& T = dec::mqtable<kD>();
  v8h ahi[2][kNStep], alo[2][kNStep];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int s = 0; s < kNStep; ++s) {
      const uint4 h = dec::ld4(T.fwd_hi[2 * w + i][s][lane]);
      const uint4 l = dec::ld4(T.fwd_lo[2 * w + i][s][lane]);
      ahi[i][s] = dec::as_v8h(h.x, h.y, h.z, h.w);
      alo[i][s] = dec::as_v8h(l.x, l.y, l.z, l.w);
    }

  float linv[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) linv[i][j] = 0.0625f;
  int64_t lam_row = -1;

  // each thread stages one 16-byte piece of one vector; the next block's piece is loaded while
  // the current block computes
  const int sv = tid >> 4, spc = tid & 15;
  uint4 nd;
  float4 ns0, ns1;
  auto load_piece = [&](int64_t blk_) {
    const int64_t gv = blk_ * kVecs + sv;
    nd = make_uint4(0u, 0u, 0u, 0u);
    ns0 = ns1 = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    if (gv < n_vec) {
      const int b = int((gv / n_tok) / kv_heads);
      nd = *reinterpret_cast<const uint4*>(x + gv * kD + spc * 8);
      ns0 = *reinterpret_cast<const float4*>(sign + b * sign_bs + spc * 8);
      ns1 = *reinterpret_cast<const float4*>(sign + b * sign_bs + spc * 8 + 4);
    }
  };
  load_piece(blockIdx.x);

  for (int64_t blk = blockIdx.x; blk * kVecs < n_vec; blk += gridDim.x) {
    // ---- stage 16 input vectors (sign bits flipped) in LDS ----
    {
      uint4 d = nd;
      d.x ^= (ns0.x < 0.0f ? 0x8000u : 0u) | (ns0.y < 0.0f ? 0x80000000u : 0u);
      d.y ^= (ns0.z < 0.0f ? 0x8000u : 0u) | (ns0.w < 0.0f ? 0x80000000u : 0u);
      d.z ^= (ns1.x < 0.0f ? 0x8000u : 0u) | (ns1.y < 0.0f ? 0x80000000u : 0u);
      d.w ^= (ns1.z < 0.0f ? 0x8000u : 0u) | (ns1.w < 0.0f ? 0x80000000u : 0u);
      xt[sv][spc ^ sv] = d;
    }
    __syncthreads();
    if ((blk + gridDim.x) * kVecs < n_vec) load_piece(blk + gridDim.x);
    // ---- transform: lane (vector n16, channels 16 cb + 4 r4 + i) ----
    v4f acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < kNStep; ++s) {
      const uint4 bx = xt[n16][(4 * s + r4) ^ n16];
      const v8h bop = dec::as_v8h(bx.x, bx.y, bx.z, bx.w);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[i][s], bop, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[i][s], bop, acc[i], 0, 0, 0);
      }
    }
    // ---- per-channel factor 1/(16 lambda) (recomputed when this lane's row changes), the group
    //      absmax, scale, codes ----
    const int64_t gv = blk * kVecs + n16;
    const int64_t row = gv < n_vec ? gv / n_tok : 0;
    if constexpr (HAS_LAMBDA) {
      if (row != lam_row) {
        lam_row = row;
        const int b = int(row / kv_heads), h = int(row - int64_t(b) * kv_heads);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float4 lm =
              *reinterpret_cast<const float4*>(lambda + b * lambda_bs + int64_t(h) * kD + 16 * (2 * w + i) + 4 * r4);
          linv[i][0] = 1.0f / (16.0f * lm.x);
          linv[i][1] = 1.0f / (16.0f * lm.y);
          linv[i][2] = 1.0f / (16.0f * lm.z);
          linv[i][3] = 1.0f / (16.0f * lm.w);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = 2 * w + i;
      float u[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) u[j] = acc[i][j] * linv[i][j];
      float a = fmaxf(fmaxf(fabsf(u[0]), fabsf(u[1])), fmaxf(fabsf(u[2]), fabsf(u[3])));
      a = fmaxf(a, __shfl_xor(a, 16));
      a = fmaxf(a, __shfl_xor(a, 32));
      const _Float16 sh = static_cast<_Float16>(scale_of<BITS>(a));
      const float sf = static_cast<float>(sh);
      const float inv = sf > 0.0f ? 1.0f / sf : 0.0f;
      uint32_t tq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float vq = fmaf(u[j], inv, CM::magic);
        vq = fminf(fmaxf(vq, CM::magic - CM::qmax), CM::magic + CM::qmax);
        tq[j] = __float_as_uint(vq);
      }
      if constexpr (BITS == 4) {
        const uint32_t byte0 = ((tq[1] << 4) | (tq[0] & 0xfu)) & 0xffu;
        const uint32_t byte1 = ((tq[3] << 4) | (tq[2] & 0xfu)) & 0xffu;
        *reinterpret_cast<uint16_t*>(&ct[n16][8 * g + 2 * r4]) = uint16_t((byte0 | (byte1 << 8)) ^ 0x8888u);
      } else {
        const uint32_t word = ((tq[0] & 0xffu) | ((tq[1] & 0xffu) << 8) | ((tq[2] & 0xffu) << 16) | (tq[3] << 24)) ^
                              CM::to_twos;
        *reinterpret_cast<uint32_t*>(&ct[n16][16 * g + 4 * r4]) = word;
      }
      if (r4 == 0) st[n16][g] = __builtin_bit_cast(uint16_t, sh);
    }
    __syncthreads();
    // ---- store codes (16 B per thread) and scales ----
    {
      constexpr int UNITS = kVecs * CB / 16;  // 16-byte code units
      if (tid < UNITS) {
        const int v = tid / (CB / 16), pc = tid - v * (CB / 16);
        const int64_t gvs = blk * kVecs + v;
        if (gvs < n_vec) {
          const int64_t rw = gvs / n_tok, tk = gvs - rw * n_tok;
          const int64_t slot = rw * capacity + pos + tk;
          *reinterpret_cast<uint4*>(codes + slot * CB + pc * 16) = *reinterpret_cast<const uint4*>(&ct[v][pc * 16]);
        }
      } else if (tid >= 128 && tid < 128 + kVecs) {
        const int v = tid - 128;
        const int64_t gvs = blk * kVecs + v;
        if (gvs < n_vec) {
          const int64_t rw = gvs / n_tok, tk = gvs - rw * n_tok;
          const int64_t slot = rw * capacity + pos + tk;
          *reinterpret_cast<uint4*>(scales + slot * (kD / 16)) = *reinterpret_cast<const uint4*>(&st[v][0]);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace mq

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

template <int BITS>
hipError_t quantize_mfma_dispatch(const QuantArgs& a, hipStream_t s) {
  const int64_t n_vec = int64_t(a.batch) * a.kv_heads * a.n_tok;
  const int64_t blocks = (n_vec + mq::kVecs - 1) / mq::kVecs;
  const int grid = int(std::min<int64_t>(blocks, 2048));
  auto* x = static_cast<const uint16_t*>(a.x);
  auto* codes = static_cast<uint8_t*>(a.codes);
  auto* scales = static_cast<uint16_t*>(a.scales);
  if (a.lambda)
    hipLaunchKernelGGL((mq::quantize_mfma_kernel<BITS, true>), dim3(grid), dim3(256), 0, s, x, a.n_tok, a.kv_heads,
                       a.pos, a.capacity, a.sign, a.sign_bs, a.lambda, a.lambda_bs, codes, scales, n_vec);
  else
    hipLaunchKernelGGL((mq::quantize_mfma_kernel<BITS, false>), dim3(grid), dim3(256), 0, s, x, a.n_tok, a.kv_heads,
                       a.pos, a.capacity, a.sign, a.sign_bs, a.lambda, a.lambda_bs, codes, scales, n_vec);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.head_dim == 128) return a.bits == 4 ? quantize_mfma_dispatch<4>(a, s) : quantize_mfma_dispatch<8>(a, s);
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
