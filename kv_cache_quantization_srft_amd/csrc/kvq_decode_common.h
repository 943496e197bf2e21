// Shared pieces of the decode-attention kernels (gfx950): workspace layout, 16-lane DPP row
// reductions, the online-softmax bookkeeping of one wave, and the epilogue that merges the
// per-chunk partials of one (sequence, kv head, head tile) in the last work-group to finish
// and applies the single inverse rotation.
//
// Partial results follow the tiled attention with online softmax of the hotdry blog
// ("Flash Attention 与 Metal 内核融合"): every chunk keeps (m, l, acc) with scores in log2
// units, and chunks combine by rescaling with exp2(m_chunk - m_max).
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq_impl {
namespace dec {

using namespace kvqd;

constexpr int kThreads = 256;  // 4 waves
constexpr int kWaves = 4;
constexpr float kLog2e = 1.44269504088896340736f;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4_t;
typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4_t;

// ------------------------------------------------------------------------------------------
// twiddles: cos/sin(2 pi m / N), m < N, exact to float rounding (compile-time)
// ------------------------------------------------------------------------------------------
template <int N>
struct TwTable {
  float c[N];
  float s[N];
  constexpr TwTable() : c(), s() {
    for (int m = 0; m < N; ++m) {
      const CosSin v = cos_sin_turn(m, N);
      c[m] = float(v.c);
      s[m] = float(v.s);
    }
  }
};

template <int D>
struct TwConst;
template <>
struct TwConst<128> {
  static constexpr TwTable<128> t = TwTable<128>();
};
template <>
struct TwConst<256> {
  static constexpr TwTable<256> t = TwTable<256>();
};

// The real orthogonal SRFT matrix (without the sign flip), Q[c][n]:
//   Q[0][n] = 1/sqrt(D), Q[1][n] = (-1)^n/sqrt(D),
//   Q[2k][n] = sqrt(2/D) cos(2 pi k n/D), Q[2k+1][n] = -sqrt(2/D) sin(2 pi k n/D),
// evaluated in double at compile time.  The tables hold 16*Q split into fp16 hi + lo (the x16
// keeps lo out of the fp16 subnormal range) laid out as B operands of v_mfma_f32_16x16x32_f16:
//   fwd[cb][s][lane][j] = 16 Q[16 cb + lane%16][32 s + 8 (lane/16) + j]   (q_hat = Q (s*q))
//   inv[nb][s][lane][j] = 16 Q[32 s + 8 (lane/16) + j][16 nb + lane%16]   (x = Q^T y)
// so one 16-byte load per lane fetches the operand of one MFMA.
// inv = 1/sqrt(D), r2 = sqrt(2/D), tw[m] = (cos, sin)(2 pi m / D)
constexpr double q_entry(int c, int n, int D, const CosSin* tw, double inv, double r2) {
  if (c == 0) return inv;
  if (c == 1) return (n & 1) ? -inv : inv;
  const CosSin w = tw[((c >> 1) * n) % D];
  return (c & 1) ? -r2 * w.s : r2 * w.c;
}

template <int D>
struct MfmaQTable {
  static constexpr int NB = D / 16, NSTEP = D / 32;
  uint32_t fwd_hi[NB][NSTEP][64][4];
  uint32_t fwd_lo[NB][NSTEP][64][4];
  uint32_t inv_hi[NB][NSTEP][64][4];
  uint32_t inv_lo[NB][NSTEP][64][4];
  constexpr MfmaQTable() : fwd_hi(), fwd_lo(), inv_hi(), inv_lo() {
    CosSin tw[D] = {};
    for (int m = 0; m < D; ++m) tw[m] = cos_sin_turn(m, D);
    const double inv = 1.0 / csqrt(double(D)), r2 = csqrt(2.0 / double(D));
    for (int b = 0; b < NB; ++b)
      for (int s = 0; s < NSTEP; ++s)
        for (int l = 0; l < 64; ++l)
          for (int j = 0; j < 8; ++j) {
            const int col = 16 * b + (l & 15), k = 32 * s + 8 * (l >> 4) + j;
            for (int which = 0; which < 2; ++which) {
              const double v = 16.0 * (which == 0 ? q_entry(col, k, D, tw, inv, r2) : q_entry(k, col, D, tw, inv, r2));
              const float vf = float(v);
              const _Float16 hi = static_cast<_Float16>(vf);
              const _Float16 lo = static_cast<_Float16>(float(v - double(static_cast<float>(hi))));
              const uint32_t hb = __builtin_bit_cast(uint16_t, hi), lb = __builtin_bit_cast(uint16_t, lo);
              uint32_t(&H)[4] = which == 0 ? fwd_hi[b][s][l] : inv_hi[b][s][l];
              uint32_t(&Lo)[4] = which == 0 ? fwd_lo[b][s][l] : inv_lo[b][s][l];
              H[j >> 1] |= hb << (16 * (j & 1));
              Lo[j >> 1] |= lb << (16 * (j & 1));
            }
          }
  }
};

__device__ const MfmaQTable<128> kMQ128 = MfmaQTable<128>();
__device__ const MfmaQTable<256> kMQ256 = MfmaQTable<256>();

template <int D>
__device__ __forceinline__ const MfmaQTable<D>& mqtable() {
  if constexpr (D == 128)
    return kMQ128;
  else
    return kMQ256;
}

__device__ __forceinline__ uint4 ld4(const uint32_t* p) { return *reinterpret_cast<const uint4*>(p); }

// ------------------------------------------------------------------------------------------
// cross-lane helpers
// ------------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// max / sum over the 16 lanes of a DPP row (rotations within the row)
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_mov<0x128>(v));  // row_ror:8
  v = fmaxf(v, dpp_mov<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_mov<0x122>(v));  // row_ror:2
  v = fmaxf(v, dpp_mov<0x121>(v));  // row_ror:1
  return v;
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<0x128>(v);
  v += dpp_mov<0x124>(v);
  v += dpp_mov<0x122>(v);
  v += dpp_mov<0x121>(v);
  return v;
}

__device__ __forceinline__ float exp2_guard(float a, float m) {
  // exp2(a - m) with the empty case (a = -inf) mapped to 0
  return a == -INFINITY ? 0.0f : exp2f(a - m);
}

// Position of token r (0..15) of a 16-token lane group inside the k order used by the value
// MFMA: the fp16 pairs built from 8 nibbles hold tokens (0,4),(1,5),(2,6),(3,7).
__host__ __device__ constexpr int kpos16(int r) {
  return (r < 8 ? 0 : 8) + ((r & 7) < 4 ? 2 * (r & 7) : 2 * ((r & 7) - 4) + 1);
}

// fp32 -> fp16 hi + lo, packed in pairs: x ~= hi + lo to ~2^-22 relative.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  const _Float16 ha = static_cast<_Float16>(a), hb = static_cast<_Float16>(b);
  const _Float16 la = static_cast<_Float16>(a - static_cast<float>(ha));
  const _Float16 lb = static_cast<_Float16>(b - static_cast<float>(hb));
  hi = uint32_t(__builtin_bit_cast(uint16_t, ha)) | (uint32_t(__builtin_bit_cast(uint16_t, hb)) << 16);
  lo = uint32_t(__builtin_bit_cast(uint16_t, la)) | (uint32_t(__builtin_bit_cast(uint16_t, lb)) << 16);
}

__device__ __forceinline__ v8h as_v8h(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  v4i t = {int(a), int(b), int(c), int(d)};
  return __builtin_bit_cast(v8h, t);
}

// ------------------------------------------------------------------------------------------
// End of a chunk.  Every wave holds, for the heads of its slots, m (uniform in each 16-lane
// row), the per-lane partial l, and acc in the value-MFMA layout: lane (c = lane % 16,
// r4 = lane / 16) holds acc[g][i] for head 4*r4 + i, channel 16*g + c.  The work-group combines
// its 4 waves in LDS and stores one partial (m, l, acc[d]) per head of the unit.
// ------------------------------------------------------------------------------------------
struct PartialArgs {
  int head_tile;
  int max_chunks, chunk_index;
  int64_t unit;
  float* pml;
  float* pacc;
};

template <int D, int NSLOT, typename HeadOf>
__device__ __forceinline__ void store_partial(float (&m_run)[NSLOT], float (&l_run)[NSLOT], v4f (&acc)[D / 16],
                                              HeadOf head_of, const PartialArgs& e, float* smem) {
  constexpr int NG = D / 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n16 = lane & 15, r4 = lane >> 4;
  const int GT = e.head_tile;
  // smem: wml[4][16][2] | wacc[4][GT][D]  (aliases the main-loop tiles)
  float* wml = smem;
  float* wacc = smem + kWaves * 16 * 2;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NSLOT; ++k) {
    const float lt = row_sum16(l_run[k]);
    const int h = head_of(k, r4);
    if (n16 == 0 && h < 16) {
      wml[(w * 16 + h) * 2] = m_run[k];
      wml[(w * 16 + h) * 2 + 1] = lt;
    }
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * r4 + i;
      if (h < GT) wacc[(w * GT + h) * D + 16 * g + n16] = acc[g][i];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < GT * D; idx += kThreads) {
    const int h = idx / D, c = idx - h * D;
    float mm = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) mm = fmaxf(mm, wml[(ww * 16 + h) * 2]);
    float a = 0.0f, ll = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = exp2_guard(wml[(ww * 16 + h) * 2], mm);
      a += wacc[(ww * GT + h) * D + c] * f;
      ll += wml[(ww * 16 + h) * 2 + 1] * f;
    }
    const int64_t prow = (e.unit * GT + h) * e.max_chunks + e.chunk_index;
    e.pacc[prow * D + c] = a;
    if (c == 0) {
      e.pml[2 * prow] = mm;
      e.pml[2 * prow + 1] = ll;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Merge: one work-group of 4 waves per unit (sequence, kv head, head tile).  Every (head,
// channel) combines its chunks, y = acc_scale * acc / l; with ROT, y is scaled by lambda_V and
// inverse-rotated with MFMAs against the inverse table (A = y split into fp16 hi + lo):
//   x[h][n] = s_n sum_c y[h][c] Q[c][n]
// ------------------------------------------------------------------------------------------
template <int D, bool ROT>
__global__ __launch_bounds__(kThreads) void merge_kernel(const float* __restrict__ pml, const float* __restrict__ pacc,
                                                        int n_chunks, int max_chunks, int head_tile, int head_tiles,
                                                        int q_heads, int kv_heads, float acc_scale,
                                                        const float* __restrict__ sign, int64_t sign_bs,
                                                        const float* __restrict__ lambda, int64_t lambda_bs,
                                                        float* __restrict__ out) {
  constexpr int MAXC = 32;  // chunks whose weights are staged in LDS at once
  __shared__ __align__(16) float y[16][D];
  __shared__ float wgt[16][MAXC];
  __shared__ float linv[16];
  __shared__ float mmax[16];
  const int unit = blockIdx.x;
  const int ht = unit % head_tiles;
  const int bk = unit / head_tiles;
  const int kvh = bk % kv_heads;
  const int b = bk / kv_heads;
  const int G = q_heads / kv_heads;
  const int GT = head_tile;
  const int64_t orow0 = int64_t(b) * q_heads + kvh * G + ht * head_tile;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int NB = D / 16, NSTEP = D / 32, NBW = NB / kWaves;
  // the inverse-rotation operands do not depend on the partials: load them first
  constexpr bool kPre = ROT && D == 128;
  uint4 pbh[kPre ? NBW : 1][NSTEP], pbl[kPre ? NBW : 1][NSTEP];
  float psg[kPre ? NBW : 1];
  if constexpr (kPre) {
    const MfmaQTable<D>& T0 = mqtable<D>();
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        pbh[j][s] = ld4(T0.inv_hi[w + kWaves * j][s][lane]);
        pbl[j][s] = ld4(T0.inv_lo[w + kWaves * j][s][lane]);
      }
      psg[j] = sign[b * sign_bs + 16 * (w + kWaves * j) + (lane & 15)];
    }
  }
  // per-head chunk weights exp2(m_i - M) and 1/l, one wave per head
  for (int h = w; h < GT; h += kWaves) {
    const float* ml = pml + (int64_t(unit) * GT + h) * max_chunks * 2;
    float mm = -INFINITY;
    for (int i = lane; i < n_chunks; i += 64) mm = fmaxf(mm, ml[2 * i]);
    for (int off = 32; off > 0; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off));
    float ll = 0.0f;
    for (int i = lane; i < n_chunks; i += 64) {
      const float f = exp2_guard(ml[2 * i], mm);
      ll += ml[2 * i + 1] * f;
      if (i < MAXC) wgt[h][i] = f;
    }
    for (int off = 32; off > 0; off >>= 1) ll += __shfl_xor(ll, off);
    if (lane == 0) {
      linv[h] = ll > 0.0f ? acc_scale / ll : 0.0f;
      mmax[h] = mm;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 16 * D; idx += kThreads) {
    const int h = idx / D, c = idx - h * D;
    float v = 0.0f;
    if (h < GT) {
      const float* pa = pacc + (int64_t(unit) * GT + h) * max_chunks * D + c;
      const float* ml = pml + (int64_t(unit) * GT + h) * max_chunks * 2;
      float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      int i = 0;
      for (; i + 4 <= n_chunks && i + 4 <= MAXC; i += 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = fmaf(pa[int64_t(i + j) * D], wgt[h][i + j], a[j]);
      }
      for (; i < n_chunks; ++i) {
        const float f = i < MAXC ? wgt[h][i] : exp2_guard(ml[2 * i], mmax[h]);
        a[0] = fmaf(pa[int64_t(i) * D], f, a[0]);
      }
      v = ((a[0] + a[1]) + (a[2] + a[3])) * linv[h];
      if constexpr (!ROT) {
        out[(orow0 + h) * D + c] = v;
      } else {
        if (lambda) v *= lambda[b * lambda_bs + int64_t(kvh) * D + c];
      }
    }
    y[h][c] = v;
  }
  if constexpr (ROT) {
    __syncthreads();
    const int n16 = lane & 15, r4 = lane >> 4;
    const MfmaQTable<D>& T = mqtable<D>();
    // A operands: y[head n16][32 s + 8 r4 + (0..7)] split into hi + lo
    v8h ahi[NSTEP], alo[NSTEP];
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      const float4 y0 = *reinterpret_cast<const float4*>(&y[n16][32 * s + 8 * r4]);
      const float4 y1 = *reinterpret_cast<const float4*>(&y[n16][32 * s + 8 * r4 + 4]);
      uint32_t h4[4], l4[4];
      split_pair(y0.x, y0.y, h4[0], l4[0]);
      split_pair(y0.z, y0.w, h4[1], l4[1]);
      split_pair(y1.x, y1.y, h4[2], l4[2]);
      split_pair(y1.z, y1.w, h4[3], l4[3]);
      ahi[s] = as_v8h(h4[0], h4[1], h4[2], h4[3]);
      alo[s] = as_v8h(l4[0], l4[1], l4[2], l4[3]);
    }
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int nb = w + kWaves * j;
      uint4 bh[NSTEP], bl[NSTEP];
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        if constexpr (kPre) {
          bh[s] = pbh[j][s];
          bl[s] = pbl[j][s];
        } else {
          bh[s] = ld4(T.inv_hi[nb][s][lane]);
          bl[s] = ld4(T.inv_lo[nb][s][lane]);
        }
      }
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        const v8h bhi = as_v8h(bh[s].x, bh[s].y, bh[s].z, bh[s].w);
        const v8h blo = as_v8h(bl[s].x, bl[s].y, bl[s].z, bl[s].w);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[s], bhi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[s], blo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[s], bhi, acc, 0, 0, 0);
      }
      const int n = 16 * nb + n16;
      float sgn;
      if constexpr (kPre)
        sgn = psg[j];
      else
        sgn = sign[b * sign_bs + n];
      const float sg = (sgn < 0.0f ? -1.0f : 1.0f) * 0.0625f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * r4 + i;
        if (h < GT) out[(orow0 + h) * D + n] = acc[i] * sg;
      }
    }
  }
}

}  // namespace dec
}  // namespace kvq_impl
