// Shared pieces of the decode-attention kernels (gfx950): the SRFT entry table and the MFMA
// operands generated from it, 16-lane DPP row reductions, the end of a chunk (work-group partial
// of the online softmax) and the merge of the chunk partials of one (sequence, kv head, head
// tile) with the single inverse rotation, done by the last work-group of the unit to finish.
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

// ------------------------------------------------------------------------------------------
// SRFT entries generated in registers.  16 Q[c][n] depends on (c, n) only through the row
// kind (c = 0, c = 1, even c, odd c) and the angle m = (c/2) n mod D, so a table of 2D fp16
// (hi | lo << 16) pairs, interleaved per angle, gives every entry with one LDS read:
//   e[2m]     = 16 sqrt(2/D) cos(2 pi m / D)     (rows c = 2k, k >= 1)
//   e[2m + 1] = -16 sqrt(2/D) sin(2 pi m / D)    (rows c = 2k + 1, k >= 1)
//   rows 0 and 1: 16/sqrt(D) and (-1)^n 16/sqrt(D).
// The split is the one of the full table above (double -> float -> fp16 hi, residual -> lo).
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ v8h as_v8h(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  v4i t = {int(a), int(b), int(c), int(d)};
  return __builtin_bit_cast(v8h, t);
}

constexpr uint32_t split16(double v) {
  const float vf = float(v);
  const _Float16 hi = static_cast<_Float16>(vf);
  const _Float16 lo = static_cast<_Float16>(float(v - double(static_cast<float>(hi))));
  return uint32_t(__builtin_bit_cast(uint16_t, hi)) | (uint32_t(__builtin_bit_cast(uint16_t, lo)) << 16);
}

template <int D>
struct SrftPairs {
  uint32_t e[2 * D];
  constexpr SrftPairs() : e() {
    const double r2 = csqrt(2.0 / double(D));
    for (int m = 0; m < D; ++m) {
      const CosSin w = cos_sin_turn(m, D);
      e[2 * m] = split16(16.0 * (r2 * w.c));
      e[2 * m + 1] = split16(16.0 * (-(r2 * w.s)));
    }
  }
};

template <int D>
struct SrftRow0 {
  static constexpr uint32_t pos = split16(16.0 * (1.0 / csqrt(double(D))));
  static constexpr uint32_t neg = split16(16.0 * (-(1.0 / csqrt(double(D)))));
};

__device__ const SrftPairs<128> kSP128 = SrftPairs<128>();
__device__ const SrftPairs<256> kSP256 = SrftPairs<256>();

// Copy the pair table to LDS (2D words), all threads of the work-group: fetch into registers,
// then store (so the caller can issue other loads in between).
template <int D>
__device__ __forceinline__ void srft_pairs_fetch(uint32_t (&v)[2 * D / kThreads]) {
  const uint32_t* src = D == 128 ? kSP128.e : kSP256.e;
#pragma unroll
  for (int i = 0; i < 2 * D / kThreads; ++i) v[i] = src[threadIdx.x + i * kThreads];
}
template <int D>
__device__ __forceinline__ void srft_pairs_store(uint32_t* tw, const uint32_t (&v)[2 * D / kThreads]) {
#pragma unroll
  for (int i = 0; i < 2 * D / kThreads; ++i) tw[threadIdx.x + i * kThreads] = v[i];
}

// 16 Q[c][n] as an fp16 (hi | lo << 16) pair.
template <int D>
__device__ __forceinline__ uint32_t q_pair(const uint32_t* tw, int c, int n) {
  const uint32_t v = tw[2 * (((c >> 1) * n) & (D - 1)) + (c & 1)];
  return c >= 2 ? v : ((c & n & 1) ? SrftRow0<D>::neg : SrftRow0<D>::pos);
}

// B operand (hi and lo halves) of v_mfma_f32_16x16x32_f16 for step s and column block blk.
// Lane l holds k = 8 (l / 16) + j (j = 0..7) of column l % 16:
//   forward (q_hat = Q x):   B[k][col] = 16 Q[16 blk + col][32 s + k]
//   inverse (x = Q^T y):     B[k][col] = 16 Q[32 s + k][16 blk + col]
template <int D, bool INV>
__device__ __forceinline__ void srft_operand(const uint32_t* tw, int blk, int s, int lane, v8h& hi, v8h& lo) {
  const int fixed = 16 * blk + (lane & 15);
  const int k0 = 32 * s + 8 * (lane >> 4);
  uint32_t e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = INV ? q_pair<D>(tw, k0 + j, fixed) : q_pair<D>(tw, fixed, k0 + j);
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = (e[2 * i] & 0xffffu) | (e[2 * i + 1] << 16);
    l[i] = (e[2 * i] >> 16) | (e[2 * i + 1] & 0xffff0000u);
  }
  hi = as_v8h(h[0], h[1], h[2], h[3]);
  lo = as_v8h(l[0], l[1], l[2], l[3]);
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

// max / sum over the whole wave: 16-lane rows by DPP, then the four row results by readlane
// (wave-uniform result)
__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float exp2_guard(float a, float m) {
  // exp2(a - m) (v_exp_f32) with the empty case (a = -inf) mapped to 0
  return a == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(a - m);
}

// Position of token r (0..15) of a 16-token lane group inside the k order used by the value
// MFMA: the fp16 pairs built from 8 nibbles hold tokens (0,4),(1,5),(2,6),(3,7).
__host__ __device__ constexpr int kpos16(int r) {
  return (r < 8 ? 0 : 8) + ((r & 7) < 4 ? 2 * (r & 7) : 2 * ((r & 7) - 4) + 1);
}

// fp32 -> fp16 hi + lo, packed in pairs: x ~= hi + lo to ~2^-21 relative (while lo stays a
// normal fp16).  Both halves are truncations (v_cvt_pkrtz_f16_f32, two values per
// instruction); the residual x - hi is exact in fp32.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(a, b);
  const auto l = __builtin_amdgcn_cvt_pkrtz(a - static_cast<float>(h[0]), b - static_cast<float>(h[1]));
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}


// ------------------------------------------------------------------------------------------
// End of a chunk.  Every wave holds, for the heads of its slots, m (uniform in each 16-lane
// row), the per-lane partial l, and acc in the value-MFMA layout: lane (c = lane % 16,
// r4 = lane / 16) holds acc[g][i] for head 4*r4 + i, channel 16*g + c.  The work-group combines
// its 4 waves in LDS and stores one partial (m, l, acc[d]) per head of the unit.
// ------------------------------------------------------------------------------------------
// Chunk partials travel between work-groups that may sit on different XCDs (separate L2s).
// They are written and read as device-scope relaxed atomics (global_store / global_load with
// the sc1 scope bit), which the memory model keeps coherent at device scope without an L2
// writeback or invalidate; ordering against the completion counter comes from waiting for the
// stores to complete before the counter is incremented (arrive_last).
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

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
  // smem: wml[4][16][2] | fw[16][4] | hml[16][2] | wacc[4][GT][D]  (aliases the main-loop tiles)
  float* wml = smem;
  float* fw = smem + kWaves * 16 * 2;
  float* hml = fw + 16 * kWaves;
  float* wacc = hml + 16 * 2;
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
  // per head: the work-group max M, the wave weights exp2(m_w - M) and l = sum_w l_w weight_w
  if (threadIdx.x < 16) {
    const int h = threadIdx.x;
    float mm = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) mm = fmaxf(mm, wml[(ww * 16 + h) * 2]);
    float ll = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = exp2_guard(wml[(ww * 16 + h) * 2], mm);
      fw[h * kWaves + ww] = f;
      ll += wml[(ww * 16 + h) * 2 + 1] * f;
    }
    hml[2 * h] = mm;
    hml[2 * h + 1] = ll;
  }
  __syncthreads();
  // four consecutive channels of one head per thread
  for (int q = threadIdx.x; q < GT * D / 4; q += kThreads) {
    const int h = (4 * q) / D, c = 4 * q - h * D;
    const float4 f = *reinterpret_cast<const float4*>(fw + h * kWaves);
    const float fv[4] = {f.x, f.y, f.z, f.w};
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float4 v = *reinterpret_cast<const float4*>(wacc + (ww * GT + h) * D + c);
      a.x = fmaf(v.x, fv[ww], a.x);
      a.y = fmaf(v.y, fv[ww], a.y);
      a.z = fmaf(v.z, fv[ww], a.z);
      a.w = fmaf(v.w, fv[ww], a.w);
    }
    const int64_t prow = (e.unit * GT + h) * e.max_chunks + e.chunk_index;
    float* dst = e.pacc + prow * D + c;
    st_dev(dst, a.x);
    st_dev(dst + 1, a.y);
    st_dev(dst + 2, a.z);
    st_dev(dst + 3, a.w);
    if (c == 0) {
      st_dev(&e.pml[2 * prow], hml[2 * h]);
      st_dev(&e.pml[2 * prow + 1], hml[2 * h + 1]);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Completion count of a unit.  Every wave of the work-group waits until its device-scope
// partial stores have completed (s_waitcnt vmcnt(0)), the work-group synchronizes, and thread 0
// adds 1 to the unit's counter (a device-scope atomic).  The work-group that brings the count to
// n_chunks resets the counter to 0 for the next call and merges the unit; its device-scope
// loads are issued after the increment has returned, so they see every chunk's partial.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ bool arrive_last(uint32_t* counter, int n_chunks, int* flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + 1u == uint32_t(n_chunks);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last ? 1 : 0;
  }
  __syncthreads();
  return *flag != 0;
}

// ------------------------------------------------------------------------------------------
// Merge of one unit (sequence, kv head, head tile) by one work-group of 4 waves.  Every
// (head, channel) combines its chunks, y = acc_scale * acc / l; with ROT, y is scaled by
// lambda_V and inverse-rotated with MFMAs against generated operands (A = y split into fp16
// hi + lo):  x[h][n] = s_n sum_c y[h][c] Q[c][n].
// ------------------------------------------------------------------------------------------
struct MergeArgs {
  const float* pml;
  const float* pacc;
  int n_chunks, max_chunks, head_tile, head_tiles, q_heads, kv_heads;
  float acc_scale;
  const float* sign;
  int64_t sign_bs;
  const float* lambda;
  int64_t lambda_bs;
  float* out;
};

template <int D>
constexpr int merge_lds_floats() {
  return 16 * D + 16 * 32 + 32;
}

template <int D, bool ROT>
__device__ __forceinline__ void merge_unit(const MergeArgs& a, int unit, float* smem, const uint32_t* tw) {
  constexpr int MAXC = 32;  // chunks whose weights are staged in LDS at once
  constexpr int NP = 16 * D / kThreads;  // (head, channel) pairs per thread, at most
  constexpr int CR = 8 * 128 / D;        // chunks of each pair prefetched into registers
  float(*y)[D] = reinterpret_cast<float(*)[D]>(smem);
  float(*wgt)[MAXC] = reinterpret_cast<float(*)[MAXC]>(smem + 16 * D);
  float* linv = smem + 16 * D + 16 * MAXC;
  float* mmax = linv + 16;
  const int ht = unit % a.head_tiles;
  const int bk = unit / a.head_tiles;
  const int kvh = bk % a.kv_heads;
  const int b = bk / a.kv_heads;
  const int G = a.q_heads / a.kv_heads;
  const int GT = a.head_tile;
  const int n_chunks = a.n_chunks, max_chunks = a.max_chunks;
  const int64_t orow0 = int64_t(b) * a.q_heads + kvh * G + ht * GT;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int NB = D / 16, NSTEP = D / 32, NBW = NB / kWaves;
  // every load that does not depend on another goes out first: the first CR chunks of this
  // thread's (head, channel) pairs, lambda and the output signs, then the (m, l) pairs
  float pre[NP][CR];
  float lamv[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int idx = threadIdx.x + k * kThreads;
    const int h = idx / D, c = idx - h * D;
    lamv[k] = 1.0f;
#pragma unroll
    for (int i = 0; i < CR; ++i) pre[k][i] = 0.0f;
    if (h < GT) {
      const float* pa = a.pacc + (int64_t(unit) * GT + h) * max_chunks * D + c;
#pragma unroll
      for (int i = 0; i < CR; ++i)
        if (i < n_chunks) pre[k][i] = ld_dev(&pa[int64_t(i) * D]);
      if (ROT && a.lambda) lamv[k] = a.lambda[b * a.lambda_bs + int64_t(kvh) * D + c];
    }
  }
  float psg[ROT ? NBW : 1];
  // d = 128: the inverse-rotation operands come from the global table (d = 256: generated)
  constexpr bool kTab = ROT && D == 128;
  uint4 pbh[kTab ? NBW : 1][NSTEP], pbl[kTab ? NBW : 1][NSTEP];
  if constexpr (ROT) {
#pragma unroll
    for (int j = 0; j < NBW; ++j) psg[j] = a.sign[b * a.sign_bs + 16 * (w + kWaves * j) + (lane & 15)];
  }
  if constexpr (kTab) {
    const MfmaQTable<D>& T = mqtable<D>();
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        pbh[j][s] = ld4(T.inv_hi[w + kWaves * j][s][lane]);
        pbl[j][s] = ld4(T.inv_lo[w + kWaves * j][s][lane]);
      }
  }
  // per-head chunk weights exp2(m_i - M) and 1/l, one wave per head
  for (int h = w; h < GT; h += kWaves) {
    const float* ml = a.pml + (int64_t(unit) * GT + h) * max_chunks * 2;
    float mv[2], lv[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + 64 * r;
      mv[r] = i < n_chunks ? ld_dev(&ml[2 * i]) : -INFINITY;
      lv[r] = i < n_chunks ? ld_dev(&ml[2 * i + 1]) : 0.0f;
    }
    float mm = fmaxf(mv[0], mv[1]);
    for (int i = lane + 128; i < n_chunks; i += 64) mm = fmaxf(mm, ld_dev(&ml[2 * i]));
    mm = wave_max(mm);
    float ll = 0.0f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + 64 * r;
      const float f = exp2_guard(mv[r], mm);
      ll += lv[r] * f;
      if (i < MAXC) wgt[h][i] = f;
    }
    for (int i = lane + 128; i < n_chunks; i += 64) ll += ld_dev(&ml[2 * i + 1]) * exp2_guard(ld_dev(&ml[2 * i]), mm);
    ll = wave_sum(ll);
    if (lane == 0) {
      linv[h] = ll > 0.0f ? a.acc_scale / ll : 0.0f;
      mmax[h] = mm;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int idx = threadIdx.x + k * kThreads;
    const int h = idx / D, c = idx - h * D;
    float v = 0.0f;
    if (h < GT) {
      const float* pa = a.pacc + (int64_t(unit) * GT + h) * max_chunks * D + c;
      const float* ml = a.pml + (int64_t(unit) * GT + h) * max_chunks * 2;
      float acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < CR; ++i)
        if (i < n_chunks) acc4[i & 3] = fmaf(pre[k][i], wgt[h][i], acc4[i & 3]);
      for (int i = CR; i < n_chunks; ++i) {
        const float f = i < MAXC ? wgt[h][i] : exp2_guard(ld_dev(&ml[2 * i]), mmax[h]);
        acc4[i & 3] = fmaf(ld_dev(&pa[int64_t(i) * D]), f, acc4[i & 3]);
      }
      v = ((acc4[0] + acc4[1]) + (acc4[2] + acc4[3])) * linv[h];
      if constexpr (!ROT)
        a.out[(orow0 + h) * D + c] = v;
      else
        v *= lamv[k];
    }
    y[h][c] = v;
  }
  if constexpr (ROT) {
    __syncthreads();
    const int n16 = lane & 15, r4 = lane >> 4;
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
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NSTEP; ++s) {
        v8h bhi, blo;
        if constexpr (kTab) {
          bhi = as_v8h(pbh[j][s].x, pbh[j][s].y, pbh[j][s].z, pbh[j][s].w);
          blo = as_v8h(pbl[j][s].x, pbl[j][s].y, pbl[j][s].z, pbl[j][s].w);
        } else {
          srft_operand<D, true>(tw, nb, s, lane, bhi, blo);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[s], bhi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[s], blo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[s], bhi, acc, 0, 0, 0);
      }
      const int n = 16 * nb + n16;
      const float sg = (psg[j] < 0.0f ? -1.0f : 1.0f) * 0.0625f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * r4 + i;
        if (h < GT) a.out[(orow0 + h) * D + n] = acc[i] * sg;
      }
    }
  }
}

}  // namespace dec
}  // namespace kvq_impl
