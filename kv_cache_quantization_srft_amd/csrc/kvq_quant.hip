// Write path for gfx950: SRFT rotation + per-channel lambda + group-of-16 absmax quantization
// + packing ("When Quantization Is Free", technical summary, Methodology 2 and 3).  The
// rotation of 16 vectors at a time is a d x d matrix product on MFMA (quantize_mfma_kernel,
// below), which leaves the VALU free for the absmax, rounding and packing.
#include <algorithm>

#include "kvq_decode_common.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq_impl {
namespace {

using namespace kvqd;

// ------------------------------------------------------------------------------------------
// Write path on MFMA.  u = Q (s * x) / lambda for 16 vectors at a time with
// v_mfma_f32_16x16x32_f16: A = the forward table (16 Q as fp16 hi + lo, rows = channels,
// k = input index n), B = the sign-flipped fp16 input (exact), fp32 accumulation.  Wave w owns
// channel blocks 2w and 2w+1 (groups 2w, 2w+1) and keeps their A operands in registers; the
// input tile is shared through LDS.  In the result each lane holds 4 consecutive channels of
// one vector, so a group of 16 channels spans 4 lanes (lane, lane+16, lane+32, lane+48).
// ------------------------------------------------------------------------------------------
// n / d for 32-bit n and a divisor fixed per launch: floor(n / d) = floor(M n / 2^64) with
// M = ceil(2^64 / d) for every n < 2^32 (Lemire, Kaser and Kurz, "Faster remainder by direct
// computation", 2019), i.e. one 32x64-bit high product instead of a division.
struct FastDiv {
  uint32_t d, mh, ml;  // M = mh 2^32 + ml (unused for d = 1)
  static FastDiv make(uint32_t d) {
    FastDiv f{d, 0u, 0u};
    if (d > 1) {
      const uint64_t m = ~uint64_t(0) / d + 1;
      f.mh = uint32_t(m >> 32);
      f.ml = uint32_t(m);
    }
    return f;
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    if (d == 1) return n;
    const uint64_t t = uint64_t(mh) * n + __umulhi(ml, n);
    return uint32_t(t >> 32);
  }
};

namespace mq {

// The real orthogonal SRFT matrix (without the sign flip), Q[c][n]:
//   Q[0][n] = 1/sqrt(D), Q[1][n] = (-1)^n/sqrt(D),
//   Q[2k][n] = sqrt(2/D) cos(2 pi k n/D), Q[2k+1][n] = -sqrt(2/D) sin(2 pi k n/D),
// evaluated in double at compile time.  The table holds 16*Q split into fp16 hi + lo (the x16
// keeps lo out of the fp16 subnormal range) laid out as operands of v_mfma_f32_16x16x32_f16:
//   fwd[cb][s][lane][j] = 16 Q[16 cb + lane%16][32 s + 8 (lane/16) + j]   (u = Q (s*x))
// so one 16-byte load per lane fetches the operand of one MFMA.
// inv = 1/sqrt(D), r2 = sqrt(2/D), tw[m] = (cos, sin)(2 pi m / D)
constexpr double q_entry(int c, int n, int D, const CosSin* tw, double inv, double r2) {
  if (c == 0) return inv;
  if (c == 1) return (n & 1) ? -inv : inv;
  const CosSin w = tw[((c >> 1) * n) % D];
  return (c & 1) ? -r2 * w.s : r2 * w.c;
}

// The SRHT (Sylvester-ordered Walsh-Hadamard) counterpart, d^-1/2 H[c][n] with
// H[c][n] = (-1)^popcount(c & n); inv = 1/sqrt(D).
constexpr double h_entry(int c, int n, double inv) { return (__builtin_popcount(c & n) & 1) ? -inv : inv; }

template <int D>
struct MfmaQTable {
  static constexpr int NB = D / 16, NSTEP = D / 32;
  uint32_t fwd_hi[NB][NSTEP][64][4];
  uint32_t fwd_lo[NB][NSTEP][64][4];
  // had = false: the SRFT matrix Q; had = true: the SRHT matrix d^-1/2 H
  constexpr MfmaQTable(bool had = false) : fwd_hi(), fwd_lo() {
    CosSin tw[D] = {};
    if (!had)
      for (int m = 0; m < D; ++m) tw[m] = cos_sin_turn(m, D);
    const double inv = 1.0 / csqrt(double(D)), r2 = csqrt(2.0 / double(D));
    for (int b = 0; b < NB; ++b)
      for (int s = 0; s < NSTEP; ++s)
        for (int l = 0; l < 64; ++l)
          for (int j = 0; j < 8; ++j) {
            const int r = 16 * b + (l & 15), cl = 32 * s + 8 * (l >> 4) + j;  // Q[r][cl]
            const double v = 16.0 * (had ? h_entry(r, cl, inv) : q_entry(r, cl, D, tw, inv, r2));
            const float vf = float(v);
            const _Float16 hi = static_cast<_Float16>(vf);
            const _Float16 lo = static_cast<_Float16>(float(v - double(static_cast<float>(hi))));
            const uint32_t hb = __builtin_bit_cast(uint16_t, hi), lb = __builtin_bit_cast(uint16_t, lo);
            fwd_hi[b][s][l][j >> 1] |= hb << (16 * (j & 1));
            fwd_lo[b][s][l][j >> 1] |= lb << (16 * (j & 1));
          }
  }
};

__device__ const MfmaQTable<128> kMQ128 = MfmaQTable<128>(false);
__device__ const MfmaQTable<256> kMQ256 = MfmaQTable<256>(false);
__device__ const MfmaQTable<128> kMH128 = MfmaQTable<128>(true);
__device__ const MfmaQTable<256> kMH256 = MfmaQTable<256>(true);

// transform: 0 = SRFT, 1 = SRHT (uniform across the launch)
template <int D>
__device__ __forceinline__ const MfmaQTable<D>& mqtable(int transform) {
  if constexpr (D == 128)
    return transform ? kMH128 : kMQ128;
  else
    return transform ? kMH256 : kMQ256;
}

using dec::v8h;
using dec::v4f;

constexpr int kVecs = kQuantVecs;  // vectors per block (MFMA columns)

// Codes by magic-number rounding: fma(u, 1/scale, M) rounds u/scale to an integer (ties to even)
// for M = 1.5 * 2^23, whose neighbourhood has unit spacing and whose low bits are zero, so the
// low 4 (8) bits of the clamped sum are the code in two's complement.
template <int BITS>
struct TwosMagic {
  static constexpr float qmax = BITS == 4 ? 7.0f : 127.0f;
  static constexpr float magic = 12582912.0f;  // 1.5 * 2^23
};

// fp32 a / (F qmax) for a power of two F, correctly rounded (reciprocal product plus one exact
// residual correction) and saturated at the fp16 maximum: the scale of a group whose absmax is
// a / F (the division by F is exact, and 1/(F qmax) rounds like 1/qmax scaled by 1/F)
template <int BITS, int F>
__device__ __forceinline__ float scale_of_scaled(float a) {
  constexpr float q = (BITS == 4 ? 7.0f : 127.0f) * F;
  constexpr float rq = 1.0f / q;
  const float y = a * rq;
  const float r = fmaf(-y, q, a);
  return fminf(fmaf(r, rq, y), 65504.0f);
}

// XOR mask that flips the fp16 signs of 8 consecutive channels where sign < 0
__device__ __forceinline__ uint4 sign_mask(float4 s0, float4 s1) {
  return make_uint4((s0.x < 0.0f ? 0x8000u : 0u) | (s0.y < 0.0f ? 0x80000000u : 0u),
                    (s0.z < 0.0f ? 0x8000u : 0u) | (s0.w < 0.0f ? 0x80000000u : 0u),
                    (s1.x < 0.0f ? 0x8000u : 0u) | (s1.y < 0.0f ? 0x80000000u : 0u),
                    (s1.z < 0.0f ? 0x8000u : 0u) | (s1.w < 0.0f ? 0x80000000u : 0u));
}

// Write path of D-dim vectors, 16 vectors per block, 2D threads per work-group: every thread
// stages one 16-byte piece of one vector; wave w rotates channel blocks 2w, 2w + 1 of all 16
// vectors with MFMAs (A = 16 Q as fp16 hi + lo from the constant table, B = the sign-flipped
// fp16 inputs), then scales, rounds and packs them.  Each work-group takes a contiguous range of
// blocks and walks it in halves, the next half's inputs in flight while the current one is
// transformed; the code and scale tiles are double-buffered.  SHARED: every row uses sign row 0
// (sign_bs == 0), so the sign mask is fixed per thread and the in-flight registers hold data
// only, which leaves room for four blocks per half (one with per-row signs).
template <int D, int BITS, bool HAS_LAMBDA, bool SHARED, bool PT>
__global__ __launch_bounds__(2 * D) __attribute__((amdgpu_waves_per_eu(D == 128 ? 3 : 2))) void quantize_mfma_kernel(const uint16_t* __restrict__ x, FastDiv fd_tok,
                                                              FastDiv fd_heads, int pos, int capacity,
                                                              const float* __restrict__ sign, int64_t sign_bs,
                                                              const float* __restrict__ lambda, int64_t lambda_bs,
                                                              uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                              uint32_t n_vec, int transform) {
  constexpr int NP = D / 8;         // 16-byte pieces per vector
  constexpr int NSTEP = D / 32;     // k steps of 32 inputs
  constexpr int CB = D * BITS / 8;  // code bytes per vector
  constexpr int NG = D / 16;        // groups (= channel blocks) per vector
  using CM = TwosMagic<BITS>;
  constexpr int HX = SHARED ? 4 : 1;                      // blocks staged per half
  __shared__ __align__(16) uint4 xt[HX][kVecs][NP];       // inputs, piece p of vector v at p ^ v
  __shared__ __align__(16) uint8_t ct[2][kVecs][CB];      // packed codes
  __shared__ __align__(16) uint16_t st[2][kVecs][NG];     // scales
  __shared__ float tmax[PT ? D / 32 : 1][kVecs];          // per-token mode: per-wave absmax
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, r4 = lane >> 4;

  // A operands of this wave's two channel blocks (constant for the kernel)
  const MfmaQTable<D>& T = mqtable<D>(transform);
  v8h ahi[2][NSTEP], alo[2][NSTEP];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
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
  uint32_t lam_lo = 1u, lam_hi = 0u;  // vectors [lam_lo, lam_hi) share the row whose linv is held
  // vector gv is token gv - row n_tok of row (sequence b, kv head h) = gv / n_tok
  auto slot_of = [&](uint32_t gv) {
    const uint32_t rw = fd_tok.div(gv);
    return int64_t(rw) * capacity + pos + (gv - rw * fd_tok.d);
  };

  // this thread's piece: vector sv of the block, channels 8 spc .. 8 spc + 7
  const int sv = tid / NP, spc = tid % NP;
  // Blocks are processed in halves of H blocks (four, or one with per-row signs).  A half first
  // stages all of its H input blocks (loaded one half earlier) in LDS, then requests the next
  // half's blocks into the other register set, then transforms and stores its blocks.  The
  // loads and stores of a wave share one completion counter and may complete out of order, so
  // the wait before staging is a full drain: staging first means it drains loads issued a whole
  // half ago, not the ones just requested.
  constexpr int H = HX;
  const uint4 smask0 = SHARED ? sign_mask(*reinterpret_cast<const float4*>(sign + spc * 8),
                                          *reinterpret_cast<const float4*>(sign + spc * 8 + 4))
                              : make_uint4(0u, 0u, 0u, 0u);
  uint4 pd[2][H], pm[2][SHARED ? 1 : H];
  // this work-group's blocks: a contiguous range, so consecutive blocks share a row (and its
  // lambda) except at row boundaries
  const uint32_t nblk = (n_vec + kVecs - 1) / kVecs;
  const uint32_t blk_begin = uint32_t(uint64_t(blockIdx.x) * nblk / gridDim.x);
  const uint32_t blk_end = uint32_t(uint64_t(blockIdx.x + 1) * nblk / gridDim.x);
  const uint32_t v_end = min(blk_end * uint32_t(kVecs), n_vec);  // the range's vectors end here
  // A half's H input blocks are read through one buffer resource over the range's vectors from
  // the half's first block on (a scalar base), at the thread's fixed byte offset in each block:
  // a vector past the range reads zeros, a block past it is never processed, and a vector past
  // the range inside a processed block has its column of the product never stored (columns do
  // not mix).
  const int loff = (sv * D + spc * 8) * 2;
  auto load_half = [&](uint32_t first, uint4 (&d_)[H], uint4 (&m_)[SHARED ? 1 : H]) {
    const uint32_t g0 = first * kVecs;
    const uint32_t nv = v_end > g0 ? min(v_end - g0, uint32_t(H * kVecs)) : 0u;
    const __amdgpu_buffer_rsrc_t r = dec::buf_rsrc(x + int64_t(g0) * D, int64_t(nv) * D * 2);
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const dec::v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, loff + i * kVecs * D * 2, 0, 0);
      d_[i] = make_uint4(uint32_t(v[0]), uint32_t(v[1]), uint32_t(v[2]), uint32_t(v[3]));
      if constexpr (!SHARED) {
        const uint32_t gv = min(g0 + uint32_t(i * kVecs + sv), n_vec - 1u);
        const int b = int(fd_heads.div(fd_tok.div(gv)));
        m_[i] = sign_mask(*reinterpret_cast<const float4*>(sign + b * sign_bs + spc * 8),
                          *reinterpret_cast<const float4*>(sign + b * sign_bs + spc * 8 + 4));
      }
    }
  };
  load_half(blk_begin, pd[0], pm[0]);
  // first slot and in-row position of the block to be stored next (work-group uniform), carried
  // from block to block: the next block starts kVecs tokens later in the same row unless the row
  // ends inside this one
  uint32_t cur_t0 = 0;
  int64_t cur_slot0 = 0;
  auto seek = [&](uint32_t b) {
    const uint32_t gv0 = b * kVecs;
    const uint32_t row0 = fd_tok.div(gv0);
    cur_t0 = gv0 - row0 * fd_tok.d;
    cur_slot0 = int64_t(row0) * capacity + pos + cur_t0;
  };
  seek(blk_begin);

  // block blk from staged tile f (0..H-1); codes and scales go through LDS buffer f & 1
  auto do_block = [&](uint32_t blk, auto F) {
    constexpr int f = decltype(F)::value;
    constexpr int buf = f & 1;
    // ---- transform: lane (vector n16, channels 16 cb + 4 r4 + i) ----
    // two accumulation chains (one per channel block), the hi and lo operands accumulating into
    // the same fp32 sum
    v4f acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      const uint4 bx = xt[f][n16][(4 * s + r4) ^ n16];
      const v8h bop = dec::as_v8h(bx.x, bx.y, bx.z, bx.w);
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[i][s], bop, acc[i], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[i][s], bop, acc[i], 0, 0, 0);
    }
    // ---- per-channel factor 1/(16 lambda) (recomputed when this lane's row changes), the group
    //      absmax, scale, codes ----
    if constexpr (HAS_LAMBDA) {
      const uint32_t gv = min(blk * kVecs + n16, n_vec - 1u);
      if (gv < lam_lo || gv >= lam_hi) {
        const uint32_t row = fd_tok.div(gv);
        lam_lo = row * fd_tok.d;
        lam_hi = lam_lo + fd_tok.d;
        const uint32_t b = fd_heads.div(row), h = row - b * fd_heads.d;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float4 lm = *reinterpret_cast<const float4*>(lambda + int64_t(b) * lambda_bs + int64_t(h) * D +
                                                             16 * (2 * w + i) + 4 * r4);
          linv[i][0] = __builtin_amdgcn_rcpf(16.0f * lm.x);
          linv[i][1] = __builtin_amdgcn_rcpf(16.0f * lm.y);
          linv[i][2] = __builtin_amdgcn_rcpf(16.0f * lm.z);
          linv[i][3] = __builtin_amdgcn_rcpf(16.0f * lm.w);
        }
      }
    }
    // u = acc / (16 lambda).  Without lambda the factor is the exact 1/16, folded into the scale's
    // divisor and into the group's reciprocal instead of applied to every value (bit-identical
    // codes), so the maxima below are 16 times the group maxima there
    float u[2][4], am[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) u[i][j] = HAS_LAMBDA ? acc[i][j] * linv[i][j] : acc[i][j];
      // NaN-propagating maxima of the magnitudes (v_maximum3_f32 with abs modifiers)
      am[i] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(fabsf(u[i][0]), fabsf(u[i][1])),
                                            __builtin_elementwise_maximum(fabsf(u[i][2]), fabsf(u[i][3])));
    }
    // Group maxima over the four 16-lane rows, both groups at once: one v_permlane32_swap of the
    // two groups' values leaves one group's pairs in one half of the wave and the other group's in
    // the other half, so after the max and a v_permlane16_swap step each half holds one group's
    // maximum for every vector.  The scale is then computed once per lane, and a second
    // v_permlane32_swap hands every lane both groups' values (non-negative floats order like their
    // bit patterns, NaN above all).
    uint32_t mh;
    {
      const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(am[0]), __float_as_uint(am[1]), false, false);
      mh = max(uint32_t(r32[0]), uint32_t(r32[1]));
      const auto r16 = __builtin_amdgcn_permlane16_swap(mh, mh, false, false);
      mh = max(uint32_t(r16[0]), uint32_t(r16[1]));
    }
    float inv[2];
    uint32_t shb[2];
    if constexpr (PT) {
      // one scale per vector: the absmax over all channels, i.e. over this wave's two groups and
      // then over the waves (every lane of vector n16 holds the same per-wave value)
      const auto r = __builtin_amdgcn_permlane32_swap(mh, mh, false, false);
      if (r4 == 0) tmax[w][n16] = __uint_as_float(max(uint32_t(r[0]), uint32_t(r[1])));
      __syncthreads();
      float m = 0.0f;
#pragma unroll
      for (int ww = 0; ww < D / 32; ++ww) m = fmaxf(m, tmax[ww][n16]);
      const _Float16 sh = static_cast<_Float16>(scale_of_scaled<BITS, HAS_LAMBDA ? 1 : 16>(m));
      const float sf = static_cast<float>(sh);
      inv[0] = inv[1] = (sf > 0.0f ? __builtin_amdgcn_rcpf(sf) : 0.0f) * (HAS_LAMBDA ? 1.0f : 0.0625f);
      shb[0] = shb[1] = __builtin_bit_cast(uint16_t, sh);
    } else {
      const _Float16 sh = static_cast<_Float16>(scale_of_scaled<BITS, HAS_LAMBDA ? 1 : 16>(__uint_as_float(mh)));
      const float sf = static_cast<float>(sh);
      const float iv = (sf > 0.0f ? __builtin_amdgcn_rcpf(sf) : 0.0f) * (HAS_LAMBDA ? 1.0f : 0.0625f);
      const auto ri = __builtin_amdgcn_permlane32_swap(__float_as_uint(iv), __float_as_uint(iv), false, false);
      inv[0] = __uint_as_float(ri[0]);
      inv[1] = __uint_as_float(ri[1]);
      const uint32_t sb = __builtin_bit_cast(uint16_t, sh);
      const auto rs = __builtin_amdgcn_permlane32_swap(sb, sb, false, false);
      shb[0] = rs[0];
      shb[1] = rs[1];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = 2 * w + i;
      uint32_t tq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float vq = fmaf(u[i][j], inv[i], CM::magic);
        vq = fminf(fmaxf(vq, CM::magic - CM::qmax), CM::magic + CM::qmax);
        tq[j] = __float_as_uint(vq);
      }
      // pack the low nibbles (bytes): two shift-or pairs, then one byte permute
      if constexpr (BITS == 4) {
        const uint32_t b0 = (tq[0] & 0xfu) | (tq[1] << 4), b1 = (tq[2] & 0xfu) | (tq[3] << 4);
        *reinterpret_cast<uint16_t*>(&ct[buf][n16][8 * g + 2 * r4]) = uint16_t(__builtin_amdgcn_perm(b1, b0, 0x0c0c0400u));
      } else {
        const uint32_t lo = __builtin_amdgcn_perm(tq[1], tq[0], 0x0c0c0400u);
        const uint32_t hi = __builtin_amdgcn_perm(tq[3], tq[2], 0x0c0c0400u);
        *reinterpret_cast<uint32_t*>(&ct[buf][n16][16 * g + 4 * r4]) = lo | (hi << 16);
      }
      if (r4 == 0 && (!PT || g == 0)) st[buf][n16][g] = uint16_t(shb[i]);
    }
    __syncthreads();
    // ---- store codes (16 B per thread) and scales ----
    {
      // the block's first slot (work-group uniform); a block inside one row needs no division
      const uint32_t gv0 = blk * kVecs;
      const uint32_t t0 = cur_t0;
      const int64_t slot0 = cur_slot0;
      const bool one_row = t0 + kVecs <= fd_tok.d;
      if (t0 + kVecs < fd_tok.d) {
        cur_t0 = t0 + kVecs;
        cur_slot0 = slot0 + kVecs;
      } else {
        seek(blk + 1);
      }
      auto vslot = [&](uint32_t gvs, int v) { return one_row ? slot0 + v : slot_of(gvs); };
      constexpr int UNITS = kVecs * CB / 16;  // 16-byte code units
      constexpr int SUNITS = kVecs * NG / 8;  // 16-byte scale units
      if (one_row && gv0 + kVecs <= n_vec) {
        // the block's 16 slots are consecutive: unit u of the LDS tiles goes to unit u of the
        // planes after the first slot (scalar base plus the thread's offset)
        if (tid < UNITS) {
          *reinterpret_cast<uint4*>(codes + slot0 * CB + 16 * tid) =
              *reinterpret_cast<const uint4*>(&ct[buf][0][0] + 16 * tid);
        } else if (PT && tid < UNITS + kVecs) {
          scales[slot0 + (tid - UNITS)] = st[buf][tid - UNITS][0];
        } else if (!PT && tid < UNITS + SUNITS) {
          *reinterpret_cast<uint4*>(scales + slot0 * NG + 8 * (tid - UNITS)) =
              *reinterpret_cast<const uint4*>(&st[buf][0][0] + 8 * (tid - UNITS));
        }
      } else if (tid < UNITS) {
        const int v = tid / (CB / 16), pc = tid - v * (CB / 16);
        const uint32_t gvs = blk * kVecs + v;
        if (gvs < n_vec)
          *reinterpret_cast<uint4*>(codes + vslot(gvs, v) * CB + pc * 16) =
              *reinterpret_cast<const uint4*>(&ct[buf][v][pc * 16]);
      } else if (PT && tid >= UNITS && tid < UNITS + kVecs) {
        const int v = tid - UNITS;  // one fp16 scale per vector
        const uint32_t gvs = blk * kVecs + v;
        if (gvs < n_vec) scales[vslot(gvs, v)] = st[buf][v][0];
      } else if (!PT && tid >= UNITS && tid < UNITS + SUNITS) {
        const int u = tid - UNITS;
        const int v = u / (NG / 8), pc = u - v * (NG / 8);
        const uint32_t gvs = blk * kVecs + v;
        if (gvs < n_vec)
          *reinterpret_cast<uint4*>(scales + vslot(gvs, v) * NG + pc * 8) =
              *reinterpret_cast<const uint4*>(&st[buf][v][pc * 8]);
      }
    }
  };
  uint32_t blk = blk_begin;
  while (blk < blk_end) {  // blk advances inside the halves
    static_for<0, 2>([&](auto HF) {
      constexpr int hf = decltype(HF)::value;
      if (blk >= blk_end) return;  // work-group uniform
      // ---- stage this half's input blocks (sign bits flipped) in LDS ----
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const uint4 m = SHARED ? smask0 : pm[hf][SHARED ? 0 : i];
        const uint4 v = pd[hf][i];
        xt[i][sv][spc ^ sv] = make_uint4(v.x ^ m.x, v.y ^ m.y, v.z ^ m.z, v.w ^ m.w);
      }
      // ---- request the next half's blocks of this range ----
      load_half(blk + uint32_t(H), pd[1 - hf], pm[1 - hf]);
      __syncthreads();
      static_for<0, H>([&](auto F) {
        const uint32_t bk = blk + uint32_t(decltype(F)::value);
        if (bk < blk_end) do_block(bk, F);  // work-group uniform
      });
      blk += uint32_t(H);
    });
  }
}

}  // namespace mq

}  // namespace

template <int D, int BITS, bool PT>
hipError_t quantize_mfma_dispatch(const QuantArgs& a, hipStream_t s) {
  const uint32_t n_vec = uint32_t(a.batch) * uint32_t(a.kv_heads) * uint32_t(a.n_tok);  // < 2^31 (validated)
  const FastDiv fd_tok = FastDiv::make(uint32_t(a.n_tok)), fd_heads = FastDiv::make(uint32_t(a.kv_heads));
  const int grid = plan_quantize(D, n_vec).grid;
  auto* x = static_cast<const uint16_t*>(a.x);
  auto* codes = static_cast<uint8_t*>(a.codes);
  auto* scales = static_cast<uint16_t*>(a.scales);
#define KVQ_QLAUNCH(LAM, SH)                                                                                        \
  hipLaunchKernelGGL((mq::quantize_mfma_kernel<D, BITS, LAM, SH, PT>), dim3(grid), dim3(2 * D), 0, s, x, fd_tok, fd_heads, \
                     a.pos, a.capacity, a.sign, a.sign_bs, a.lambda, a.lambda_bs, codes, scales, n_vec, a.transform)
  const bool shared = a.sign_bs == 0;
  if (a.lambda) {
    if (shared)
      KVQ_QLAUNCH(true, true);
    else
      KVQ_QLAUNCH(true, false);
  } else {
    if (shared)
      KVQ_QLAUNCH(false, true);
    else
      KVQ_QLAUNCH(false, false);
  }
#undef KVQ_QLAUNCH
  return hipGetLastError();
}

template <bool PT>
hipError_t launch_quantize_g(const QuantArgs& a, hipStream_t s) {
  if (a.head_dim == 128)
    return a.bits == 4 ? quantize_mfma_dispatch<128, 4, PT>(a, s) : quantize_mfma_dispatch<128, 8, PT>(a, s);
  return a.bits == 4 ? quantize_mfma_dispatch<256, 4, PT>(a, s) : quantize_mfma_dispatch<256, 8, PT>(a, s);
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  // group == head_dim: one scale per vector (the per-token comparison mode)
  return a.group == a.head_dim ? launch_quantize_g<true>(a, s) : launch_quantize_g<false>(a, s);
}

}  // namespace kvq_impl
