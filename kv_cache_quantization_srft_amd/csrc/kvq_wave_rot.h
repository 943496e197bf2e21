// The rotation of up to 16 head vectors by one work-group, for the decode kernel's query
// (forward) and output (inverse) rotations: wave w transforms rows w, w+4, w+8, w+12 in registers,
// with the butterflies' partners fetched across lanes (DPP and lane-swap instructions), so no
// work-group barrier sits inside a transform.
//
// SRFT ("When Quantization Is Free", technical summary, Methodology 1 and 2): the d-point real
// DFT of y = s * x is computed as the M = d/2-point complex FFT of z[m] = y[2m] + i y[2m+1],
// followed by the Hermitian unpack of its half spectrum into the packed real slots
//   [X0, X_{d/2}, sqrt2 Re X1, sqrt2 Im X1, ...] / sqrt(d).
// Lane l holds complex points m = l + 64 p (p < M/64).  The FFT is radix-2 decimation in
// frequency: the span-64 stage (d = 256) pairs the two points of a lane, the spans 32 .. 1 pair
// lane l with lane l ^ span.  Its output is in bit-reversed order; the unpack fetches the
// mirrored bin Z_{M-k} from the lane that holds it.  The inverse packs the slots into the half
// spectrum in natural order, runs the same stages with conjugate twiddles and writes the
// outputs of the bit-reversed positions.
// SRHT (the Walsh-Hadamard alternative): lane l holds values n = l + 64 e; the Hadamard stages
// are the same butterflies without twiddles, in natural order.
//
// All arithmetic is float32; the only table is each lane's twiddles (64 or 96 bytes per lane).
#pragma once
#include "kvq_device.h"

namespace kvq_impl {
namespace dec {

template <int D>
struct RotGeom {
  static constexpr int M = D / 2;       // complex points
  static constexpr int P = M / 64;      // complex points per lane and row
  static constexpr int E = D / 64;      // real values per lane and row (Hadamard)
  static constexpr int LOGM = D == 128 ? 6 : 7;
  static constexpr int NST = LOGM;      // FFT stages (spans M/2 .. 1)
  static constexpr int PITCH = D + 4;   // floats per row of the forward output block
};

// ---- cross-lane partner: the value of lane l ^ H ----
template <int CTRL>
__device__ __forceinline__ float rot_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int H>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (H == 1) {
    return rot_dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (H == 2) {
    return rot_dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (H == 4) {
    return rot_dpp<0x1B>(rot_dpp<0x141>(v));  // row_half_mirror, then quad_perm [3,2,1,0]
  } else if constexpr (H == 8) {
    return rot_dpp<0x128>(v);  // row_ror:8
  } else {
    // the swap leaves the lane's own value in one result and its partner's in the other
    const uint32_t u = __float_as_uint(v);
    if constexpr (H == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      return __uint_as_float(r[0] ^ r[1] ^ u);
    } else {
      const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      return __uint_as_float(r[0] ^ r[1] ^ u);
    }
  }
}

// m with its LOGM low bits reversed
template <int D>
__host__ __device__ constexpr int bitrev_m(int m) {
  return int(__builtin_bitreverse32(uint32_t(m)) >> (32 - RotGeom<D>::LOGM));
}

// Per-lane twiddles of the transforms, one contiguous record per lane (read with 16-byte loads):
//   sc[j], ss[j]: stage j (span H = M >> (j+1)) twiddle W_M^{(m mod H) M/(2H)} of this lane's
//          upper points ((1, 0) on the lower points of a cross-lane stage; the span-64 stage of
//          d = 256 uses the lane's own point m = l)
//   uc[p], us[p]: forward unpack, W_D^k for the bin k = bitrev(l + 64 p) the lane holds after
//          the FFT; inverse pack (INVERSE): W_D^k for k = l + 64 p
template <int D>
struct RotTw {
  float sc[RotGeom<D>::NST], ss[RotGeom<D>::NST];
  float uc[RotGeom<D>::P], us[RotGeom<D>::P];
};

template <int D>
struct LaneTwiddles {
  static constexpr int NST = RotGeom<D>::NST, P = RotGeom<D>::P;
  static constexpr int F = 2 * (NST + 2 * P);  // stages, forward unpack, inverse pack
  static constexpr int Q4 = (F + 3) / 4;       // float4 per lane
  float v[64][4 * Q4];
  constexpr LaneTwiddles() : v() {
    constexpr int M = RotGeom<D>::M;
    for (int l = 0; l < 64; ++l) {
      for (int j = 0; j < NST; ++j) {
        const int H = M >> (j + 1);
        const bool one = H < 64 && (l & H) == 0;
        const int t = H == 64 ? 2 * l : 2 * (l & (H - 1)) * (M / (2 * H));
        const kvqd::CosSin cs = kvqd::cos_sin_turn(t, D);
        v[l][2 * j] = one ? 1.0f : float(cs.c);
        v[l][2 * j + 1] = one ? 0.0f : float(cs.s);
      }
      for (int p = 0; p < P; ++p) {
        const kvqd::CosSin f = kvqd::cos_sin_turn(bitrev_m<D>(l + 64 * p), D);
        const kvqd::CosSin i = kvqd::cos_sin_turn(l + 64 * p, D);
        v[l][2 * NST + 2 * p] = float(f.c);
        v[l][2 * NST + 2 * p + 1] = float(f.s);
        v[l][2 * NST + 2 * P + 2 * p] = float(i.c);
        v[l][2 * NST + 2 * P + 2 * p + 1] = float(i.s);
      }
    }
  }
};
__device__ const LaneTwiddles<128> kLaneTw128{};
__device__ const LaneTwiddles<256> kLaneTw256{};

template <int D, bool INVERSE>
__device__ __forceinline__ void load_rot_tw(RotTw<D>& tw) {
  using LT = LaneTwiddles<D>;
  const int lane = threadIdx.x & 63;
  const float* src;
  if constexpr (D == 128)
    src = kLaneTw128.v[lane];
  else
    src = kLaneTw256.v[lane];
  float f[4 * LT::Q4];
#pragma unroll
  for (int q = 0; q < LT::Q4; ++q) {
    const float4 x = reinterpret_cast<const float4*>(src)[q];
    f[4 * q] = x.x, f[4 * q + 1] = x.y, f[4 * q + 2] = x.z, f[4 * q + 3] = x.w;
  }
#pragma unroll
  for (int j = 0; j < LT::NST; ++j) {
    tw.sc[j] = f[2 * j];
    tw.ss[j] = f[2 * j + 1];
  }
  constexpr int U = 2 * LT::NST + (INVERSE ? 2 * LT::P : 0);
#pragma unroll
  for (int p = 0; p < LT::P; ++p) {
    tw.uc[p] = f[U + 2 * p];
    tw.us[p] = f[U + 2 * p + 1];
  }
}

// (re, im) times (c - i s) (forward) or (c + i s) (inverse)
template <bool INV>
__device__ __forceinline__ void cmul_tw(float& re, float& im, float c, float s) {
  const float r0 = re, i0 = im;
  if constexpr (!INV) {
    re = fmaf(r0, c, i0 * s);
    im = fmaf(i0, c, -(r0 * s));
  } else {
    re = fmaf(r0, c, -(i0 * s));
    im = fmaf(i0, c, r0 * s);
  }
}

// Cross-lane DIF stage of span H on one complex value per lane.  With a the lower and b the upper
// point of a pair, the lower lane keeps a + b and the upper one (a - b) W, i.e. partner - own
// (its twiddle is (1, 0) on the lower lanes).
template <int H, bool INV>
__device__ __forceinline__ void dif_xstage(float& re, float& im, float c, float s, int lane) {
  const float pr = lane_xor<H>(re), pi = lane_xor<H>(im);
  const float sg = (lane & H) ? -1.0f : 1.0f;
  re = fmaf(sg, re, pr);  // lower: own + partner; upper: partner - own
  im = fmaf(sg, im, pi);
  cmul_tw<INV>(re, im, c, s);
}

// Full M-point DIF FFT of the lane-distributed points z[p] (point l + 64 p); bit-reversed output.
template <int D, bool INV>
__device__ __forceinline__ void fft_wave(float (&zr)[RotGeom<D>::P], float (&zi)[RotGeom<D>::P], const RotTw<D>& tw,
                                         int lane) {
  using G = RotGeom<D>;
  int j = 0;
  if constexpr (G::P == 2) {  // span 64: the two points of the lane
    const float ar = zr[0], ai = zi[0], br = zr[1], bi = zi[1];
    zr[0] = ar + br;
    zi[0] = ai + bi;
    float dr = ar - br, di = ai - bi;
    cmul_tw<INV>(dr, di, tw.sc[0], tw.ss[0]);
    zr[1] = dr;
    zi[1] = di;
    j = 1;
  }
#pragma unroll
  for (int p = 0; p < G::P; ++p) {
    dif_xstage<32, INV>(zr[p], zi[p], tw.sc[j + 0], tw.ss[j + 0], lane);
    dif_xstage<16, INV>(zr[p], zi[p], tw.sc[j + 1], tw.ss[j + 1], lane);
    dif_xstage<8, INV>(zr[p], zi[p], tw.sc[j + 2], tw.ss[j + 2], lane);
    dif_xstage<4, INV>(zr[p], zi[p], tw.sc[j + 3], tw.ss[j + 3], lane);
    dif_xstage<2, INV>(zr[p], zi[p], tw.sc[j + 4], tw.ss[j + 4], lane);
    dif_xstage<1, INV>(zr[p], zi[p], tw.sc[j + 5], tw.ss[j + 5], lane);
  }
}

// Walsh-Hadamard of the lane-distributed values v[e] (value l + 64 e), natural order.
template <int D>
__device__ __forceinline__ void wht_wave(float (&v)[RotGeom<D>::E], int lane) {
  kvqd::wht<RotGeom<D>::E>(v);  // spans 64 (and 128): within the lane
#pragma unroll
  for (int e = 0; e < RotGeom<D>::E; ++e) {
    float x = v[e];
    x = fmaf((lane & 32) ? -1.0f : 1.0f, x, lane_xor<32>(x));
    x = fmaf((lane & 16) ? -1.0f : 1.0f, x, lane_xor<16>(x));
    x = fmaf((lane & 8) ? -1.0f : 1.0f, x, lane_xor<8>(x));
    x = fmaf((lane & 4) ? -1.0f : 1.0f, x, lane_xor<4>(x));
    x = fmaf((lane & 2) ? -1.0f : 1.0f, x, lane_xor<2>(x));
    x = fmaf((lane & 1) ? -1.0f : 1.0f, x, lane_xor<1>(x));
    v[e] = x;
  }
}

// ---------------------------------------------------------------------------------------------
// Forward rotation of rows w + 4 i (wave w, i < 4).  fwd_load issues the loads (row_src(r, x)
// returns whether row r has an input and sets its fp16 row; every row takes the signs srow,
// except row 15 when s15 is not null); fwd_wave transforms and writes the rows to qo (LDS,
// pitch PITCH; rows without input are written as zeros).  The caller's barrier publishes qo.
// ---------------------------------------------------------------------------------------------
template <int D>
struct FwdIn {
  uint32_t x[4][RotGeom<D>::E];  // SRFT: dwords l + 64 p (P of them); SRHT: halves l + 64 e
  float s[RotGeom<D>::E];        // signs of those values (SRFT: pairs) in the sign row of all rows
  float s15[RotGeom<D>::E];      // ... in the sign row of row 15 when it has its own
  bool live[4];
  bool own15;                    // row 15 of this wave takes s15
};

template <int D>
__device__ __forceinline__ void load_signs(float (&sv)[RotGeom<D>::E], const float* srow, int transform) {
  using G = RotGeom<D>;
  const int lane = threadIdx.x & 63;
  if (transform) {
#pragma unroll
    for (int e = 0; e < G::E; ++e) sv[e] = srow[lane + 64 * e];
  } else {
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
      const float2 v = reinterpret_cast<const float2*>(srow)[lane + 64 * p];
      sv[2 * p] = v.x;
      sv[2 * p + 1] = v.y;
    }
  }
}

template <int D, typename RowSrc>
__device__ __forceinline__ void fwd_load(FwdIn<D>& in, int transform, const float* srow, const float* s15,
                                         RowSrc&& row_src) {
  using G = RotGeom<D>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const uint16_t* x = nullptr;
    in.live[rr] = row_src(w + 4 * rr, x);
#pragma unroll
    for (int e = 0; e < G::E; ++e) in.x[rr][e] = 0u;
    if (!in.live[rr]) continue;
    if (transform) {
#pragma unroll
      for (int e = 0; e < G::E; ++e) in.x[rr][e] = x[lane + 64 * e];
    } else {
#pragma unroll
      for (int p = 0; p < G::P; ++p) in.x[rr][p] = reinterpret_cast<const uint32_t*>(x)[lane + 64 * p];
    }
  }
  load_signs<D>(in.s, srow, transform);
  in.own15 = s15 != nullptr && w == 3 && in.live[3];
  if (in.own15) load_signs<D>(in.s15, s15, transform);
}

__device__ __forceinline__ float signed_half(uint32_t bits16, float s) {
  const float v = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
  return s < 0.0f ? -v : v;
}

template <int D>
__device__ __forceinline__ void fwd_wave(const FwdIn<D>& in, const RotTw<D>& tw, int transform, float* qo) {
  using G = RotGeom<D>;
  constexpr int M = G::M;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    float* o = qo + (w + 4 * rr) * G::PITCH;
    if (!in.live[rr]) {
#pragma unroll
      for (int e = 0; e < G::E; ++e) o[lane + 64 * e] = 0.0f;
      continue;
    }
    if (transform) {
      const bool o15 = rr == 3 && in.own15;
      float v[G::E];
#pragma unroll
      for (int e = 0; e < G::E; ++e) v[e] = signed_half(in.x[rr][e] & 0xffffu, o15 ? in.s15[e] : in.s[e]);
      wht_wave<D>(v, lane);
      constexpr float nrm = kvqd::inv_sqrt_d<D>();
#pragma unroll
      for (int e = 0; e < G::E; ++e) o[lane + 64 * e] = v[e] * nrm;
      continue;
    }
    const bool o15 = rr == 3 && in.own15;
    float zr[G::P], zi[G::P];
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
      zr[p] = signed_half(in.x[rr][p] & 0xffffu, o15 ? in.s15[2 * p] : in.s[2 * p]);
      zi[p] = signed_half(in.x[rr][p] >> 16, o15 ? in.s15[2 * p + 1] : in.s[2 * p + 1]);
    }
    fft_wave<D, false>(zr, zi, tw, lane);
    // lane l, point p now holds Z_k, k = bitrev(l + 64 p); fetch Z_{M-k} from the lane holding it
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
      const int k = bitrev_m<D>(lane + 64 * p);
      const int mm = bitrev_m<D>((M - k) & (M - 1));  // position of Z_{M-k}
      const int addr = (mm & 63) * 4;
      float br, bi;
      if constexpr (G::P == 1) {
        br = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(zr[0])));
        bi = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(zi[0])));
      } else {
        const float r0 = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(zr[0])));
        const float i0 = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(zi[0])));
        const float r1 = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(zr[1])));
        const float i1 = __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(zi[1])));
        br = mm >= 64 ? r1 : r0;
        bi = mm >= 64 ? i1 : i0;
      }
      const float ar = zr[p], ai = zi[p];
      if (k == 0) {
        constexpr float n0 = kvqd::inv_sqrt_d<D>();
        *reinterpret_cast<float2*>(o) = make_float2((ar + ai) * n0, (ar - ai) * n0);
      } else {
        constexpr float nh = float(1.0 / kvqd::csqrt(2.0 * double(D)));  // sqrt2 / sqrt(D) on 2 X_k
        const float er = ar + br, ei = ai - bi;  // 2E = a + conj(b)
        float orr = ai + bi, oi = br - ar;       // 2O = -i (a - conj(b))
        cmul_tw<false>(orr, oi, tw.uc[p], tw.us[p]);
        *reinterpret_cast<float2*>(o + 2 * k) = make_float2((er + orr) * nh, (ei + oi) * nh);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Inverse rotation of rows w + 4 i (< n_rows) of y (LDS, pitch yp, unitary packed slots).
// sg[]: this lane's output signs (SRFT: outputs 2n, 2n+1 of n = bitrev(l + 64 p), in pairs;
// SRHT: outputs l + 64 e), loaded by load_inv_signs.  store(row, n, v) receives output n of the
// row, normalized and sign-flipped; SRFT stores come in pairs (n even, then n + 1) through
// store2(row, n, v0, v1).  Begins after a barrier that made y visible.
// ---------------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void load_inv_signs(float (&sg)[RotGeom<D>::E], const float* srow, int transform) {
  using G = RotGeom<D>;
  const int lane = threadIdx.x & 63;
  if (transform) {
#pragma unroll
    for (int e = 0; e < G::E; ++e) sg[e] = srow[lane + 64 * e];
  } else {
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
      const float2 v = reinterpret_cast<const float2*>(srow)[bitrev_m<D>(lane + 64 * p)];
      sg[2 * p] = v.x;
      sg[2 * p + 1] = v.y;
    }
  }
}

template <int D, typename Store2, typename Store1>
__device__ __forceinline__ void inv_wave(const float* y, int yp, int n_rows, int transform, const RotTw<D>& tw,
                                         const float (&sg)[RotGeom<D>::E], Store2&& store2, Store1&& store1) {
  using G = RotGeom<D>;
  constexpr int M = G::M;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int row = w + 4 * rr;
    if (row >= n_rows) break;
    const float* a = y + row * yp;
    if (transform) {
      float v[G::E];
#pragma unroll
      for (int e = 0; e < G::E; ++e) v[e] = a[lane + 64 * e];
      wht_wave<D>(v, lane);
      constexpr float nrm = kvqd::inv_sqrt_d<D>();
#pragma unroll
      for (int e = 0; e < G::E; ++e) {
        const float u = v[e] * nrm;
        store1(row, lane + 64 * e, sg[e] < 0.0f ? -u : u);
      }
      continue;
    }
    // Hermitian pack of the slots into Z_k, k = l + 64 p (real_inv_raw's steps)
    float zr[G::P], zi[G::P];
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
      const int k = lane + 64 * p;
      const float2 A = *reinterpret_cast<const float2*>(a + 2 * k);
      const float2 B = *reinterpret_cast<const float2*>(a + 2 * ((M - k) & (M - 1)));
      if (k == 0) {
        constexpr float kSqrt2 = 1.41421356237309504880f;
        const float a0 = kSqrt2 * A.x, am = kSqrt2 * A.y;  // slot 0 = X0, slot 1 = X_{D/2}
        zr[p] = a0 + am;
        zi[p] = a0 - am;
      } else {
        const float er = A.x + B.x, ei = A.y - B.y;  // E = A[k] + conj(A[M-k])
        float dr = A.x - B.x, di = A.y + B.y;        // A[k] - conj(A[M-k])
        cmul_tw<true>(dr, di, tw.uc[p], tw.us[p]);   // conj(W^k) (.)
        zr[p] = er - di;                             // E + i conj(W^k) (.)
        zi[p] = ei + dr;
      }
    }
    fft_wave<D, true>(zr, zi, tw, lane);
    constexpr float nrm = kvqd::inv_norm<D>();
#pragma unroll
    for (int p = 0; p < G::P; ++p) {
      const int n = bitrev_m<D>(lane + 64 * p);
      const float v0 = zr[p] * nrm, v1 = zi[p] * nrm;
      store2(row, 2 * n, sg[2 * p] < 0.0f ? -v0 : v0, sg[2 * p + 1] < 0.0f ? -v1 : v1);
    }
  }
}

}  // namespace dec
}  // namespace kvq_impl
