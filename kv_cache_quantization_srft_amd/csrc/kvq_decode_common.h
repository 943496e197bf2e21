// Shared pieces of the decode-attention kernels (gfx950): 16-lane DPP row reductions, the end of
// a chunk (work-group partial of the online softmax) and the merge of the chunk partials of one
// (sequence, kv head, head tile) with the single inverse rotation, done by the last work-group of
// the unit to finish.
//
// Partial results follow the tiled attention with online softmax of the hotdry blog
// ("Flash Attention 与 Metal 内核融合"): every chunk keeps (m, l, acc) with scores in log2
// units, and chunks combine by rescaling with exp2(m_chunk - m_max).
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_wave_rot.h"

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

__device__ __forceinline__ v8h as_v8h(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  v4i t = {int(a), int(b), int(c), int(d)};
  return __builtin_bit_cast(v8h, t);
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
// They are written and read with device-scope accesses (the sc1 scope bit, as the memory model
// uses for device-scope relaxed atomics), which stay coherent at device scope without an L2
// writeback or invalidate; ordering against the completion counter comes from waiting for the
// stores to complete before the counter is incremented (arrive_last).
// The accesses go through buffer resources over the unit's partials with the cache policy of
// device scope (sc1: written through to / read from the device's coherence point), 8 or 16
// bytes at a time.
constexpr int kDevScope = 16;  // cache-policy operand of the buffer intrinsics: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int64_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(n), 0x00020000);
}
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t r, int off, float4 v) {
  const v4f x = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, x), r, off, 0, kDevScope);
}
__device__ __forceinline__ void st_dev2(__amdgpu_buffer_rsrc_t r, int off, float a, float b) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i x = {__float_as_int(a), __float_as_int(b)};
  __builtin_amdgcn_raw_buffer_store_b64(x, r, off, 0, kDevScope);
}
__device__ __forceinline__ float4 ld_dev4(__amdgpu_buffer_rsrc_t r, int off) {
  const v4i x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDevScope);
  return make_float4(__int_as_float(x[0]), __int_as_float(x[1]), __int_as_float(x[2]), __int_as_float(x[3]));
}
__device__ __forceinline__ float2 ld_dev2(__amdgpu_buffer_rsrc_t r, int off) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kDevScope);
  return make_float2(__int_as_float(x[0]), __int_as_float(x[1]));
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
  // four consecutive channels of one head per thread; the unit's partials: pacc rows
  // (h, chunk) of D floats, pml pairs (m, l) per (h, chunk)
  const __amdgpu_buffer_rsrc_t racc = buf_rsrc(e.pacc + e.unit * GT * e.max_chunks * D, int64_t(GT) * e.max_chunks * D * 4);
  const __amdgpu_buffer_rsrc_t rml = buf_rsrc(e.pml + e.unit * GT * e.max_chunks * 2, int64_t(GT) * e.max_chunks * 8);
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
    const int prow = h * e.max_chunks + e.chunk_index;
    st_dev4(racc, (prow * D + c) * 4, a);
    if (c == 0) st_dev2(rml, prow * 8, hml[2 * h], hml[2 * h + 1]);
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
// A unit is ((sequence b, kv head) x head tile ht) x query-token tile tt; it owns `rows` (head_tile
// below) query rows, row r = (token tt * tok_tile + r / gt, head ht * gt + r % gt).  Single-token
// decode has tok_tile = tok_tiles = n_query = 1 and rows = gt.
struct MergeArgs {
  const float* pml;
  const float* pacc;
  int n_chunks, max_chunks, head_tile, head_tiles, q_heads, kv_heads;
  int gt, tok_tile, tok_tiles, n_query;
  float acc_scale;
  const float* sign;
  int64_t sign_bs;
  const float* lambda;
  int64_t lambda_bs;
  float* out;
  int transform;  // rotation to invert: 0 = SRFT, 1 = SRHT
};

template <int D>
constexpr int merge_lds_floats() {
  return 16 * D + 16 * 32 + 32;
}

// Values the inverse rotation takes from global memory, loaded ahead of the merge: this lane's
// twiddles and output signs.
template <int D>
struct RotOps {
  RotTw<D> tw;
  float sg[RotGeom<D>::E];
};

template <int D>
__device__ __forceinline__ void rot_prefetch(RotOps<D>& o, const MergeArgs& a, int b) {
  load_rot_tw<D, true>(o.tw);
  load_inv_signs<D>(o.sg, a.sign + b * a.sign_bs, a.transform);
}

// Sequence and kv head of a unit; orow0 = output row of the unit's row 0, tt = its token tile.
__device__ __forceinline__ void unit_coords(const MergeArgs& a, int unit, int& b, int& kvh, int64_t& orow0) {
  const int tt = unit % a.tok_tiles;
  const int hu = unit / a.tok_tiles;
  const int ht = hu % a.head_tiles;
  const int bk = hu / a.head_tiles;
  kvh = bk % a.kv_heads;
  b = bk / a.kv_heads;
  orow0 = (int64_t(b) * a.n_query + tt * a.tok_tile) * a.q_heads + kvh * (a.q_heads / a.kv_heads) + ht * a.gt;
}

// Output row of row r of the unit whose row 0 is orow0, or -1 past the last query token.
__device__ __forceinline__ int64_t out_row(const MergeArgs& a, int unit, int64_t orow0, int r) {
  if (a.tok_tiles == 1 && a.tok_tile == 1) return orow0 + r;
  const int i = r / a.gt;
  if ((unit % a.tok_tiles) * a.tok_tile + i >= a.n_query) return -1;
  return orow0 + int64_t(i) * a.q_heads + (r - i * a.gt);
}

// out[h][n] = s_n (SRFT^-1 y[h])_n (SRHT: s_n d^-1/2 (H y[h])_n) for the rows h < head_tile of
// the unit (the output rows of query tokens past the last are skipped), with y in LDS (pitch D).
template <int D>
__device__ __forceinline__ void rotate_store(const MergeArgs& a, int unit, const float* y, const RotOps<D>& o) {
  int b, kvh;
  int64_t orow0;
  unit_coords(a, unit, b, kvh, orow0);
  inv_wave<D>(
      y, D, a.head_tile, a.transform, o.tw, o.sg,
      [&](int h, int n, float v0, float v1) {
        const int64_t orow = out_row(a, unit, orow0, h);
        if (orow >= 0) *reinterpret_cast<float2*>(a.out + orow * D + n) = make_float2(v0, v1);
      },
      [&](int h, int n, float v) {
        const int64_t orow = out_row(a, unit, orow0, h);
        if (orow >= 0) a.out[orow * D + n] = v;
      });
}

// Merge of the n_chunks partials of one unit from the workspace (the last work-group to
// finish).  Every (head, channel) combines its chunks, y = acc_scale * acc / l; with ROT, y is
// scaled by lambda_V and inverse-rotated.  Each thread owns quads of 4 consecutive channels of
// one head; the first CR chunks of its quads are loaded at once, before the (m, l) pairs.
template <int D, bool ROT>
__device__ __forceinline__ void merge_unit(const MergeArgs& a, int unit, float* smem) {
  constexpr int MAXC = 32;                    // chunks whose weights are staged in LDS at once
  constexpr int GTMAX = D == 128 ? 16 : 8;    // largest head tile
  constexpr int NQ = (GTMAX * D / 4 + kThreads - 1) / kThreads;  // quads per thread, at most
  constexpr int CR = 8;                       // chunks prefetched into registers
  float(*y)[D] = reinterpret_cast<float(*)[D]>(smem);
  float(*wgt)[MAXC] = reinterpret_cast<float(*)[MAXC]>(smem + 16 * D);
  float* linv = smem + 16 * D + 16 * MAXC;
  float* mmax = linv + 16;
  int b, kvh;
  int64_t orow0;
  unit_coords(a, unit, b, kvh, orow0);
  const int GT = a.head_tile;
  const int n_chunks = a.n_chunks, max_chunks = a.max_chunks;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t racc =
      buf_rsrc(a.pacc + int64_t(unit) * GT * max_chunks * D, int64_t(GT) * max_chunks * D * 4);
  const __amdgpu_buffer_rsrc_t rml = buf_rsrc(a.pml + int64_t(unit) * GT * max_chunks * 2, int64_t(GT) * max_chunks * 8);
  float4 pre[NQ][CR];
  float4 lam4[NQ];
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int q = threadIdx.x + k * kThreads;
    const int h = (4 * q) / D, c = 4 * q - h * D;
    lam4[k] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
#pragma unroll
    for (int i = 0; i < CR; ++i) pre[k][i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (h < GT) {
#pragma unroll
      for (int i = 0; i < CR; ++i)
        if (i < n_chunks) pre[k][i] = ld_dev4(racc, ((h * max_chunks + i) * D + c) * 4);
      if (ROT && a.lambda)
        lam4[k] = *reinterpret_cast<const float4*>(a.lambda + b * a.lambda_bs + int64_t(kvh) * D + c);
    }
  }
  RotOps<D> ro;
  if constexpr (ROT) rot_prefetch<D>(ro, a, b);
  // per-head chunk weights exp2(m_i - M) and 1/l, one wave per head
  for (int h = w; h < GT; h += kWaves) {
    float mv[2], lv[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + 64 * r;
      const float2 v = i < n_chunks ? ld_dev2(rml, (h * max_chunks + i) * 8) : make_float2(-INFINITY, 0.0f);
      mv[r] = v.x;
      lv[r] = v.y;
    }
    float mm = fmaxf(mv[0], mv[1]);
    for (int i = lane + 128; i < n_chunks; i += 64) mm = fmaxf(mm, ld_dev2(rml, (h * max_chunks + i) * 8).x);
    mm = wave_max(mm);
    float ll = 0.0f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + 64 * r;
      const float f = exp2_guard(mv[r], mm);
      ll += lv[r] * f;
      if (i < MAXC) wgt[h][i] = f;
    }
    for (int i = lane + 128; i < n_chunks; i += 64) {
      const float2 v = ld_dev2(rml, (h * max_chunks + i) * 8);
      ll += v.y * exp2_guard(v.x, mm);
    }
    ll = wave_sum(ll);
    if (lane == 0) {
      linv[h] = ll > 0.0f ? a.acc_scale / ll : 0.0f;
      mmax[h] = mm;
    }
  }
  __syncthreads();
  float4 yv[NQ];
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int q = threadIdx.x + k * kThreads;
    const int h = (4 * q) / D, c = 4 * q - h * D;
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (h < GT) {
#pragma unroll
      for (int i = 0; i < CR; ++i)
        if (i < n_chunks) {
          const float f = wgt[h][i];
          v = make_float4(fmaf(pre[k][i].x, f, v.x), fmaf(pre[k][i].y, f, v.y), fmaf(pre[k][i].z, f, v.z),
                          fmaf(pre[k][i].w, f, v.w));
        }
      for (int i = CR; i < n_chunks; ++i) {
        const float f = i < MAXC ? wgt[h][i] : exp2_guard(ld_dev2(rml, (h * max_chunks + i) * 8).x, mmax[h]);
        const float4 p = ld_dev4(racc, ((h * max_chunks + i) * D + c) * 4);
        v = make_float4(fmaf(p.x, f, v.x), fmaf(p.y, f, v.y), fmaf(p.z, f, v.z), fmaf(p.w, f, v.w));
      }
      const float li = linv[h];
      v = make_float4(v.x * li * lam4[k].x, v.y * li * lam4[k].y, v.z * li * lam4[k].z, v.w * li * lam4[k].w);
      if constexpr (!ROT) *reinterpret_cast<float4*>(a.out + out_row(a, unit, orow0, h) * D + c) = v;
    }
    yv[k] = v;
  }
  if constexpr (ROT) {
    // rows of y past the head tile are zero
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const int q = threadIdx.x + k * kThreads;
      if (4 * q < 16 * D) *reinterpret_cast<float4*>(&y[(4 * q) / D][(4 * q) % D]) = yv[k];
    }
    for (int q = threadIdx.x + NQ * kThreads; 4 * q < 16 * D; q += kThreads)
      *reinterpret_cast<float4*>(&y[(4 * q) / D][(4 * q) % D]) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    __syncthreads();
    rotate_store<D>(a, unit, &y[0][0], ro);
  }
}

// ------------------------------------------------------------------------------------------
// A unit covered by one chunk (one work-group) needs no workspace round trip: the work-group
// combines its waves, normalizes, and (ROT) applies lambda_V and the inverse rotation itself.
// ------------------------------------------------------------------------------------------
template <int D, bool ROT, int NSLOT, typename HeadOf>
__device__ __forceinline__ void finish_direct(float (&m_run)[NSLOT], float (&l_run)[NSLOT], v4f (&acc)[D / 16],
                                              HeadOf head_of, const MergeArgs& a, int unit, float* smem) {
  constexpr int NG = D / 16;
  constexpr int NQ = (16 * D / 4 + kThreads - 1) / kThreads;  // float4 quads per thread, at most
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n16 = lane & 15, r4 = lane >> 4;
  const int GT = a.head_tile;
  int b, kvh;
  int64_t orow0;
  unit_coords(a, unit, b, kvh, orow0);
  RotOps<D> ro;
  if constexpr (ROT) rot_prefetch<D>(ro, a, b);
  float4 lam4[NQ];
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    lam4[k] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    const int q = threadIdx.x + k * kThreads;
    const int h = (4 * q) / D, c = 4 * q - h * D;
    if (ROT && a.lambda && h < GT)
      lam4[k] = *reinterpret_cast<const float4*>(a.lambda + b * a.lambda_bs + int64_t(kvh) * D + c);
  }
  // smem: wml[4][16][2] | fw[16][4] | hml[16][2] | wacc[4][GT][D]; y[16][D] reuses it afterwards
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
    hml[2 * h] = ll > 0.0f ? a.acc_scale / ll : 0.0f;
  }
  __syncthreads();
  float4 yv[NQ];
#pragma unroll
  for (int k = 0; k < NQ; ++k) {
    const int q = threadIdx.x + k * kThreads;
    const int h = (4 * q) / D, c = 4 * q - h * D;
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (h < GT) {
      const float4 f = *reinterpret_cast<const float4*>(fw + h * kWaves);
      const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float4 v = *reinterpret_cast<const float4*>(wacc + (ww * GT + h) * D + c);
        s.x = fmaf(v.x, fv[ww], s.x);
        s.y = fmaf(v.y, fv[ww], s.y);
        s.z = fmaf(v.z, fv[ww], s.z);
        s.w = fmaf(v.w, fv[ww], s.w);
      }
      const float li = hml[2 * h];
      s = make_float4(s.x * li * lam4[k].x, s.y * li * lam4[k].y, s.z * li * lam4[k].z, s.w * li * lam4[k].w);
      if constexpr (!ROT) *reinterpret_cast<float4*>(a.out + out_row(a, unit, orow0, h) * D + c) = s;
    }
    yv[k] = s;
  }
  if constexpr (ROT) {
    __syncthreads();
    float(*y)[D] = reinterpret_cast<float(*)[D]>(smem);
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const int q = threadIdx.x + k * kThreads;
      if (q < 16 * D / 4) *reinterpret_cast<float4*>(&y[(4 * q) / D][(4 * q) % D]) = yv[k];
    }
    __syncthreads();
    rotate_store<D>(a, unit, &y[0][0], ro);
  }
}

}  // namespace dec
}  // namespace kvq_impl
