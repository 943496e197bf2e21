// Decode attention over an fp16 KV cache on gfx950: the comparator of the quantized path,
// built the same way so the two differ only in what they read.
//
//   decode_f16_kernel   : one work-group of 4 waves per (sequence, kv head, head tile, chunk).
//     scores : v_mfma_f32_16x16x32_f16 with A = the fp16 query heads and B = the fp16 keys
//              exactly as stored (no conversion), fp32 accumulation;
//     softmax: online per head over 16-lane DPP rows;
//     values : v_mfma_f32_16x16x32_f16 with A = p split into fp16 hi + lo and B = the fp16
//              values read transposed from LDS with ds_read_b64_tr_b16;
//     epilogue: the same chunk partials and last-work-group merge as the quantized path,
//              without rotation.
#include <algorithm>

#include "kvq_decode_common.h"

namespace kvq_impl {
namespace {

using namespace dec;

constexpr int kSB16 = 32;  // tokens per wave superblock

template <int D>
struct FGeom {
  static constexpr int NG = D / 16;
  static constexpr int NSTEP = D / 32;                 // score MFMA steps (32 channels each)
  static constexpr int ROWB = 2 * D;                   // bytes per token
  static constexpr int VLU = kSB16 * ROWB / 16 / 64;  // 16-byte V units per lane per superblock
  static constexpr int LDS_V = kSB16 * ROWB;
  static constexpr int LDS_P = 16 * kSB16 * 4;
  static constexpr int LDS_WAVE = LDS_V + LDS_P + 16 * 4;
  static constexpr int LDS_EPI = (kWaves * 16 * 2 + 16 * kWaves + 32 + kWaves * (D == 128 ? 16 : 8) * D) * 4;
  static constexpr int LDS_M = merge_lds_floats<D>() * 4;
  static constexpr int LDS_A = kWaves * LDS_WAVE > LDS_EPI ? kWaves * LDS_WAVE : LDS_EPI;
  static constexpr int LDS = LDS_A > LDS_M ? LDS_A : LDS_M;
};

template <int D>
__global__ __launch_bounds__(kThreads) void decode_f16_kernel(
    const uint16_t* __restrict__ kx, const uint16_t* __restrict__ vx, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ seq_lens, int seq_len, int kv_heads, int q_heads, int capacity, int head_tile,
    int head_tiles, int chunk, int n_chunks, int max_chunks, float qscale, float* __restrict__ pml,
    float* __restrict__ pacc, uint32_t* __restrict__ counters, const MergeArgs merge) {
  using Gm = FGeom<D>;
  constexpr int NG = Gm::NG, NSTEP = Gm::NSTEP;
  __shared__ __align__(16) uint8_t smem[Gm::LDS];
  __shared__ int last_flag;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n16 = lane & 15, r4 = lane >> 4;
  const int ch = blockIdx.x % n_chunks;
  const int64_t unit = blockIdx.x / n_chunks;
  const int ht = int(unit % head_tiles);
  const int bk = int(unit / head_tiles);
  const int kvh = bk % kv_heads;
  const int b = bk / kv_heads;
  const int G = q_heads / kv_heads;
  const int h0 = kvh * G + ht * head_tile;
  int L = seq_len;
  if (seq_lens) L = min(max(seq_lens[b], 0), seq_len);
  const int t_begin = ch * chunk;
  const int t_end = min(L, t_begin + chunk);

  uint8_t* wbase = smem + w * Gm::LDS_WAVE;
  uint8_t* vtile = wbase;
  float* ptile = reinterpret_cast<float*>(wbase + Gm::LDS_V);
  float* atile = reinterpret_cast<float*>(wbase + Gm::LDS_V + Gm::LDS_P);

  // A operands: query head n16 (zero beyond the tile), channels 32 s + 8 r4 + (0..7)
  v8h aq[NSTEP];
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (n16 < head_tile)
      v = *reinterpret_cast<const uint4*>(q + (int64_t(b) * q_heads + h0 + n16) * D + 32 * s + 8 * r4);
    aq[s] = as_v8h(v.x, v.y, v.z, v.w);
  }
  if (lane < 16) atile[lane] = 1.0f;

  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
  }
  v4f acc[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t rowbase = (int64_t(b) * kv_heads + kvh) * capacity;
  const int last_tok = max(L - 1, 0);

  for (int base = t_begin + w * kSB16; base < t_end; base += kWaves * kSB16) {
    // ---------------- loads ----------------
    uint4 kw[2][NSTEP];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int t = min(base + 16 * sb + n16, last_tok);
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
        kw[sb][s] = *reinterpret_cast<const uint4*>(kx + (rowbase + t) * D + 32 * s + 8 * r4);
    }
    uint4 vw[Gm::VLU];
#pragma unroll
    for (int i = 0; i < Gm::VLU; ++i) {
      const int f = i * 64 + lane;
      const int tl = f / (Gm::ROWB / 16);
      const int piece = f - tl * (Gm::ROWB / 16);
      const int t = base + tl;
      // tokens past the end read as zeros (their p is zero, and 0 * garbage could be NaN)
      vw[i] = t < t_end ? *reinterpret_cast<const uint4*>(vx + (rowbase + t) * D + piece * 8)
                        : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < Gm::VLU; ++i) *reinterpret_cast<uint4*>(vtile + (i * 64 + lane) * 16) = vw[i];

    // ---------------- scores ----------------
    float sc[2][4];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      v4f c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NSTEP; ++s)
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[s], as_v8h(kw[sb][s].x, kw[sb][s].y, kw[sb][s].z, kw[sb][s].w),
                                                    c, 0, 0, 0);
      const bool valid = base + 16 * sb + n16 < t_end;
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[sb][i] = valid ? c[i] * qscale : -INFINITY;
    }

    // ---------------- online softmax: slot i = head 4 r4 + i ----------------
    bool rescale = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mb = row_max16(fmaxf(sc[0][i], sc[1][i]));
      const float mn = fmaxf(m_run[i], mb);
      const float alpha = exp2_guard(m_run[i], mn);
      rescale |= mn != m_run[i];
      m_run[i] = mn;
      const float p0 = exp2_guard(sc[0][i], mn), p1 = exp2_guard(sc[1][i], mn);
      l_run[i] = l_run[i] * alpha + (p0 + p1);
      ptile[(4 * r4 + i) * kSB16 + n16] = p0;
      ptile[(4 * r4 + i) * kSB16 + 16 + n16] = p1;
      if (n16 == 0) atile[4 * r4 + i] = alpha;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (__builtin_amdgcn_ballot_w64(rescale) != 0ull) {
      const float4 al = *reinterpret_cast<const float4*>(atile + 4 * r4);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        acc[g][0] *= al.x;
        acc[g][1] *= al.y;
        acc[g][2] *= al.z;
        acc[g][3] *= al.w;
      }
    }

    // ---------------- A: p of head n16, tokens 8 r4 + (0..7) ----------------
    uint32_t ahi[4], alo[4];
    {
      const float* pr = ptile + n16 * kSB16 + 8 * r4;
      const float4 p0 = *reinterpret_cast<const float4*>(pr);
      const float4 p1 = *reinterpret_cast<const float4*>(pr + 4);
      split_pair(p0.x, p0.y, ahi[0], alo[0]);
      split_pair(p0.z, p0.w, ahi[1], alo[1]);
      split_pair(p1.x, p1.y, ahi[2], alo[2]);
      split_pair(p1.z, p1.w, ahi[3], alo[3]);
    }
    const v8h a_hi = as_v8h(ahi[0], ahi[1], ahi[2], ahi[3]);
    const v8h a_lo = as_v8h(alo[0], alo[1], alo[2], alo[3]);

    // ---------------- values ----------------
    // ds_read_b64_tr_b16: in each 16-lane group, lane (row = l/4, part = l%4) points at 4 halves
    // (columns 4 part .. 4 part + 3) of row `row`; lane c receives column c of the 4 rows.
    const int rrow = n16 >> 2, part = n16 & 3;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      uint32_t bv[4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int tok = 8 * r4 + 4 * half + rrow;
        lds_fp16x4_t* src = (lds_fp16x4_t*)(vtile + tok * Gm::ROWB + 2 * (16 * g + 4 * part));
        const fp16x4_t tr = __builtin_amdgcn_ds_read_tr16_b64_v4f16(src);
        const v2i_t ti = __builtin_bit_cast(v2i_t, tr);
        bv[2 * half] = uint32_t(ti.x);
        bv[2 * half + 1] = uint32_t(ti.y);
      }
      const v8h bop = as_v8h(bv[0], bv[1], bv[2], bv[3]);
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi, bop, acc[g], 0, 0, 0);
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo, bop, acc[g], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  if (n_chunks == 1) {
    finish_direct<D, false, 4>(m_run, l_run, acc, [](int k, int rr) { return 4 * rr + k; }, merge, int(unit),
                               reinterpret_cast<float*>(smem));
    return;
  }
  PartialArgs e;
  e.head_tile = head_tile;
  e.max_chunks = max_chunks;
  e.chunk_index = ch;
  e.unit = unit;
  e.pml = pml;
  e.pacc = pacc;
  store_partial<D, 4>(m_run, l_run, acc, [](int k, int rr) { return 4 * rr + k; }, e,
                      reinterpret_cast<float*>(smem));
  if (!arrive_last(counters + unit, n_chunks, &last_flag)) return;
  merge_unit<D, false>(merge, int(unit), reinterpret_cast<float*>(smem));
}

template <int D>
hipError_t launch_f16(const DecodeF16Args& a, const DecodePlan& p, const WsLayout& w, hipStream_t s) {
  char* ws = static_cast<char*>(a.workspace);
  auto* pml = reinterpret_cast<float*>(ws + w.pml);
  auto* pacc = reinterpret_cast<float*>(ws + w.pacc);
  const int units = a.batch * a.kv_heads * p.head_tiles;
  auto* counters = reinterpret_cast<uint32_t*>(ws + w.counters);
  MergeArgs m{};
  m.pml = pml;
  m.pacc = pacc;
  m.n_chunks = p.n_chunks;
  m.max_chunks = p.max_chunks;
  m.head_tile = p.head_tile;
  m.head_tiles = p.head_tiles;
  m.q_heads = a.q_heads;
  m.kv_heads = a.kv_heads;
  m.gt = p.head_tile;
  m.tok_tile = m.tok_tiles = m.n_query = 1;
  m.acc_scale = 1.0f;
  m.out = a.out;
  hipLaunchKernelGGL((decode_f16_kernel<D>), dim3(units * p.n_chunks), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
                     static_cast<const uint16_t*>(a.q), a.seq_lens, a.seq_len, a.kv_heads, a.q_heads, a.capacity,
                     p.head_tile, p.head_tiles, p.chunk, p.n_chunks, p.max_chunks, a.sm_scale * kLog2e, pml, pacc,
                     counters, m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_f16(const DecodeF16Args& a, const DecodePlan& p, hipStream_t s) {
  const WsLayout w = ws_layout(a.batch * a.kv_heads * p.head_tiles, p.head_tile, a.head_dim, p.max_chunks);
  if (a.head_dim == 128) return launch_f16<128>(a, p, w, s);
  return launch_f16<256>(a, p, w, s);
}

}  // namespace kvq_impl
