// Fused dequant + single-token decode attention over the SRFT-rotated quantized cache (gfx950).
//
// The rotation is orthogonal ("When Quantization Is Free", technical summary, Methodology 1),
// so attention runs in the rotated domain without reconstructing K or V:
//   score_t = (SRFT_sK(q) * lambda_K * sm_scale * log2 e) . (code_K,t * scale_K,t)      [log2 units]
//   out     = s_V * SRFT^-1( lambda_V * sum_t p_t code_V,t * scale_V,t / sum_t p_t )
//
// One launch per call: a work-group of 4 waves per (sequence, kv head, head tile, chunk of
// tokens).
//   prologue: the first superblock's loads go out, then the work-group rotates its query heads
//             (v_mfma_f32_16x16x32_f16, A = the sign-flipped fp16 query, B = 16 Q split into
//             fp16 hi + lo from a constant table in operand order) and splits every rotated
//             channel into a 24-bit integer (three int8 digits, per-head step sigma) laid out as
//             the A operand of the score MFMA.
//   main loop: each wave walks 64-token superblocks:
//     scores : v_mfma_i32_16x16x64_i8.  A rows are (head, group) pairs holding the query digits
//              of one group of 16 channels (block diagonal); B is the packed K codes widened to
//              bytes (x16 for int4: one shift and one mask per 8 codes, no unpacking).  The exact
//              integer group dots are scaled by the fp16 group scales in fp32.
//     softmax: online, per head, over 16-lane DPP rows.
//     values : v_mfma_f32_16x16x32_f16 per group of 16 channels.  The V codes of the superblock
//              are staged in LDS and read with ds_read_b64_tr_b4 so that every lane holds 16
//              tokens of one channel; B = code * scale split exactly into fp16 hi + lo,
//              A = p split into fp16 hi + lo (three products per tile, fp32 accumulation).
//   epilogue: the work-group merges its waves and stores a chunk partial; the last work-group
//             of the unit to finish merges the chunks, applies lambda_V and the inverse rotation
//             and writes the output.  A unit covered by a single chunk skips the workspace.
#pragma once

#include <algorithm>

#include "kvq_decode_common.h"

namespace kvq_impl {
namespace {

using namespace dec;

constexpr int kSB = 64;  // tokens per wave superblock

// Channel held by byte b (0..15) of the widened K codes of one group.
template <int KB>
__host__ __device__ constexpr int kbyte_channel(int b) {
  // int4: dwords hold 16x[c0 c2 c4 c6], 16x[c1 c3 c5 c7], 16x[c8 c10 c12 c14], 16x[c9 ...]
  return KB == 8 ? b : ((b >> 2) & 2 ? 8 : 0) + 2 * (b & 3) + ((b >> 2) & 1);
}

// ------------------------------------------------------------------------------------------
// Main kernel.
// ------------------------------------------------------------------------------------------
constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int D, int KB, int VB>
struct QGeom {
  static constexpr int NS = D / 64;             // score MFMA steps (64 channels each)
  static constexpr int NG = D / 16;             // groups of 16 channels
  static constexpr int KRB = D * KB / 8;        // K code bytes per token
  static constexpr int VRB = D * VB / 8;        // V code bytes per token
  static constexpr int KLB = KRB / 4;           // K code bytes per lane per 16-token block
  static constexpr int KLW = KLB / 4;           // ... in dwords
  static constexpr int VLU = kSB * VRB / 64 / 16;  // 16-byte V units per lane per superblock
  static constexpr int SLW = NG * 2 / 4;        // scale dwords per token
  // LDS (bytes) per wave: V codes, V scales (transposed, k order), K scales, P, alpha
  // int4 V rows are padded by 16 bytes: the transposed reads of one group by the 64 tokens of a
  // superblock (8 bytes each) then spread over 16 bank quads instead of 4 (d 128) or 2 (d 256),
  // and every address stays a per-lane base plus an immediate
  static constexpr int VROW = VB == 4 ? VRB + 16 : VRB;
  static constexpr int LDS_V = kSB * VROW;
  static constexpr int LDS_S = NG * kSB * 2;
  static constexpr int LDS_K = kSB * NG * 2;
  static constexpr int LDS_P = 32 * kSB * 2;  // p as fp16 hi and lo parts, 16 heads each
  static constexpr int LDS_WAVE = LDS_V + LDS_S + LDS_K + LDS_P + 16 * 4;
  static constexpr int LDS_EPI = (kWaves * 16 * 2 + 16 * kWaves + 32 + kWaves * (D == 128 ? 16 : 8) * D) * 4;
  // prologue: digit operands (256 bytes per operand: 4 row blocks x NS steps x 3 digits at most),
  // head maxima, rotation scratch
  static constexpr int DIG_BYTES = 4 * NS * 3 * 256;
  static constexpr int LDS_Q = DIG_BYTES + 256 + 16 * RotGeom<D>::PITCH * 4;
  static constexpr int LDS_M = merge_lds_floats<D>() * 4;
  // append staging: K codes, K scales, V codes, V scales of the new token (16-byte aligned parts)
  static constexpr int APP_KS = KRB, APP_V = KRB + NG * 2, APP_VS = APP_V + VRB, APP_BYTES = APP_VS + NG * 2;
  static constexpr int LDS = cmax(cmax(kWaves * LDS_WAVE, LDS_EPI), cmax(LDS_Q, LDS_M));
};

// Widen the int4 codes of one group (2 dwords, 16 codes) to the 16 int8 bytes 16*code.
__device__ __forceinline__ v4i widen_int4(uint32_t w0, uint32_t w1) {
  return v4i{int((w0 << 4) & 0xf0f0f0f0u), int(w0 & 0xf0f0f0f0u), int((w1 << 4) & 0xf0f0f0f0u),
             int(w1 & 0xf0f0f0f0u)};
}

// 8 nibbles (tokens r = 0..7 of one channel) -> 4 fp16 pairs of code / 16, pairs holding tokens
// (0,4), (1,5), (2,6), (3,7).  After the offset-binary flip (nibble n = code + 8), nibbles 0 and 4
// sit in mantissa bits 0-3 of the two halves (magic 0x6400: 1024 + n) and nibbles 1 and 5 in bits
// 4-7 (1024 + 16 n); one shift by 8 brings nibbles 2, 6 and 3, 7 to the same places.  One packed
// FMA per pair then gives code / 16 exactly: (1024 + n) / 16 - 64.5 and (1024 + 16 n) / 256 - 4.5.
// The masks and the magic come in VGPRs (VOP3 takes no literal here), so each pair costs one
// v_and_or_b32 and one v_pk_fma_f16.
__device__ __forceinline__ void nibbles_to_half16(uint32_t x, uint32_t m_lo, uint32_t m_hi, uint32_t magic,
                                                  uint32_t (&p)[4]) {
  x ^= 0x88888888u;
  const uint32_t y = x >> 8;
  const v2h f_lo = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
  const v2h o_lo = {static_cast<_Float16>(-64.5f), static_cast<_Float16>(-64.5f)};
  const v2h f_hi = {static_cast<_Float16>(0.00390625f), static_cast<_Float16>(0.00390625f)};
  const v2h o_hi = {static_cast<_Float16>(-4.5f), static_cast<_Float16>(-4.5f)};
  const uint32_t t[4] = {(x & m_lo) | magic, (x & m_hi) | magic, (y & m_lo) | magic, (y & m_hi) | magic};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2h c = __builtin_elementwise_fma(__builtin_bit_cast(v2h, t[i]), (i & 1) ? f_hi : f_lo, (i & 1) ? o_hi : o_lo);
    p[i] = __builtin_bit_cast(uint32_t, c);
  }
}

// Global data of one 64-token superblock held in registers (prefetched one superblock ahead).
template <int D, int KB, int VB>
struct SBRegs {
  using Gm = QGeom<D, KB, VB>;
  uint32_t kw[4][Gm::KLW];  // K codes: 16-token block sb, token n16, lane group r4's bytes
  uint32_t ksw[Gm::SLW];    // K scales of token base + lane
  uint4 vw[Gm::VLU];        // V codes, coalesced 16-byte units
  uint32_t vsw[Gm::SLW];    // V scales of token base + lane
};

// Buffer resource over the bytes [p, p + n) (raw buffer, stride 0): loads at offsets >= n
// return 0, so tokens past the sequence end need no clamping.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, 0x00020000);
}

__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, int off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Loads of the superblock whose first token sits at plane slot t0 (wave-uniform); nrem = the
// row's tokens from that one on (loads past them return zero).  The resources start at the superblock, so every lane offset
// is a constant and the address arithmetic is scalar.  Two parts: the K codes (consumed by the
// scores) and the rest (V codes, V scales, K scales: staged in LDS first thing), so that the
// rest of the next superblock can be requested as soon as this one's is staged.
template <int D, int KB, int VB>
__device__ __forceinline__ void load_sb_kcodes(SBRegs<D, KB, VB>& r, const uint8_t* kc, int64_t t0, int nrem, int lane) {
  using Gm = QGeom<D, KB, VB>;
  const int n16 = lane & 15, r4 = lane >> 4;
  const __amdgpu_buffer_rsrc_t rk = row_rsrc(kc + t0 * Gm::KRB, nrem * Gm::KRB);
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
    for (int i = 0; i < Gm::KLW; i += 4) {
      const uint4 v = buf_ld16(rk, (16 * sb + n16) * Gm::KRB + r4 * Gm::KLB + 4 * i);
      r.kw[sb][i] = v.x;
      r.kw[sb][i + 1] = v.y;
      r.kw[sb][i + 2] = v.z;
      r.kw[sb][i + 3] = v.w;
    }
  }
}

template <int D, int KB, int VB>
__device__ __forceinline__ void load_sb_rest(SBRegs<D, KB, VB>& r, const uint16_t* ks, const uint8_t* vc,
                                             const uint16_t* vs, int64_t t0, int nrem, int lane) {
  using Gm = QGeom<D, KB, VB>;
  const __amdgpu_buffer_rsrc_t rks = row_rsrc(ks + t0 * Gm::NG, nrem * Gm::NG * 2);
  const __amdgpu_buffer_rsrc_t rv = row_rsrc(vc + t0 * Gm::VRB, nrem * Gm::VRB);
  const __amdgpu_buffer_rsrc_t rvs = row_rsrc(vs + t0 * Gm::NG, nrem * Gm::NG * 2);
#pragma unroll
  for (int i = 0; i < Gm::SLW; i += 4) {
    const uint4 v = buf_ld16(rks, lane * Gm::NG * 2 + 4 * i);
    r.ksw[i] = v.x;
    r.ksw[i + 1] = v.y;
    r.ksw[i + 2] = v.z;
    r.ksw[i + 3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < Gm::VLU; ++i) r.vw[i] = buf_ld16(rv, (i * 64 + lane) * 16);  // token-major, contiguous
#pragma unroll
  for (int i = 0; i < Gm::SLW; i += 4) {
    const uint4 v = buf_ld16(rvs, lane * Gm::NG * 2 + 4 * i);
    r.vsw[i] = v.x;
    r.vsw[i + 1] = v.y;
    r.vsw[i + 2] = v.z;
    r.vsw[i + 3] = v.w;
  }
}

template <int D, int KB, int VB>
__device__ __forceinline__ void load_superblock(SBRegs<D, KB, VB>& r, const uint8_t* kc, const uint16_t* ks,
                                                const uint8_t* vc, const uint16_t* vs, int64_t t0, int nrem,
                                                int lane) {
  load_sb_kcodes<D, KB, VB>(r, kc, t0, nrem, lane);
  load_sb_rest<D, KB, VB>(r, ks, vc, vs, t0, nrem, lane);
}

// Overwrite, in the registers of a loaded superblock, the token at superblock offset tl
// (wave-uniform) with the new token staged in LDS (app: K codes, K scales, V codes, V scales).
// The lanes holding each part follow load_superblock's layout.
template <int D, int KB, int VB>
__device__ __forceinline__ void patch_superblock(SBRegs<D, KB, VB>& r, int tl, const uint8_t* app, int lane) {
  using Gm = QGeom<D, KB, VB>;
  const int n16 = lane & 15, r4 = lane >> 4;
  const uint32_t* ak = reinterpret_cast<const uint32_t*>(app);
  const uint32_t* aks = reinterpret_cast<const uint32_t*>(app + Gm::APP_KS);
  const uint4* av = reinterpret_cast<const uint4*>(app + Gm::APP_V);
  const uint32_t* avs = reinterpret_cast<const uint32_t*>(app + Gm::APP_VS);
  uint32_t kn[Gm::KLW];
#pragma unroll
  for (int i = 0; i < Gm::KLW; ++i) kn[i] = ak[r4 * Gm::KLW + i];
  // per-lane selects (a uniform branch per block would index the registers dynamically)
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    const bool hit = 16 * sb + n16 == tl;
#pragma unroll
    for (int i = 0; i < Gm::KLW; ++i) r.kw[sb][i] = hit ? kn[i] : r.kw[sb][i];
  }
  const bool sl = lane == tl;
#pragma unroll
  for (int i = 0; i < Gm::SLW; ++i) {
    r.ksw[i] = sl ? aks[i] : r.ksw[i];
    r.vsw[i] = sl ? avs[i] : r.vsw[i];
  }
#pragma unroll
  for (int i = 0; i < Gm::VLU; ++i) {
    const int byte = (i * 64 + lane) * 16;
    if (byte / Gm::VRB == tl) r.vw[i] = av[(byte % Gm::VRB) / 16];
  }
}

// c + a * h, with h the low (HI = 0) or high (HI = 1) fp16 half of h2, in one instruction
// (the conversion of h is exact, so this equals fmaf(a, float(h), c))
template <int HI>
__device__ __forceinline__ float fma_mix_f16(float a, uint32_t h2, float c) {
  float d;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(h2), "v"(c));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(h2), "v"(c));
  return d;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Token (0..15) of a 16-token lane group at position p of the value MFMA's k order (inverse of
// kpos16).
__host__ __device__ constexpr int kinv16(int p) {
  return (p < 8 ? 0 : 8) + ((p & 7) % 2 == 0 ? (p & 7) / 2 : (p & 7) / 2 + 4);
}

// One value MFMA step: acc += P * B for B = code * scale split into fp16 hi + lo.
//   TWO (head tile <= 8): the A rows are (head, part) -- rows 0-7 the hi parts of p of heads 0-7,
//       rows 8-15 the lo parts -- so two products (A b_hi, A b_lo) cover hi*hi, lo*hi, hi*lo (and
//       the negligible lo*lo); the hi and lo rows of a head are added once, at the chunk's end.
//   otherwise the rows are heads: three products (a_hi b_hi, a_hi b_lo, a_lo b_hi).
template <bool TWO>
__device__ __forceinline__ v4f value_mfma(const v8h& a0, const v8h& a1, const v8h& b_hi, const v8h& b_lo, v4f acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b_hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b_lo, acc, 0, 0, 0);
  if constexpr (!TWO) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b_hi, acc, 0, 0, 0);
  return acc;
}

// Value accumulation over int8 V codes staged in LDS (rows swizzled as in the staging).
// ds_read_b64_tr_b8 hands lane c + 8 h of each 16-lane group byte c of the rows that lanes
// 2 j + h supplied, j = 0..7; so lane 2 j + h points at channel half h of group g of the token
// in k slot j, and lane n16 receives channel n16 of the 8 tokens of its k slots.  Bytes become
// fp16 pairs with one v_perm_b32 (exponent byte 0x64 beside each offset-binary code) and one
// packed add; B = code * (staged scale) split exactly into fp16 hi + lo.
template <int D, int KB, int VB, bool TWO>
__device__ __forceinline__ void values_int8(int lane, const v8h (&a0)[2], const v8h (&a1)[2], v4f (&acc)[D / 16],
                                            const uint8_t* vtile, const uint16_t* stile) {
  using Gm = QGeom<D, KB, VB>;
  constexpr int NG = Gm::NG;
  const int n16 = lane & 15, r4 = lane >> 4;
  const int j = n16 >> 1, h = n16 & 1;
  int tok[2];
#pragma unroll
  for (int hblk = 0; hblk < 2; ++hblk) tok[hblk] = 16 * r4 + kinv16(8 * hblk + j);
  const uint32_t expo = 0x64646464u;
  const v2h off = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint4 s0 = *reinterpret_cast<const uint4*>(stile + g * kSB + 16 * r4);
    const uint4 s1 = *reinterpret_cast<const uint4*>(stile + g * kSB + 16 * r4 + 8);
    const uint32_t sp[2][4] = {{s0.x, s0.y, s0.z, s0.w}, {s1.x, s1.y, s1.z, s1.w}};
#pragma unroll
    for (int hblk = 0; hblk < 2; ++hblk) {
      const int tk = tok[hblk];
      lds_v2i_t* src = (lds_v2i_t*)(vtile + tk * Gm::VRB + 16 * (g ^ (tk & 7)) + 8 * h);
      const v2i_t tr = __builtin_amdgcn_ds_read_tr8_b64_v2i32(src);
      const uint32_t w0 = uint32_t(tr.x) ^ 0x80808080u, w1 = uint32_t(tr.y) ^ 0x80808080u;
      const uint32_t raw[4] = {__builtin_amdgcn_perm(expo, w0, 0x04010400u), __builtin_amdgcn_perm(expo, w0, 0x04030402u),
                               __builtin_amdgcn_perm(expo, w1, 0x04010400u), __builtin_amdgcn_perm(expo, w1, 0x04030402u)};
      uint32_t bh[4], bl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v2h c = __builtin_bit_cast(v2h, raw[i]) + off;  // 1024 + code + 128 - 1152
        const v2h sc2 = __builtin_bit_cast(v2h, sp[hblk][i]);
        const v2h hi = c * sc2;
        const v2h lo = __builtin_elementwise_fma(c, sc2, -hi);
        bh[i] = __builtin_bit_cast(uint32_t, hi);
        bl[i] = __builtin_bit_cast(uint32_t, lo);
      }
      acc[g] = value_mfma<TWO>(a0[hblk], a1[hblk], as_v8h(bh[0], bh[1], bh[2], bh[3]), as_v8h(bl[0], bl[1], bl[2], bl[3]),
                               acc[g]);
    }
  }
}

// Sum over the four 16-lane rows for every lane position (v_permlane32_swap, v_permlane16_swap).
__device__ __forceinline__ float rows_sum4(float a) {
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  a = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
}

// 65536 hi + 256 mid + lo of three exact int32 digit dots, as two v_lshl_add_u32 (the empty asm
// keeps the compiler from reassociating it into two shifts and an add3)
__device__ __forceinline__ int digit_dot(int hi, int mid, int lo) {
  uint32_t t = (uint32_t(hi) << 8) + uint32_t(mid);
  asm volatile("" : "+v"(t));
  return int((t << 8) + uint32_t(lo));
}

// Everything one wave does with one superblock already in registers.
//   aop: score MFMA A operands.  G1 (head tile 1): one operand per step s whose rows are
//        (group slot, digit): the three digits of the query, so one MFMA gives every digit's dot
//        of four groups and the lanes of a slot combine them.  Otherwise aop[rb][s][digit] with
//        rows (head, group slot).
//   ptile: p of the superblock as fp16 hi and lo parts, row part * 16 + head, 64 tokens in the
//        value MFMA's k order.
template <int D, int KB, int VB, int NRB, bool G1>
__device__ __forceinline__ void process_superblock(SBRegs<D, KB, VB>& r, int base, int t_end, int lane,
                                                   const v4i (&aop)[G1 ? 1 : NRB][D / 64][G1 ? 1 : 3],
                                                   const float (&sig)[NRB], const int (&rlo)[NRB], const int (&rhi)[NRB],
                                                   int lo_max, int hi_min, float (&m_run)[NRB], float (&l_run)[NRB],
                                                   v4f (&acc)[D / 16], uint8_t* vtile, uint16_t* stile,
                                                   uint16_t* ktile, uint16_t* ptile, float* atile,
                                                   const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks,
                                                   const uint8_t* __restrict__ vc, const uint16_t* __restrict__ vs,
                                                   int next_base, int64_t next_t0, int next_nrem) {
  using Gm = QGeom<D, KB, VB>;
  constexpr int NS = Gm::NS, NG = Gm::NG;
  constexpr bool TWO = NRB <= 2;
  const int n16 = lane & 15, r4 = lane >> 4;

  // ---------------- stage V codes, V scales (k order) and K scales in LDS ----------------
  bool vbig = false;
  if constexpr (VB == 8) {
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < Gm::SLW; ++i) mx = max(mx, max(r.vsw[i] & 0x7fffu, (r.vsw[i] >> 16) & 0x7fffu));
    vbig = __builtin_amdgcn_ballot_w64(mx > 0x6000u) != 0ull;  // 0x6000 = 512 in fp16
  }
#pragma unroll
  for (int i = 0; i < Gm::VLU; ++i) {
    const int u = i * 64 + lane;  // 16-byte unit of the superblock, token-major
    if constexpr (VB == 4) {
      constexpr int UPT = Gm::VRB / 16;
      const int tk = u / UPT, k = u % UPT;
      *reinterpret_cast<uint4*>(vtile + tk * Gm::VROW + 16 * k) = r.vw[i];
    } else {
      // int8: unit k (group k) of token t goes to slot k ^ (t & 7) of the token's row, so that
      // the transposed reads of 8 tokens of one group hit 8 different bank quads
      constexpr int UPT = Gm::VRB / 16;
      const int tk = u / UPT, k = u % UPT;
      *reinterpret_cast<uint4*>(vtile + tk * Gm::VRB + 16 * (k ^ (tk & 7))) = r.vw[i];
    }
  }
  {
    // V scales, transposed to [group][k order].  int4: the scale as stored (the codes come out of
    // the conversion as code / 16, which keeps code * scale inside the fp16 range; the merge undoes
    // the 1/16).  int8: the scale as it is (scales of calibrated values are small, and a
    // pre-factor would push them into fp16 subnormals), unless a scale of this superblock exceeds
    // 512, where code * scale could overflow: then B takes scale / 128 and A takes p * 128.  No
    // mask is needed: a superblock never crosses a chunk end (chunks are whole multiples of the
    // work-group stride), so its tokens past t_end are past the row end, where the loads returned
    // zero.  (The int8 factor stays in float: a packed-half multiply here was miscompiled, both
    // halves stored from the low-half product.)
    const int pos = 16 * (lane >> 4) + kpos16(lane & 15);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint32_t bits = (r.vsw[g >> 1] >> (16 * (g & 1))) & 0xffffu;
      if constexpr (VB == 4) {
        stile[g * kSB + pos] = uint16_t(bits);
      } else {
        const float sv = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(bits))) * (vbig ? 0.0078125f : 1.0f);
        stile[g * kSB + pos] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(sv));
      }
    }
    uint32_t* kt = reinterpret_cast<uint32_t*>(ktile + lane * NG);
#pragma unroll
    for (int i = 0; i < Gm::SLW; i += 4)
      *reinterpret_cast<uint4*>(kt + i) = make_uint4(r.ksw[i], r.ksw[i + 1], r.ksw[i + 2], r.ksw[i + 3]);
  }
  // the staged parts of the next superblock load during this one's scores, softmax and values
  if (next_base < t_end) load_sb_rest<D, KB, VB>(r, ks, vc, vs, next_t0, next_nrem, lane);
  wave_sync_lds();

  // ---------------- scores (int8 MFMA, exact integer group dots) ----------------
  // A group dot of the 21-bit (int8 keys: 20-bit) query digits, hi * 65536 + mid * 256 + lo, is
  // exact in int32 (|hi| <= 16, or 8; 16 channels of codes up to 112 = 16 * 7, or 127).
  // wave-uniform: only the chunk's last superblock and those at a row's causal end or window start
  // hold masked tokens
  const bool tail = base + kSB > min(t_end, hi_min) || base < lo_max;
  float sc[4][NRB];
#pragma unroll
  for (int sb = 0; sb < 4; ++sb) {
    v4i bop[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (KB == 4)
        bop[s] = widen_int4(r.kw[sb][2 * s], r.kw[sb][2 * s + 1]);
      else
        bop[s] = v4i{int(r.kw[sb][4 * s]), int(r.kw[sb][4 * s + 1]), int(r.kw[sb][4 * s + 2]),
                     int(r.kw[sb][4 * s + 3])};
    }
    const v4i zero = {0, 0, 0, 0};
    if constexpr (G1) {
      // lane (token n16, slot r4): the scales of groups r4 * NS + s, s = 0..NS-1, are adjacent
      const uint16_t* kt = ktile + (16 * sb + n16) * NG + r4 * NS;
      uint32_t kr[(NS + 1) / 2];
      if constexpr (NS == 2) {
        kr[0] = *reinterpret_cast<const uint32_t*>(kt);
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(kt);
        kr[0] = v.x;
        kr[1] = v.y;
      }
      float s_acc = 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const v4i c = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[0][s][0], bop[s], zero, 0, 0, 0);
        const int dot = digit_dot(c[0], c[1], c[2]);
        s_acc = (s & 1) ? fma_mix_f16<1>(static_cast<float>(dot), kr[s >> 1], s_acc)
                        : fma_mix_f16<0>(static_cast<float>(dot), kr[s >> 1], s_acc);
      }
      s_acc = rows_sum4(s_acc) * sig[0];
      const int tok = base + 16 * sb + n16;
      sc[sb][0] = (tail && (tok >= t_end || tok < rlo[0] || tok >= rhi[0])) ? -INFINITY : s_acc;
    } else {
      uint32_t kraw[Gm::SLW];
      {
        const uint32_t* kt = reinterpret_cast<const uint32_t*>(ktile + (16 * sb + n16) * NG);
#pragma unroll
        for (int i = 0; i < Gm::SLW; i += 4) {
          const uint4 v = *reinterpret_cast<const uint4*>(kt + i);
          kraw[i] = v.x;
          kraw[i + 1] = v.y;
          kraw[i + 2] = v.z;
          kraw[i + 3] = v.w;
        }
      }
      // the fp16 group scales stay packed; the FMA takes them as fp16 operands (v_fma_mix_f32)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        float s_acc = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const v4i chi = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[rb][s][0], bop[s], zero, 0, 0, 0);
          const v4i cmi = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[rb][s][1], bop[s], zero, 0, 0, 0);
          const v4i clo = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[rb][s][2], bop[s], zero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int dot = digit_dot(chi[i], cmi[i], clo[i]);
            const int gi = i * NS + s;
            s_acc = (gi & 1) ? fma_mix_f16<1>(static_cast<float>(dot), kraw[gi >> 1], s_acc)
                             : fma_mix_f16<0>(static_cast<float>(dot), kraw[gi >> 1], s_acc);
          }
        }
        s_acc *= sig[rb];
        const int tok = base + 16 * sb + n16;
        sc[sb][rb] = (tail && (tok >= t_end || tok < rlo[rb] || tok >= rhi[rb])) ? -INFINITY : s_acc;
      }
    }
  }

  // the K codes of this superblock are consumed: the next one's load during softmax + values
  if (next_base < t_end) load_sb_kcodes<D, KB, VB>(r, kc, next_t0, next_nrem, lane);

  // ---------------- online softmax per head (16-lane rows); p as fp16 hi + lo in LDS ----------------
  // A row whose tokens so far are all masked keeps m = -inf; the exponent's reference is then 0, so
  // exp2(-inf - 0) = 0 and no NaN arises.
  bool rescale = false;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    float mb = fmaxf(fmaxf(sc[0][rb], sc[1][rb]), fmaxf(sc[2][rb], sc[3][rb]));
    mb = row_max16(mb);
    const float mn = fmaxf(m_run[rb], mb);
    const float mref = mn == -INFINITY ? 0.0f : mn;
    const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - mref);
    rescale |= mn != m_run[rb];
    m_run[rb] = mn;
    float p[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) p[sb] = __builtin_amdgcn_exp2f(sc[sb][rb] - mref);
    l_run[rb] = l_run[rb] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    const int head = 4 * rb + r4;
    uint16_t* prow = ptile + head * kSB + kpos16(n16);
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const auto hi = __builtin_amdgcn_cvt_pkrtz(p[2 * q2], p[2 * q2 + 1]);
      const auto lo = __builtin_amdgcn_cvt_pkrtz(p[2 * q2] - static_cast<float>(hi[0]),
                                                 p[2 * q2 + 1] - static_cast<float>(hi[1]));
      const uint32_t hb = __builtin_bit_cast(uint32_t, hi), lb = __builtin_bit_cast(uint32_t, lo);
      prow[16 * (2 * q2)] = uint16_t(hb);
      prow[16 * (2 * q2 + 1)] = uint16_t(hb >> 16);
      prow[16 * kSB + 16 * (2 * q2)] = uint16_t(lb);
      prow[16 * kSB + 16 * (2 * q2 + 1)] = uint16_t(lb >> 16);
    }
    if (n16 == 0) atile[head] = alpha;
  }
  wave_sync_lds();
  if (__builtin_amdgcn_ballot_w64(rescale) != 0ull) {
    // acc rows: heads 4 r4 + i, or with TWO (head, part) rows, heads 4 (r4 & 1) + i
    const float4 al = *reinterpret_cast<const float4*>(atile + 4 * (TWO ? (r4 & 1) : r4));
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      acc[g][0] *= al.x;
      acc[g][1] *= al.y;
      acc[g][2] *= al.z;
      acc[g][3] *= al.w;
    }
  }

  // ---------------- A operands from the staged p parts, tokens 16 r4 + (0..15) ----------------
  v8h a0[2], a1[2];
  {
    const int row0 = TWO ? (n16 >> 3) * 16 + (n16 & 7) : n16;
#pragma unroll
    for (int hblk = 0; hblk < 2; ++hblk) {
      const uint4 x = *reinterpret_cast<const uint4*>(ptile + row0 * kSB + 16 * r4 + 8 * hblk);
      a0[hblk] = as_v8h(x.x, x.y, x.z, x.w);
      if constexpr (!TWO) {
        const uint4 y = *reinterpret_cast<const uint4*>(ptile + (16 + n16) * kSB + 16 * r4 + 8 * hblk);
        a1[hblk] = as_v8h(y.x, y.y, y.z, y.w);
      } else {
        a1[hblk] = a0[hblk];
      }
    }
    if constexpr (VB == 8) {
      if (vbig) {
        const v8h k128 = {static_cast<_Float16>(128.0f), static_cast<_Float16>(128.0f), static_cast<_Float16>(128.0f),
                          static_cast<_Float16>(128.0f), static_cast<_Float16>(128.0f), static_cast<_Float16>(128.0f),
                          static_cast<_Float16>(128.0f), static_cast<_Float16>(128.0f)};
#pragma unroll
        for (int hblk = 0; hblk < 2; ++hblk) {
          a0[hblk] *= k128;
          a1[hblk] *= k128;
        }
      }
    }
  }

  // ---------------- values (fp16 MFMA over LDS-transposed codes) ----------------
  if constexpr (VB == 8) {
    values_int8<D, KB, VB, TWO>(lane, a0, a1, acc, vtile, stile);
    wave_sync_lds();
    return;
  }
  uint32_t m_lo = 0x000f000fu, m_hi = 0x00f000f0u, nmagic = 0x64006400u;
  asm volatile("" : "+v"(m_lo), "+v"(m_hi), "+v"(nmagic));
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    // lane r of each 16-lane group points at token 16*r4 + r, group g
    lds_v2i_t* src = (lds_v2i_t*)(vtile + (16 * r4 + n16) * Gm::VROW + 8 * g);
    const v2i_t tr = __builtin_amdgcn_ds_read_tr4_b64_v2i32(src);
    const uint4 s0 = *reinterpret_cast<const uint4*>(stile + g * kSB + 16 * r4);
    const uint4 s1 = *reinterpret_cast<const uint4*>(stile + g * kSB + 16 * r4 + 8);
    const uint32_t sp[2][4] = {{s0.x, s0.y, s0.z, s0.w}, {s1.x, s1.y, s1.z, s1.w}};
#pragma unroll
    for (int hblk = 0; hblk < 2; ++hblk) {
      uint32_t cp[4];
      nibbles_to_half16(uint32_t(hblk == 0 ? tr.x : tr.y), m_lo, m_hi, nmagic, cp);
      uint32_t bh[4], bl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v2h c = __builtin_bit_cast(v2h, cp[i]);
        const v2h sc2 = __builtin_bit_cast(v2h, sp[hblk][i]);
        const v2h hi = c * sc2;
        const v2h lo = __builtin_elementwise_fma(c, sc2, -hi);
        bh[i] = __builtin_bit_cast(uint32_t, hi);
        bl[i] = __builtin_bit_cast(uint32_t, lo);
      }
      acc[g] = value_mfma<TWO>(a0[hblk], a1[hblk], as_v8h(bh[0], bh[1], bh[2], bh[3]), as_v8h(bl[0], bl[1], bl[2], bl[3]),
                               acc[g]);
    }
  }
  // the next superblock overwrites this wave's tiles
  wave_sync_lds();
}

struct QDecodeParams {
  const uint8_t* kc;
  const uint16_t* ks;
  const uint8_t* vc;
  const uint16_t* vs;
  const int32_t* seq_lens;
  int seq_len, kv_heads, q_heads, capacity;
  int head_tile, head_tiles, chunk, n_chunks, max_chunks;
  const uint16_t* q;
  const float* sign_k;
  const float* lambda_k;
  int64_t sign_bs, lambda_bs;
  float score_scale;  // sm_scale * log2 e
  uint32_t* counters;
  float* pml;
  float* pacc;
  MergeArgs merge;
  // append (k_new == nullptr: none): the new K and V vectors [batch, kv_heads, D] of every
  // row, quantized into position L - 1 of the planes by the work-group holding that position
  const uint16_t* k_new;
  const uint16_t* v_new;
  // paged cache (page_table == nullptr: contiguous rows of `capacity` tokens): token t of
  // sequence b sits at slot (page * kv_heads + kv head) * page_size + t % page_size of the
  // planes, page = page_table[b * pages_per_seq + t / page_size] clamped to [0, num_pages)
  const int32_t* page_table;
  int page_size, pages_per_seq, num_pages;
  // rows of a unit: tok_tile query tokens x head_tile heads; query i of a sequence of length L
  // sits at position L - n_query + i and attends positions [max(0, p - window + 1) if window,
  // else 0; p]; ring: token t at plane position t % capacity
  int tok_tile, tok_tiles, rows, n_query, window, ring;
};

// APP: the appending variant (kvq_decode_attn_append), a separate instance so that the plain
// decode carries none of its code.  G1: the head tile is one query head (the score MFMA rows carry
// the query's three digits instead of heads).
template <int D, int KB, int VB, int NRB, bool APP, bool G1>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : 1))) void decode_kernel(
    const QDecodeParams P) {
  using Gm = QGeom<D, KB, VB>;
  constexpr int NS = Gm::NS, NG = Gm::NG;
  constexpr int NBW = D / 16 / kWaves;
  __shared__ __align__(16) uint8_t smem[Gm::LDS];
  __shared__ int last_flag;
  __shared__ __align__(16) uint8_t appbuf[Gm::APP_BYTES];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index (uniform)
  const int n16 = lane & 15, r4 = lane >> 4;
  const int ch = blockIdx.x % P.n_chunks;
  const int unit = blockIdx.x / P.n_chunks;
  const int tti = unit % P.tok_tiles;
  const int hu = unit / P.tok_tiles;
  const int ht = hu % P.head_tiles;
  const int bk = hu / P.head_tiles;
  const int kvh = bk % P.kv_heads;
  const int b = bk / P.kv_heads;
  const int GT = P.head_tile;  // query heads of the unit
  const int ROWS = P.rows;     // rows: query tokens x heads
  const int h0 = kvh * (P.q_heads / P.kv_heads) + ht * GT;
  int L = P.seq_len;
  if (P.seq_lens) L = min(max(P.seq_lens[b], 0), P.seq_len);
  // the unit's query tokens i0 .. i_last sit at positions L - n_query + i; it attends from the
  // window start of its first query (aligned down to a superblock) to its last query's position
  const int i0 = tti * P.tok_tile;
  const int i_last = min(i0 + P.tok_tile, P.n_query) - 1;
  const int p0 = L - P.n_query + i0, p_last = L - P.n_query + i_last;
  const int u_end = max(p_last + 1, 0);
  const int u_start = P.window > 0 ? max(p0 + 1 - P.window, 0) : 0;
  const int t_begin = (u_start / kSB) * kSB + ch * P.chunk;
  const int t_end = min(u_end, t_begin + P.chunk);
  // tokens that some row of the unit masks: below lo_max or from hi_min on (wave-uniform)
  const int hi_min = max(p0 + 1, 0);
  const int lo_max = P.window > 0 ? max(p_last + 1 - P.window, 0) : 0;
  const int64_t rowbase = (int64_t(b) * P.kv_heads + kvh) * P.capacity;
  // not restrict: an appending call writes one token of these planes
  const uint8_t* kc = P.kc;
  const uint16_t* ks = P.ks;
  const uint8_t* vc = P.vc;
  const uint16_t* vs = P.vs;
  constexpr int kStride = kWaves * kSB;

  // Paged cache: lane k of this wave holds the page of the wave's superblock k (token
  // t_begin + 64 w + 256 k; a superblock never straddles a page since page_size is a multiple
  // of 64).  Issued first, so the first superblock's address waits only for this load.  Entries
  // past the row's tokens read a valid entry and are not used; pages are clamped to the planes.
  const bool paged = P.page_table != nullptr;
  int pg_v = 0, po_v = 0;  // lane k: page of superblock k and its first token's offset in the page
  if (paged) {
    int tb = min(t_begin + w * kSB + lane * kStride, max(L - 1, 0));
    if (P.ring) tb %= P.capacity;
    const int e = min(tb / P.page_size, P.pages_per_seq - 1);
    pg_v = min(max(P.page_table[int64_t(b) * P.pages_per_seq + e], 0), P.num_pages - 1);
    po_v = tb - e * P.page_size;
  }
  // plane slot of superblock k of this wave from its row position ls (the first token's position,
  // taken modulo the capacity in a ring; a multiple of 64, and a ring's capacity is a multiple of
  // 64, so a superblock never wraps).  The position advances by the wave stride per superblock:
  // by one compare and subtract in a ring (step_ring = stride % capacity), no division per step.
  auto sb_slot = [&](int ls, int k) -> int64_t {
    if (!paged) return rowbase + ls;
    const int kk = min(k, 63);
    const int pg = __builtin_amdgcn_readlane(pg_v, kk);
    return (int64_t(pg) * P.kv_heads + kvh) * P.page_size + __builtin_amdgcn_readlane(po_v, kk);
  };
  const int step_ring = P.ring ? kWaves * kSB % P.capacity : 0;
  auto next_pos = [&](int ls) -> int {
    if (!P.ring) return ls + kWaves * kSB;
    const int n = ls + step_ring;
    return n >= P.capacity ? n - P.capacity : n;
  };

  // ---------------- prologue: rotated query -> int8 digit operands ----------------
  // Its few loads go out first (loads complete in issue order), then the first superblock's.
  // Rows of the rotation: row n = (query token i0 + n / GT, head h0 + n % GT); an appending
  // work-group (the one holding position L - 1 of its row; the head tile is then at most 14)
  // also rotates the new K vector as row 14 (signs s_K) and the new V vector as row 15 (s_V).
  // Every load is unconditional per row (a null lambda reads valid memory whose value is then
  // discarded), so that all of them are in flight together.
  const int t_app = L - 1;
  const bool app = APP && t_app >= t_begin && t_app < t_end;  // work-group uniform
  const float* srow_k = P.sign_k + b * P.sign_bs;
  const float* srow_v = P.merge.sign + b * P.sign_bs;
  FwdIn<D> fin;
  fwd_load<D>(fin, P.merge.transform, srow_k, app ? srow_v : nullptr, [&](int n, const uint16_t*& x) -> bool {
    if (app && n >= 14) {
      x = (n == 14 ? P.k_new : P.v_new) + (int64_t(b) * P.kv_heads + kvh) * D;
      return true;
    }
    const int qr = min(n, ROWS - 1);
    const int qi = min(i0 + qr / GT, P.n_query - 1);
    x = P.q + ((int64_t(b) * P.n_query + qi) * P.q_heads + h0 + qr % GT) * D;
    return n < ROWS && i0 + n / GT < P.n_query;
  });
  RotTw<D> rtw;
  load_rot_tw<D, false>(rtw);
  // lambda_K of the channels this lane's query values take: c = 16 (w + 4 j) + kbyte_channel(n16),
  // so that the four lanes of a quad hold the four bytes of one dword of the score operand
  // (1 where absent); the append decision takes channel 16 (w + 4 j) + n16 of both lambdas
  const int64_t lofs = b * P.lambda_bs + int64_t(kvh) * D;
  const float* lkrow = P.lambda_k ? P.lambda_k + lofs : srow_k;
  const float* lvrow = P.merge.lambda ? P.merge.lambda + lofs : srow_k;
  const int qch = kbyte_channel<KB>(n16);
  float nlk[NBW], alk[NBW], alv[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    nlk[j] = lkrow[16 * (w + kWaves * j) + qch];
    if constexpr (APP) {
      alk[j] = lkrow[16 * (w + kWaves * j) + n16];
      alv[j] = lvrow[16 * (w + kWaves * j) + n16];
    }
  }

  SBRegs<D, KB, VB> ra;
  int base = t_begin + w * kSB;
  int pos = P.ring ? base % P.capacity : base;  // row position of this wave's superblock
  if (base < t_end) load_superblock<D, KB, VB>(ra, kc, ks, vc, vs, sb_slot(pos, 0), min(L - base, kSB), lane);

  // LDS of the prologue (aliases the main-loop tiles): digit operands, per-wave head maxima, and
  // the rotated rows
  constexpr int kDigBytes = Gm::DIG_BYTES;
  uint32_t* dig = reinterpret_cast<uint32_t*>(smem);
  float* pmax = reinterpret_cast<float*>(smem + kDigBytes);  // [kWaves][16]
  float* qo = reinterpret_cast<float*>(smem + kDigBytes + 256);  // [16][PITCH] rotated rows
  float lam[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    nlk[j] = P.lambda_k ? nlk[j] : 1.0f;
    lam[j] = nlk[j] * P.score_scale;
    if constexpr (APP) {
      alk[j] = P.lambda_k ? alk[j] : 1.0f;
      alv[j] = P.merge.lambda ? alv[j] : 1.0f;
    }
  }
  fwd_wave<D>(fin, rtw, P.merge.transform, qo);
  __syncthreads();
  constexpr int QP = RotGeom<D>::PITCH;
  // q_hat[h][c] * lambda_c * score_scale for the heads h = r4 + 4 i (i < NRB: the row blocks of
  // the score operands) and channel c = 16 (w + 4j) + qch
  float qv_[NBW][NRB];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int g = w + kWaves * j;
#pragma unroll
    for (int i = 0; i < NRB; ++i) qv_[j][i] = qo[(r4 + 4 * i) * QP + 16 * g + qch] * lam[j];
    if (app) {
      // the write path on rows 14 (K) and 15 (V), lanes 48..63, channel c = 16 g + n16:
      // u = SRFT(x)_c / lambda_c, group absmax over the row's 16 lanes, fp16 scale, rounded
      // codes, packed into the LDS staging of the new token
      const float uk = qo[14 * QP + 16 * g + n16] * __builtin_amdgcn_rcpf(alk[j]);
      const float uv = qo[15 * QP + 16 * g + n16] * __builtin_amdgcn_rcpf(alv[j]);
      const _Float16 shk = static_cast<_Float16>(scale_of<KB>(row_max16(fabsf(uk))));
      const _Float16 shv = static_cast<_Float16>(scale_of<VB>(row_max16(fabsf(uv))));
      const float sfk = static_cast<float>(shk), sfv = static_cast<float>(shv);
      const uint32_t ck = code_byte<KB>(uk, sfk > 0.0f ? __builtin_amdgcn_rcpf(sfk) : 0.0f);
      const uint32_t cv = code_byte<VB>(uv, sfv > 0.0f ? __builtin_amdgcn_rcpf(sfv) : 0.0f);
      // int4: two's-complement nibbles, the even channel low (odd partner n16 ^ 1 by DPP)
      const uint32_t nk = (ck ^ 8u) & 0xfu, nvv = (cv ^ 8u) & 0xfu;
      const uint32_t pk = uint32_t(__builtin_amdgcn_mov_dpp(int(nk), 0xB1, 0xf, 0xf, false));
      const uint32_t pv = uint32_t(__builtin_amdgcn_mov_dpp(int(nvv), 0xB1, 0xf, 0xf, false));
      if (r4 == 3) {
        if constexpr (KB == 8)
          appbuf[16 * g + n16] = uint8_t(ck ^ 0x80u);
        else if ((n16 & 1) == 0)
          appbuf[8 * g + n16 / 2] = uint8_t(nk | (pk << 4));
        if constexpr (VB == 8)
          appbuf[Gm::APP_V + 16 * g + n16] = uint8_t(cv ^ 0x80u);
        else if ((n16 & 1) == 0)
          appbuf[Gm::APP_V + 8 * g + n16 / 2] = uint8_t(nvv | (pv << 4));
        if (n16 == 0) {
          reinterpret_cast<uint16_t*>(appbuf + Gm::APP_KS)[g] = __builtin_bit_cast(uint16_t, shk);
          reinterpret_cast<uint16_t*>(appbuf + Gm::APP_VS)[g] = __builtin_bit_cast(uint16_t, shv);
        }
      }
    }
  }
  // per-head maximum of |q_hat| over this wave's channels (16-lane DPP rows), then over waves
#pragma unroll
  for (int i = 0; i < NRB; ++i) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < NBW; ++j) m = fmaxf(m, fabsf(qv_[j][i]));
    m = row_max16(m);
    if (n16 == 0) pmax[w * 16 + r4 + 4 * i] = m;
  }
  __syncthreads();
  if (app && ht == 0) {
    // the new token leaves for the planes (every head tile patches its own registers)
    constexpr int UK = Gm::KRB / 16, US = NG * 2 / 16, UV = Gm::VRB / 16;
    const int tid = threadIdx.x;
    int64_t slot = rowbase + t_app;
    if (paged) {
      const int e = min(t_app / P.page_size, P.pages_per_seq - 1);
      const int pg = min(max(P.page_table[int64_t(b) * P.pages_per_seq + e], 0), P.num_pages - 1);
      slot = (int64_t(pg) * P.kv_heads + kvh) * P.page_size + t_app % P.page_size;
    }
    if (tid < UK) {
      *reinterpret_cast<uint4*>(const_cast<uint8_t*>(kc) + slot * Gm::KRB + 16 * tid) =
          *reinterpret_cast<const uint4*>(appbuf + 16 * tid);
    } else if (tid < UK + US) {
      const int u = tid - UK;
      *reinterpret_cast<uint4*>(const_cast<uint16_t*>(ks) + slot * NG + 8 * u) =
          *reinterpret_cast<const uint4*>(appbuf + Gm::APP_KS + 16 * u);
    } else if (tid < UK + US + UV) {
      const int u = tid - UK - US;
      *reinterpret_cast<uint4*>(const_cast<uint8_t*>(vc) + slot * Gm::VRB + 16 * u) =
          *reinterpret_cast<const uint4*>(appbuf + Gm::APP_V + 16 * u);
    } else if (tid < UK + 2 * US + UV) {
      const int u = tid - UK - US - UV;
      *reinterpret_cast<uint4*>(const_cast<uint16_t*>(vs) + slot * NG + 8 * u) =
          *reinterpret_cast<const uint4*>(appbuf + Gm::APP_VS + 16 * u);
    }
  }
  // per-head step: the largest |q_hat| maps to QTOT = 2^20 (int8 keys: 2^19), so the digits
  // hi, mid, lo of Q = 65536 hi + 256 mid + lo fit int8 with |hi| <= 16 (8) and a group dot of Q
  // with 16 codes stays exact in int32 (two 8-bit digits, 16 bits relative to the largest
  // channel, left score errors up to ~1e-2 when lambda_K spans a decade and keys exceed the
  // calibration range)
  constexpr float QTOT = KB == 4 ? 1048576.0f : 524288.0f;
  // step of head r4 + 4 i (the heads of this lane's query values)
  float sgm[NRB];
#pragma unroll
  for (int i = 0; i < NRB; ++i) {
    float mxh = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) mxh = fmaxf(mxh, pmax[ww * 16 + r4 + 4 * i]);
    sgm[i] = mxh > 0.0f ? mxh / QTOT : 1.0f;
  }
  // score multiplier of the rows this lane's scores belong to: heads 4 rb + r4 (G1: head 0 in
  // every lane)
  float sig[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int hr = G1 ? 0 : 4 * rb + r4;
    float mxh = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) mxh = fmaxf(mxh, pmax[ww * 16 + hr]);
    const float sg = mxh > 0.0f ? mxh / QTOT : 1.0f;
    // step of the exact dot of Q, times 1/16 for int4 codes widened as 16 * code
    sig[rb] = (hr < ROWS ? sg : 0.0f) * (KB == 4 ? 0.0625f : 1.0f);
  }
  // positions the rows of this lane's scores attend, [rlo, rhi) (rows past the unit's query
  // tokens and phantom rows: unmasked, their results are never stored)
  int rlo[NRB], rhi[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int hr = G1 ? 0 : 4 * rb + r4;
    const int qt = i0 + hr / GT;
    const bool real = hr < ROWS && qt < P.n_query;
    const int pr = L - P.n_query + qt;
    rhi[rb] = real ? max(pr + 1, 0) : 0x7fffffff;
    rlo[rb] = real && P.window > 0 ? max(pr + 1 - P.window, 0) : 0;
  }
  // the three int8 digits of every channel (Q = 65536 hi + 256 mid + lo) as the score MFMA's A
  // operands.  For (row block rb, step s, digit dg) lane l holds row r = l%16 = (head 4rb + r/4,
  // slot r%4) and the k bytes of lane group l/16; it is non-zero only when l/16 == r%4, where the
  // 16 bytes are the digits of group g = (r%4) NS + s in the byte order of the widened K codes.
  // G1: one operand per step s, row r = 4 slot + digit (row 4 slot + 3 zero), non-zero where
  // l/16 == slot.  Only the non-zero lanes' 16 bytes are staged: 256 bytes per operand, at
  // (4 slot + head in block) * 16 (G1: (4 slot + digit) * 16).  The lanes of a quad hold the
  // four bytes of one dword (channel kbyte_channel(n16)); two DPP swaps assemble it.  Lane (n16,
  // r4) holds head r4 + 4 i of row block i.
  {
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int g = w + kWaves * j;
      const int slot = g / NS, s = g % NS;
#pragma unroll
      for (int i = 0; i < NRB; ++i) {
        const int h = r4 + 4 * i;
        constexpr int QI = int(QTOT);
        int Q = static_cast<int>(rintf(qv_[j][i] * (1.0f / sgm[i])));
        Q = min(max(Q, -QI), QI);
        const int t1 = (Q + 128) >> 8;  // in [-QI / 256, QI / 256]
        const int lo = Q - 256 * t1;     // in [-128, 127]
        const int hi = (t1 + 128) >> 8;  // in [-16, 16] (int8 keys: [-8, 8])
        const int mid = t1 - 256 * hi;   // in [-128, 127]
        const int sh = 8 * (n16 & 3);
        uint32_t dw[3] = {uint32_t(hi & 0xff) << sh, uint32_t(mid & 0xff) << sh, uint32_t(lo & 0xff) << sh};
#pragma unroll
        for (int dg = 0; dg < 3; ++dg) {
          dw[dg] |= uint32_t(__builtin_amdgcn_mov_dpp(int(dw[dg]), 0xB1, 0xf, 0xf, false));  // quad [1,0,3,2]
          dw[dg] |= uint32_t(__builtin_amdgcn_mov_dpp(int(dw[dg]), 0x4E, 0xf, 0xf, false));  // quad [2,3,0,1]
        }
        if ((n16 & 3) == 0 && h < ROWS) {
          if constexpr (G1) {
            if (h == 0) {
#pragma unroll
              for (int dg = 0; dg < 3; ++dg) dig[s * 64 + (4 * slot + dg) * 4 + (n16 >> 2)] = dw[dg];
            }
          } else {
#pragma unroll
            for (int dg = 0; dg < 3; ++dg) dig[((i * NS + s) * 3 + dg) * 64 + (4 * slot + r4) * 4 + (n16 >> 2)] = dw[dg];
          }
        }
      }
    }
  }
  __syncthreads();
  v4i aop[G1 ? 1 : NRB][NS][G1 ? 1 : 3];
  {
    const int r = lane & 15, slot = lane >> 4;
#pragma unroll
    for (int rb = 0; rb < (G1 ? 1 : NRB); ++rb)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int dg = 0; dg < (G1 ? 1 : 3); ++dg) {
          bool on;
          int off;
          if constexpr (G1) {
            on = (r >> 2) == slot && (r & 3) < 3;
            off = s * 64 + r * 4;
          } else {
            on = (r & 3) == slot && 4 * rb + (r >> 2) < ROWS;
            off = ((rb * NS + s) * 3 + dg) * 64 + (4 * slot + (r >> 2)) * 4;
          }
          const uint4 v = on ? *reinterpret_cast<const uint4*>(dig + off) : make_uint4(0u, 0u, 0u, 0u);
          aop[rb][s][dg] = v4i{int(v.x), int(v.y), int(v.z), int(v.w)};
        }
  }
  __syncthreads();  // the main loop's tiles overwrite the prologue's LDS

  uint8_t* wbase = smem + w * Gm::LDS_WAVE;
  uint8_t* vtile = wbase;
  uint16_t* stile = reinterpret_cast<uint16_t*>(wbase + Gm::LDS_V);
  uint16_t* ktile = reinterpret_cast<uint16_t*>(wbase + Gm::LDS_V + Gm::LDS_S);
  uint16_t* ptile = reinterpret_cast<uint16_t*>(wbase + Gm::LDS_V + Gm::LDS_S + Gm::LDS_K);
  float* atile = reinterpret_cast<float*>(wbase + Gm::LDS_V + Gm::LDS_S + Gm::LDS_K + Gm::LDS_P);

  // P rows never produced by a score row block and alpha of such heads stay neutral
  for (int i = lane; i < 32 * kSB / 2; i += 64) reinterpret_cast<uint32_t*>(ptile)[i] = 0u;
  if (lane < 16) atile[lane] = 1.0f;

  float m_run[NRB], l_run[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.0f;
  }
  v4f acc[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  for (int k = 0; base < t_end; ++k) {
    if (app && t_app >= base && t_app < base + kSB) patch_superblock<D, KB, VB>(ra, t_app - base, appbuf, lane);
    process_superblock<D, KB, VB, NRB, G1>(ra, base, t_end, lane, aop, sig, rlo, rhi, lo_max, hi_min, m_run, l_run, acc,
                                           vtile, stile, ktile, ptile, atile, kc, ks, vc, vs, base + kStride,
                                           sb_slot(next_pos(pos), k + 1), min(L - (base + kStride), kSB));
    base += kStride;
    pos = next_pos(pos);
  }
  if constexpr (NRB <= 2) {
    // (head, part) rows: add the lo rows of a head (lanes 32-63) to its hi rows (lanes 0-31)
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[g][i]), __float_as_uint(acc[g][i]), false,
                                                        false);
        acc[g][i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
  }

  if (P.n_chunks == 1) {
    finish_direct<D, true, NRB>(m_run, l_run, acc, [](int k, int rr) { return 4 * k + rr; }, P.merge, unit,
                                reinterpret_cast<float*>(smem));
    return;
  }
  PartialArgs e;
  e.head_tile = ROWS;
  e.max_chunks = P.max_chunks;
  e.chunk_index = ch;
  e.unit = unit;
  e.pml = P.pml;
  e.pacc = P.pacc;
  store_partial<D, NRB>(m_run, l_run, acc, [](int k, int rr) { return 4 * k + rr; }, e,
                        reinterpret_cast<float*>(smem));
  if (!arrive_last(P.counters + unit, P.n_chunks, &last_flag)) return;
  merge_unit<D, true>(P.merge, unit, reinterpret_cast<float*>(smem));
}

template <int D, int KB, int VB>
hipError_t launch_q(const DecodeArgs& a, const DecodePlan& p, const WsLayout& w, hipStream_t s) {
  char* ws = static_cast<char*>(a.workspace);
  const int units = a.batch * a.kv_heads * p.head_tiles * p.tok_tiles;
  QDecodeParams P;
  P.kc = static_cast<const uint8_t*>(a.k_codes);
  P.ks = static_cast<const uint16_t*>(a.k_scales);
  P.vc = static_cast<const uint8_t*>(a.v_codes);
  P.vs = static_cast<const uint16_t*>(a.v_scales);
  P.seq_lens = a.seq_lens;
  P.seq_len = a.seq_len;
  P.kv_heads = a.kv_heads;
  P.q_heads = a.q_heads;
  P.capacity = a.capacity;
  P.head_tile = p.head_tile;
  P.head_tiles = p.head_tiles;
  P.chunk = p.chunk;
  P.n_chunks = p.n_chunks;
  P.max_chunks = p.max_chunks;
  P.q = static_cast<const uint16_t*>(a.q);
  P.sign_k = a.sign_k;
  P.lambda_k = a.lambda_k;
  P.sign_bs = a.sign_bs;
  P.lambda_bs = a.lambda_bs;
  P.score_scale = a.sm_scale * kLog2e;
  P.counters = reinterpret_cast<uint32_t*>(ws + w.counters);
  P.pml = reinterpret_cast<float*>(ws + w.pml);
  P.pacc = reinterpret_cast<float*>(ws + w.pacc);
  // int4: code * scale was staged as code * scale / 16 in fp16, acc_scale 16 undoes it (int8
  // keeps the product's scale)
  MergeArgs& m = P.merge;
  m = MergeArgs{};
  m.pml = P.pml;
  m.pacc = P.pacc;
  m.n_chunks = p.n_chunks;
  m.max_chunks = p.max_chunks;
  m.head_tile = p.rows;
  m.head_tiles = p.head_tiles;
  m.q_heads = a.q_heads;
  m.kv_heads = a.kv_heads;
  m.gt = p.head_tile;
  m.tok_tile = p.tok_tile;
  m.tok_tiles = p.tok_tiles;
  m.n_query = a.n_query;
  m.acc_scale = VB == 4 ? 16.0f : 1.0f;
  m.sign = a.sign_v;
  m.sign_bs = a.sign_bs;
  m.lambda = a.lambda_v;
  m.lambda_bs = a.lambda_bs;
  m.out = a.out;
  m.transform = a.transform;
  P.tok_tile = p.tok_tile;
  P.tok_tiles = p.tok_tiles;
  P.rows = p.rows;
  P.n_query = a.n_query;
  P.window = a.window;
  P.ring = a.ring;
  P.k_new = static_cast<const uint16_t*>(a.k_new);
  P.v_new = static_cast<const uint16_t*>(a.v_new);
  P.page_table = a.page_table;
  P.page_size = a.page_size;
  P.pages_per_seq = a.pages_per_seq;
  P.num_pages = a.num_pages;
  const dim3 grid(units * p.n_chunks), block(kThreads);
  const bool app = a.k_new != nullptr;
#define KVQ_DLAUNCH(NRB, G1)                                                          \
  if (app)                                                                            \
    hipLaunchKernelGGL((decode_kernel<D, KB, VB, NRB, true, G1>), grid, block, 0, s, P);  \
  else                                                                                \
    hipLaunchKernelGGL((decode_kernel<D, KB, VB, NRB, false, G1>), grid, block, 0, s, P);
  switch ((p.rows + 3) / 4) {
    case 1:
      if (p.rows == 1) {
        KVQ_DLAUNCH(1, true);
      } else {
        KVQ_DLAUNCH(1, false);
      }
      break;
    case 2:
      KVQ_DLAUNCH(2, false);
      break;
    case 3:
      KVQ_DLAUNCH(3, false);
      break;
    case 4:
      KVQ_DLAUNCH(4, false);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef KVQ_DLAUNCH
  return hipGetLastError();
}

}  // namespace

// The instances of one head dimension (each is built in a translation unit of its own).
template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const WsLayout w = ws_layout(a.batch * a.kv_heads * p.head_tiles * p.tok_tiles, p.rows, a.head_dim, p.max_chunks);
  switch (a.k_bits * 10 + a.v_bits) {
    case 44: return launch_q<D, 4, 4>(a, p, w, s);
    case 84: return launch_q<D, 8, 4>(a, p, w, s);
    case 48: return launch_q<D, 4, 8>(a, p, w, s);
    case 88: return launch_q<D, 8, 8>(a, p, w, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq_impl
