// Read path for gfx950: single-token decode attention over the quantized cache, computed in
// the rotated domain, and the same attention over an fp16 cache (the comparator).
//
// The quantized path never reconstructs K or V in the original domain:
//   score_t = q . x_hat_K,t = (SRFT_sK(q) * lambda_K) . (code_K,t * scale_K,t)
//   out     = s_V * SRFT^-1( lambda_V * sum_t p_t code_V,t * scale_V,t )
// because the rotation is orthogonal ("When Quantization Is Free", technical summary,
// Methodology 1).  The sum over tokens is split into chunks handled by independent
// work-groups, each keeping an online softmax (running max m, sum l, accumulator acc), and the
// chunks are merged with a log-sum-exp combine before the single inverse rotation (the tiled,
// online-softmax attention of the hotdry blog, "Flash Attention 与 Metal 内核融合").
//
// Kernels
//   qhat_kernel    : q_hat = SRFT_sK(q) * lambda_K * sm_scale * log2(e), one work-group per
//                    (sequence, query head), one thread per output channel (O(d^2) with an LDS
//                    twiddle table: this vector count is tiny and latency matters)
//   decode_q_kernel: split-K main loop, one work-group per (sequence, kv head, head tile, chunk)
//   decode_f16_kernel: the same over fp16 K/V
//   merge_kernel   : combine chunks, apply lambda_V, inverse rotation (quantized) -> out fp32
#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq_impl {
namespace {

using namespace kvqd;

constexpr int kDecThreads = 256;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kMaxHeadsPerTile = 4;
constexpr int kTargetWorkgroups = 2048;
constexpr int kMinChunk = 256;

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

__constant__ TwTable<128> kTw128 = TwTable<128>();
__constant__ TwTable<256> kTw256 = TwTable<256>();

template <int D>
__device__ __forceinline__ const TwTable<D>& tw_table() {
  if constexpr (D == 128)
    return kTw128;
  else
    return kTw256;
}

// Workspace sections (byte offsets are 256-aligned).
struct WsLayout {
  size_t qhat, pml, pacc, total;
};

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

__host__ __device__ inline WsLayout ws_layout(int batch, int q_heads, int head_dim, int max_chunks) {
  WsLayout w;
  const size_t rows = size_t(batch) * q_heads;
  w.qhat = 0;
  w.pml = align256(rows * head_dim * sizeof(float));
  w.pacc = w.pml + align256(rows * max_chunks * 2 * sizeof(float));
  w.total = w.pacc + align256(rows * max_chunks * size_t(head_dim) * sizeof(float));
  return w;
}

__device__ __forceinline__ float exp2_guard(float a, float m) {
  // exp2(a - m) with exp2(-inf - -inf) := 0
  return a == -INFINITY ? 0.0f : exp2f(a - m);
}

// q_hat[b, h, c] for every (b, h): block = D threads, grid = batch * q_heads.
template <int D>
__global__ __launch_bounds__(D) void qhat_kernel(const uint16_t* __restrict__ q, int q_heads, int kv_heads,
                                                 const float* __restrict__ sign, int64_t sign_bs,
                                                 const float* __restrict__ lambda, int64_t lambda_bs, float scale,
                                                 float* __restrict__ qhat) {
  __shared__ float qs[D];
  __shared__ float tc[D], ts[D];
  const int bh = blockIdx.x;
  const int b = bh / q_heads;
  const int h = bh - b * q_heads;
  const int c = threadIdx.x;
  {
    const float sg = sign[b * sign_bs + c] < 0.0f ? -1.0f : 1.0f;
    qs[c] = sg * static_cast<float>(__builtin_bit_cast(_Float16, q[int64_t(bh) * D + c]));
    tc[c] = tw_table<D>().c[c];
    ts[c] = tw_table<D>().s[c];
  }
  __syncthreads();
  float acc = 0.0f;
  if (c < 2) {
    for (int n = 0; n < D; ++n) acc += ((c == 1 && (n & 1)) ? -qs[n] : qs[n]);
    acc *= float(1.0 / csqrt(double(D)));
  } else {
    const int k = c >> 1;
    const bool im = c & 1;
    int m = 0;
    for (int n = 0; n < D; ++n) {
      acc = fmaf(qs[n], im ? ts[m] : tc[m], acc);
      m = (m + k) & (D - 1);
    }
    acc *= (im ? -1.0f : 1.0f) * float(csqrt(2.0 / double(D)));
  }
  const int kvh = h / (q_heads / kv_heads);
  const float lam = lambda ? lambda[b * lambda_bs + int64_t(kvh) * D + c] : 1.0f;
  qhat[int64_t(bh) * D + c] = acc * lam * scale;
}

// Unpack 16 codes of one group to float.
template <int BITS>
__device__ __forceinline__ void load_group_codes(const uint8_t* __restrict__ p, float (&f)[16]) {
  if constexpr (BITS == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    static_for<0, 8>([&](auto I) {
      constexpr int i = decltype(I)::value;
      f[i] = static_cast<float>(static_cast<int32_t>(w.x << (28 - 4 * i)) >> 28);
      f[8 + i] = static_cast<float>(static_cast<int32_t>(w.y << (28 - 4 * i)) >> 28);
    });
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    static_for<0, 16>([&](auto I) {
      constexpr int i = decltype(I)::value;
      f[i] = static_cast<float>(static_cast<int32_t>(ww[i / 4] << (24 - 8 * (i % 4))) >> 24);
    });
  }
}

__device__ __forceinline__ float half_bits_to_float(uint16_t v) {
  return static_cast<float>(__builtin_bit_cast(_Float16, v));
}

// Cross-slot combine at the end of a work-group's chunk and store of one partial
// (m, l, acc) per query head.  Each lane holds 16 channels (group gi) of one token slot.
template <int D, int GT>
__device__ __forceinline__ void finish_chunk(float (&m)[GT], float (&l)[GT], float (&acc)[GT][16], int gi,
                                             float* __restrict__ pml, float* __restrict__ pacc, int64_t row0,
                                             int q_stride_rows, int max_chunks, int ch) {
  constexpr int LPT = D / 16;
  __shared__ float sm_m[4][GT], sm_l[4][GT];
  __shared__ float sm_acc[4][GT][D];
  // within a wave: lanes with the same gi, different slots, differ in lane bits >= log2(LPT)
  static_for<0, GT>([&](auto H) {
    constexpr int h = decltype(H)::value;
    float mm = m[h];
    for (int off = LPT; off < 64; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off));
    const float f = exp2_guard(m[h], mm);
    float ll = l[h] * f;
    for (int off = LPT; off < 64; off <<= 1) ll += __shfl_xor(ll, off);
    static_for<0, 16>([&](auto C) {
      constexpr int c = decltype(C)::value;
      float a = acc[h][c] * f;
      for (int off = LPT; off < 64; off <<= 1) a += __shfl_xor(a, off);
      acc[h][c] = a;
    });
    m[h] = mm;
    l[h] = ll;
  });
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  if (lane < LPT) {
    static_for<0, GT>([&](auto H) {
      constexpr int h = decltype(H)::value;
      if (lane == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
      static_for<0, 16>([&](auto C) {
        constexpr int c = decltype(C)::value;
        sm_acc[wave][h][16 * gi + c] = acc[h][c];
      });
    });
  }
  __syncthreads();
  for (int i = threadIdx.x; i < GT * D; i += blockDim.x) {
    const int h = i / D, c = i - h * D;
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, sm_m[w][h]);
    float a = 0.0f, ll = 0.0f;
    for (int w = 0; w < 4; ++w) {
      const float f = exp2_guard(sm_m[w][h], mm);
      a += sm_acc[w][h][c] * f;
      ll += sm_l[w][h] * f;
    }
    const int64_t prow = (row0 + int64_t(h) * q_stride_rows) * max_chunks + ch;
    pacc[prow * D + c] = a;
    if (c == 0) {
      pml[2 * prow] = mm;
      pml[2 * prow + 1] = ll;
    }
  }
}

template <int D, int KB, int VB, int GT>
__global__ __launch_bounds__(kDecThreads) void decode_q_kernel(
    const uint8_t* __restrict__ kc, const uint16_t* __restrict__ ks, const uint8_t* __restrict__ vc,
    const uint16_t* __restrict__ vs, const float* __restrict__ qhat, const int32_t* __restrict__ seq_lens,
    int seq_len, int kv_heads, int q_heads, int capacity, int head_tiles, int chunk, int n_chunks,
    int max_chunks, float* __restrict__ pml, float* __restrict__ pacc) {
  constexpr int LPT = D / 16;
  constexpr int SLOTS = kDecThreads / LPT;
  const int G = q_heads / kv_heads;
  const int ch = blockIdx.x % n_chunks;
  const int unit = blockIdx.x / n_chunks;
  const int ht = unit % head_tiles;
  const int bk = unit / head_tiles;
  const int kvh = bk % kv_heads;
  const int b = bk / kv_heads;
  const int h0 = kvh * G + ht * GT;
  int L = seq_len;
  if (seq_lens) L = min(max(seq_lens[b], 0), seq_len);
  const int t_begin = ch * chunk;
  const int t_end = min(L, t_begin + chunk);
  const int slot = threadIdx.x / LPT;
  const int gi = threadIdx.x - slot * LPT;

  float qv[GT][16];
  static_for<0, GT>([&](auto H) {
    constexpr int h = decltype(H)::value;
    const float4* q4 = reinterpret_cast<const float4*>(qhat + (int64_t(b) * q_heads + h0 + h) * D + 16 * gi);
    static_for<0, 4>([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      const float4 f = q4[q];
      qv[h][4 * q] = f.x;
      qv[h][4 * q + 1] = f.y;
      qv[h][4 * q + 2] = f.z;
      qv[h][4 * q + 3] = f.w;
    });
  });
  float acc[GT][16], m[GT], l[GT];
  static_for<0, GT>([&](auto H) {
    constexpr int h = decltype(H)::value;
    m[h] = -INFINITY;
    l[h] = 0.0f;
    static_for<0, 16>([&](auto C) { acc[h][decltype(C)::value] = 0.0f; });
  });

  const int64_t rowbase = (int64_t(b) * kv_heads + kvh) * capacity;
  for (int t0 = t_begin; t0 < t_end; t0 += SLOTS) {
    const int t = t0 + slot;
    const bool valid = t < t_end;
    const int64_t tok = rowbase + (valid ? t : t_begin);
    float kf[16];
    load_group_codes<KB>(kc + tok * (D * KB / 8) + gi * (16 * KB / 8), kf);
    const float ksc = half_bits_to_float(ks[tok * (D / 16) + gi]);
    float vf[16];
    load_group_codes<VB>(vc + tok * (D * VB / 8) + gi * (16 * VB / 8), vf);
    const float vsc = half_bits_to_float(vs[tok * (D / 16) + gi]);
    static_for<0, GT>([&](auto H) {
      constexpr int h = decltype(H)::value;
      float s = 0.0f;
      static_for<0, 16>([&](auto C) { s = fmaf(qv[h][decltype(C)::value], kf[decltype(C)::value], s); });
      s *= ksc;
      for (int off = 1; off < LPT; off <<= 1) s += __shfl_xor(s, off);
      s = valid ? s : -INFINITY;
      const float mn = fmaxf(m[h], s);
      const float alpha = exp2_guard(m[h], mn);
      const float p = exp2_guard(s, mn);
      m[h] = mn;
      l[h] = l[h] * alpha + p;
      const float w = p * vsc;
      static_for<0, 16>([&](auto C) {
        constexpr int c = decltype(C)::value;
        acc[h][c] = fmaf(acc[h][c], alpha, w * vf[c]);
      });
    });
  }
  const int64_t row0 = int64_t(b) * q_heads + h0;
  finish_chunk<D, GT>(m, l, acc, gi, pml, pacc, row0, 1, max_chunks, ch);
}

template <int D, int GT>
__global__ __launch_bounds__(kDecThreads) void decode_f16_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ seq_lens, int seq_len, int kv_heads, int q_heads, int capacity, int head_tiles,
    int chunk, int n_chunks, int max_chunks, float qscale, float* __restrict__ pml, float* __restrict__ pacc) {
  constexpr int LPT = D / 16;
  constexpr int SLOTS = kDecThreads / LPT;
  const int G = q_heads / kv_heads;
  const int ch = blockIdx.x % n_chunks;
  const int unit = blockIdx.x / n_chunks;
  const int ht = unit % head_tiles;
  const int bk = unit / head_tiles;
  const int kvh = bk % kv_heads;
  const int b = bk / kv_heads;
  const int h0 = kvh * G + ht * GT;
  int L = seq_len;
  if (seq_lens) L = min(max(seq_lens[b], 0), seq_len);
  const int t_begin = ch * chunk;
  const int t_end = min(L, t_begin + chunk);
  const int slot = threadIdx.x / LPT;
  const int gi = threadIdx.x - slot * LPT;

  float qv[GT][16];
  static_for<0, GT>([&](auto H) {
    constexpr int h = decltype(H)::value;
    const uint4* q4 = reinterpret_cast<const uint4*>(q + (int64_t(b) * q_heads + h0 + h) * D + 16 * gi);
    static_for<0, 2>([&](auto Q) {
      constexpr int j = decltype(Q)::value;
      const uint4 w = q4[j];
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
      static_for<0, 4>([&](auto I) {
        constexpr int i = decltype(I)::value;
        qv[h][8 * j + 2 * i] = half_lo(ww[i]) * qscale;
        qv[h][8 * j + 2 * i + 1] = half_hi(ww[i]) * qscale;
      });
    });
  });
  float acc[GT][16], m[GT], l[GT];
  static_for<0, GT>([&](auto H) {
    constexpr int h = decltype(H)::value;
    m[h] = -INFINITY;
    l[h] = 0.0f;
    static_for<0, 16>([&](auto C) { acc[h][decltype(C)::value] = 0.0f; });
  });
  const int64_t rowbase = (int64_t(b) * kv_heads + kvh) * capacity;
  for (int t0 = t_begin; t0 < t_end; t0 += SLOTS) {
    const int t = t0 + slot;
    const bool valid = t < t_end;
    const int64_t tok = rowbase + (valid ? t : t_begin);
    float kf[16], vf[16];
    {
      const uint4* k4 = reinterpret_cast<const uint4*>(k + tok * D + 16 * gi);
      const uint4* v4 = reinterpret_cast<const uint4*>(v + tok * D + 16 * gi);
      static_for<0, 2>([&](auto Q) {
        constexpr int j = decltype(Q)::value;
        const uint4 kw = k4[j], vw = v4[j];
        const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w};
        const uint32_t vv[4] = {vw.x, vw.y, vw.z, vw.w};
        static_for<0, 4>([&](auto I) {
          constexpr int i = decltype(I)::value;
          kf[8 * j + 2 * i] = half_lo(kk[i]);
          kf[8 * j + 2 * i + 1] = half_hi(kk[i]);
          vf[8 * j + 2 * i] = half_lo(vv[i]);
          vf[8 * j + 2 * i + 1] = half_hi(vv[i]);
        });
      });
    }
    static_for<0, GT>([&](auto H) {
      constexpr int h = decltype(H)::value;
      float s = 0.0f;
      static_for<0, 16>([&](auto C) { s = fmaf(qv[h][decltype(C)::value], kf[decltype(C)::value], s); });
      for (int off = 1; off < LPT; off <<= 1) s += __shfl_xor(s, off);
      s = valid ? s : -INFINITY;
      const float mn = fmaxf(m[h], s);
      const float alpha = exp2_guard(m[h], mn);
      const float p = exp2_guard(s, mn);
      m[h] = mn;
      l[h] = l[h] * alpha + p;
      static_for<0, 16>([&](auto C) {
        constexpr int c = decltype(C)::value;
        acc[h][c] = fmaf(acc[h][c], alpha, p * vf[c]);
      });
    });
  }
  const int64_t row0 = int64_t(b) * q_heads + h0;
  finish_chunk<D, GT>(m, l, acc, gi, pml, pacc, row0, 1, max_chunks, ch);
}

// Combine the chunks of one (sequence, query head); quantized path applies lambda_V and the
// inverse rotation.  block = D threads, grid = batch * q_heads.
template <int D, bool ROT>
__global__ __launch_bounds__(D) void merge_kernel(const float* __restrict__ pml, const float* __restrict__ pacc,
                                                  int n_chunks, int max_chunks, int q_heads, int kv_heads,
                                                  const float* __restrict__ sign, int64_t sign_bs,
                                                  const float* __restrict__ lambda, int64_t lambda_bs,
                                                  float* __restrict__ out) {
  __shared__ float y[D];
  __shared__ float tc[D], ts[D];
  const int bh = blockIdx.x;
  const int c = threadIdx.x;
  const float* ml = pml + int64_t(bh) * max_chunks * 2;
  float mm = -INFINITY;
  for (int i = 0; i < n_chunks; ++i) mm = fmaxf(mm, ml[2 * i]);
  float a = 0.0f, ll = 0.0f;
  for (int i = 0; i < n_chunks; ++i) {
    const float f = exp2_guard(ml[2 * i], mm);
    ll += ml[2 * i + 1] * f;
    a += pacc[(int64_t(bh) * max_chunks + i) * D + c] * f;
  }
  float val = ll > 0.0f ? a / ll : 0.0f;
  if constexpr (!ROT) {
    out[int64_t(bh) * D + c] = val;
  } else {
    const int b = bh / q_heads;
    const int h = bh - b * q_heads;
    const int kvh = h / (q_heads / kv_heads);
    if (lambda) val *= lambda[b * lambda_bs + int64_t(kvh) * D + c];
    y[c] = val;
    tc[c] = tw_table<D>().c[c];
    ts[c] = tw_table<D>().s[c];
    __syncthreads();
    // x_n = y0/sqrt(D) + (-1)^n y1/sqrt(D) + sqrt(2/D) sum_k (y_2k cos(2pi k n/D) - y_2k+1 sin(..))
    const int n = c;
    float acc = 0.0f;
    int mi = n;
    for (int k = 1; k < D / 2; ++k) {
      acc = fmaf(y[2 * k], tc[mi], acc);
      acc = fmaf(-y[2 * k + 1], ts[mi], acc);
      mi = (mi + n) & (D - 1);
    }
    const float base = (y[0] + ((n & 1) ? -y[1] : y[1])) * float(1.0 / csqrt(double(D)));
    const float x = base + acc * float(csqrt(2.0 / double(D)));
    const float sg = sign[b * sign_bs + n] < 0.0f ? -1.0f : 1.0f;
    out[int64_t(bh) * D + n] = sg * x;
  }
}

template <int D, int KB>
hipError_t decode_dispatch_gt(const DecodeArgs& a, const DecodePlan& p, const WsLayout& w, hipStream_t s) {
  char* ws = static_cast<char*>(a.workspace);
  float* qhat = reinterpret_cast<float*>(ws + w.qhat);
  float* pml = reinterpret_cast<float*>(ws + w.pml);
  float* pacc = reinterpret_cast<float*>(ws + w.pacc);
  const float scale = a.sm_scale * kLog2e;
  hipLaunchKernelGGL((qhat_kernel<D>), dim3(a.batch * a.q_heads), dim3(D), 0, s, static_cast<const uint16_t*>(a.q),
                     a.q_heads, a.kv_heads, a.sign_k, a.sign_bs, a.lambda_k, a.lambda_bs, scale, qhat);
  const dim3 grid(a.batch * a.kv_heads * p.head_tiles * p.n_chunks), block(kDecThreads);
  auto* kc = static_cast<const uint8_t*>(a.k_codes);
  auto* ks = static_cast<const uint16_t*>(a.k_scales);
  auto* vc = static_cast<const uint8_t*>(a.v_codes);
  auto* vs = static_cast<const uint16_t*>(a.v_scales);
#define KVQ_DEC_CASE(GTV)                                                                                        \
  case GTV:                                                                                                      \
    hipLaunchKernelGGL((decode_q_kernel<D, KB, 4, GTV>), grid, block, 0, s, kc, ks, vc, vs, qhat, a.seq_lens,     \
                       a.seq_len, a.kv_heads, a.q_heads, a.capacity, p.head_tiles, p.chunk, p.n_chunks,          \
                       p.max_chunks, pml, pacc);                                                                 \
    break;
  switch (p.heads_per_tile) {
    KVQ_DEC_CASE(1)
    KVQ_DEC_CASE(2)
    KVQ_DEC_CASE(3)
    KVQ_DEC_CASE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef KVQ_DEC_CASE
  hipLaunchKernelGGL((merge_kernel<D, true>), dim3(a.batch * a.q_heads), dim3(D), 0, s, pml, pacc, p.n_chunks,
                     p.max_chunks, a.q_heads, a.kv_heads, a.sign_v, a.sign_bs, a.lambda_v, a.lambda_bs, a.out);
  return hipGetLastError();
}

template <int D>
hipError_t decode_f16_dispatch(const DecodeF16Args& a, const DecodePlan& p, const WsLayout& w, hipStream_t s) {
  char* ws = static_cast<char*>(a.workspace);
  float* pml = reinterpret_cast<float*>(ws + w.pml);
  float* pacc = reinterpret_cast<float*>(ws + w.pacc);
  const float qscale = a.sm_scale * kLog2e;
  const dim3 grid(a.batch * a.kv_heads * p.head_tiles * p.n_chunks), block(kDecThreads);
  auto* k = static_cast<const uint16_t*>(a.k);
  auto* v = static_cast<const uint16_t*>(a.v);
  auto* q = static_cast<const uint16_t*>(a.q);
#define KVQ_F16_CASE(GTV)                                                                                      \
  case GTV:                                                                                                    \
    hipLaunchKernelGGL((decode_f16_kernel<D, GTV>), grid, block, 0, s, k, v, q, a.seq_lens, a.seq_len,         \
                       a.kv_heads, a.q_heads, a.capacity, p.head_tiles, p.chunk, p.n_chunks, p.max_chunks,     \
                       qscale, pml, pacc);                                                                     \
    break;
  switch (p.heads_per_tile) {
    KVQ_F16_CASE(1)
    KVQ_F16_CASE(2)
    KVQ_F16_CASE(3)
    KVQ_F16_CASE(4)
    default:
      return hipErrorInvalidValue;
  }
#undef KVQ_F16_CASE
  hipLaunchKernelGGL((merge_kernel<D, false>), dim3(a.batch * a.q_heads), dim3(D), 0, s, pml, pacc, p.n_chunks,
                     p.max_chunks, a.q_heads, a.kv_heads, nullptr, 0, nullptr, 0, a.out);
  return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int batch, int kv_heads, int q_heads, int head_dim, int seq_len, int max_seq_len) {
  (void)head_dim;
  DecodePlan p{};
  const int G = q_heads / kv_heads;
  int ht = 1;
  for (int d = std::min(G, kMaxHeadsPerTile); d >= 1; --d)
    if (G % d == 0) {
      ht = d;
      break;
    }
  p.heads_per_tile = ht;
  p.head_tiles = G / ht;
  const long units = long(batch) * kv_heads * p.head_tiles;
  const long cap_chunks = std::max(1L, (kTargetWorkgroups + units - 1) / units);
  auto chunk_for = [&](int len) {
    long per = (len + cap_chunks - 1) / cap_chunks;
    per = ((per + 63) / 64) * 64;
    return int(std::max<long>(kMinChunk, per));
  };
  p.chunk = chunk_for(std::max(seq_len, 1));
  p.n_chunks = (std::max(seq_len, 1) + p.chunk - 1) / p.chunk;
  const int mc = chunk_for(std::max(max_seq_len, 1));
  p.max_chunks = std::max(p.n_chunks, (std::max(max_seq_len, 1) + mc - 1) / mc);
  return p;
}

size_t decode_workspace_bytes(int batch, int kv_heads, int q_heads, int head_dim, int max_seq_len) {
  const DecodePlan p = plan_decode(batch, kv_heads, q_heads, head_dim, max_seq_len, max_seq_len);
  return ws_layout(batch, q_heads, head_dim, p.max_chunks).total;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  const WsLayout w = ws_layout(a.batch, a.q_heads, a.head_dim, p.max_chunks);
  if (a.head_dim == 128) return a.k_bits == 4 ? decode_dispatch_gt<128, 4>(a, p, w, s) : decode_dispatch_gt<128, 8>(a, p, w, s);
  return a.k_bits == 4 ? decode_dispatch_gt<256, 4>(a, p, w, s) : decode_dispatch_gt<256, 8>(a, p, w, s);
}

hipError_t launch_decode_f16(const DecodeF16Args& a, const DecodePlan& p, hipStream_t s) {
  const WsLayout w = ws_layout(a.batch, a.q_heads, a.head_dim, p.max_chunks);
  if (a.head_dim == 128) return decode_f16_dispatch<128>(a, p, w, s);
  return decode_f16_dispatch<256>(a, p, w, s);
}

}  // namespace kvq_impl
