// Internal launch interface between the C ABI (kvq_api.cpp) and the HIP kernels.
// Arguments arrive here already validated; launchers only compute grids and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq_impl {

struct QuantArgs {
  int batch, kv_heads, head_dim, bits, capacity;
  int pos, n_tok;
  const void* x;  // fp16 [batch, kv_heads, n_tok, d]
  const float* sign;
  int64_t sign_bs;
  const float* lambda;  // nullable
  int64_t lambda_bs;
  void* codes;
  void* scales;
  int transform;  // 0 = SRFT, 1 = SRHT
  int group;      // 16, or head_dim (one scale per vector)
};

struct DequantArgs {
  int batch, kv_heads, head_dim, bits, capacity;
  int pos, n_tok;
  const void* codes;
  const void* scales;
  const float* sign;
  int64_t sign_bs;
  const float* lambda;
  int64_t lambda_bs;
  float* out;
  int transform;
  int group;  // 16, or head_dim (one scale per vector)
};

struct CalibArgs {
  int batch, kv_heads, head_dim;
  int n_tok, n_cal;
  const void* x;
  const float* sign;
  int64_t sign_bs;
  float* lambda;
  int transform;
};

// Split of a decode / attention call into work-groups (shared by the quantized and the fp16
// kernels).  A unit is (sequence, kv head, head tile, query-token tile); its rows are
// tok_tile x head_tile (query token, head) pairs, at most 16 (8 at d = 256).
struct DecodePlan {
  int head_tile;   // query heads handled by one work-group (a divisor of G)
  int head_tiles;  // G / head_tile
  int tok_tile;    // query tokens handled by one work-group (1 for single-token decode)
  int tok_tiles;   // ceil(n_query / tok_tile)
  int rows;        // head_tile * tok_tile
  int chunk;       // tokens per work-group
  int n_chunks;    // work-groups per unit
  int max_chunks;  // chunk count the workspace layout is laid out for
};

struct DecodeArgs {
  int batch, kv_heads, q_heads, head_dim, k_bits, v_bits, capacity;
  int seq_len;
  const int32_t* seq_lens;  // nullable
  const void* q;
  const void* k_codes;
  const void* k_scales;
  const void* v_codes;
  const void* v_scales;
  const float* sign_k;
  const float* sign_v;
  int64_t sign_bs;
  const float* lambda_k;
  const float* lambda_v;
  int64_t lambda_bs;
  float sm_scale;
  void* workspace;
  float* out;
  int transform;
  // append (nullptr: none): new K and V vectors [batch, kv_heads, head_dim] fp16, quantized into
  // position L - 1 of every row before it is attended (the planes above are then written)
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  // paged cache (nullptr: contiguous rows): page_table [batch, pages_per_seq] device int32;
  // planes [num_pages, kv_heads, page_size, .]; page_size a multiple of 64
  const int32_t* page_table = nullptr;
  int page_size = 0, pages_per_seq = 0, num_pages = 0;
  // several query tokens (q and out [batch, n_query, q_heads, d]; query i of a sequence of
  // length L sits at position L - n_query + i and attends causally), a sliding window (0: none)
  // and ring-buffer slots (token t at slot t % capacity)
  int n_query = 1, window = 0, ring = 0;
};

struct DecodeF16Args {
  int batch, kv_heads, q_heads, head_dim, capacity;
  int seq_len;
  const int32_t* seq_lens;
  const void* q;
  const void* k;
  const void* v;
  float sm_scale;
  void* workspace;
  float* out;
};

// Decode workspace.  The first kDecodeCounterBytes hold one completion counter per unit
// (sequence, kv head, head tile); they must be zero before the first call and every call
// leaves them zero.  Then the per-chunk partials (m, l) and acc[d].
constexpr int kMaxDecodeUnits = 16384;
constexpr size_t kDecodeCounterBytes = size_t(kMaxDecodeUnits) * sizeof(uint32_t);

// Workspace of the allocation-free decode (kvq_decode_attn_noalloc): a device array of this
// many bytes per GPU, resolved on the first call on each device.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(hipStream_t stream, void** out);

struct WsLayout {
  size_t counters;  // uint32 per unit
  size_t pml;       // per (unit, head, chunk): m, l
  size_t pacc;      // per (unit, head, chunk): acc[d]
  size_t total;
};

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

__host__ __device__ inline WsLayout ws_layout(int units, int head_tile, int head_dim, int max_chunks) {
  WsLayout w;
  w.counters = 0;
  w.pml = kDecodeCounterBytes;
  w.pacc = w.pml + align256(size_t(units) * head_tile * max_chunks * 2 * sizeof(float));
  w.total = w.pacc + align256(size_t(units) * head_tile * max_chunks * size_t(head_dim) * sizeof(float));
  return w;
}

// Grid of the write path: 16-vector blocks, each work-group a contiguous range of them.
struct QuantPlan {
  int grid;          // work-groups
  int64_t blocks;    // 16-vector blocks in the call
};
constexpr int kQuantVecs = 16;  // vectors per block (MFMA columns)

// Host-side planning (pure host code, no HIP call).
QuantPlan plan_quantize(int head_dim, int64_t n_vec);
DecodePlan plan_decode(int batch, int kv_heads, int q_heads, int head_dim, int seq_len, int max_seq_len, bool f16,
                       bool append = false, bool paged = false, int n_query = 1, int window = 0);
size_t decode_workspace_bytes(int batch, int kv_heads, int q_heads, int head_dim, int max_seq_len);
// workspace of the multi-token / windowed attention (both the contiguous and the paged call)
size_t attn_workspace_bytes(int batch, int kv_heads, int q_heads, int head_dim, int max_seq_len, int n_query,
                            int window);

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
// the write path with the rotation as an in-register FFT on the vector ALUs (comparison form)
hipError_t launch_quantize_fft(const QuantArgs& a, hipStream_t stream);
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t stream);
hipError_t launch_calibrate(const CalibArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream);
// instances of one head dimension (128, 256), each built in its own translation unit
template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream);
hipError_t launch_decode_f16(const DecodeF16Args& a, const DecodePlan& p, hipStream_t stream);

}  // namespace kvq_impl
