// Host-side planning of decode launches: head tiling, chunk size and workspace size.
// Pure host code (no HIP call), shared by the quantized and the fp16 paths.
#include <algorithm>

#include "kvq_internal.h"

namespace kvq_impl {
namespace {

// Work-groups one launch should have: every CU holds two work-groups of the d = 128 kernels
// at once and one of the d = 256 kernels (register-limited), and the chunk split aims at one
// full round of resident work-groups.
long target_workgroups(int head_dim) { return head_dim == 128 ? 512 : 256; }

int token_align(bool f16) { return f16 ? 4 * 32 : 4 * 64; }  // 4 waves x superblock

}  // namespace

QuantPlan plan_quantize(int head_dim, int64_t n_vec) {
  QuantPlan q;
  q.blocks = (n_vec + kQuantVecs - 1) / kQuantVecs;
  // resident work-groups: 3 per CU at d = 128 (256 threads), 1 at d = 256 (512 threads)
  const int64_t resident = head_dim == 128 ? 3 * 256 : 256;
  q.grid = int(std::max<int64_t>(1, std::min<int64_t>(q.blocks, resident)));
  return q;
}

DecodePlan plan_decode(int batch, int kv_heads, int q_heads, int head_dim, int seq_len, int max_seq_len, bool f16,
                       bool append, bool paged, int n_query, int window) {
  DecodePlan p{};
  const int G = q_heads / kv_heads;
  const int T = std::max(n_query, 1);
  // epilogue LDS holds 4 x rows x d floats; an appending call rotates the new K and V vectors
  // in rows 14 and 15 of the query rotation
  const int max_rows = head_dim == 128 ? (append ? 14 : 16) : 8;
  // (head tile, token tile) with rows <= max_rows and the fewest tiles per kv head (each tile reads
  // the kv head's cache once); ties go to the larger head tile
  int best_gt = 1, best_tt = 1;
  long best_tiles = -1;
  for (int gt = std::min(G, max_rows); gt >= 1; --gt) {
    if (G % gt) continue;
    const int tt = std::min(T, max_rows / gt);
    const long tiles = long(G / gt) * ((T + tt - 1) / tt);
    if (best_tiles < 0 || tiles < best_tiles) {
      best_tiles = tiles;
      best_gt = gt;
      best_tt = tt;
    }
  }
  p.head_tile = best_gt;
  p.head_tiles = G / best_gt;
  p.tok_tile = best_tt;
  p.tok_tiles = (T + best_tt - 1) / best_tt;
  p.rows = best_gt * best_tt;
  const long units = long(batch) * kv_heads * p.head_tiles * p.tok_tiles;
  const long cap_chunks = std::max(1L, (target_workgroups(head_dim) + units - 1) / units);
  const int align = token_align(f16);
  // tokens one unit attends: its queries' prefix, or with a window the window of its first query
  // through its last query, plus up to 63 tokens before the window's start (superblocks start at
  // multiples of 64)
  auto span = [&](int len) {
    return window > 0 ? int(std::min<long>(len, long(window) + p.tok_tile - 1 + 63)) : len;
  };
  auto chunk_for = [&](int len) {
    long per = (std::max(len, 1) + cap_chunks - 1) / cap_chunks;
    per = ((per + align - 1) / align) * align;
    // a paged call keeps each wave's page list in one register: at most 64 superblocks a wave
    if (paged) per = std::min<long>(per, 64L * align);
    return int(std::max<long>(align, per));
  };
  p.chunk = chunk_for(span(seq_len));
  p.n_chunks = (std::max(span(seq_len), 1) + p.chunk - 1) / p.chunk;
  const int mc = chunk_for(span(max_seq_len));
  p.max_chunks = std::max(p.n_chunks, (std::max(span(max_seq_len), 1) + mc - 1) / mc);
  return p;
}

size_t decode_workspace_bytes(int batch, int kv_heads, int q_heads, int head_dim, int max_seq_len) {
  size_t need = 0;
  // variants: quantized, fp16, quantized + append, then both quantized ones on a paged cache
  for (int variant = 0; variant < 5; ++variant) {
    const DecodePlan p = plan_decode(batch, kv_heads, q_heads, head_dim, max_seq_len, max_seq_len, variant == 1,
                                     variant == 2 || variant == 4, variant >= 3);
    const WsLayout w = ws_layout(batch * kv_heads * p.head_tiles * p.tok_tiles, p.rows, head_dim, p.max_chunks);
    need = std::max(need, w.total);
  }
  return need;
}

size_t attn_workspace_bytes(int batch, int kv_heads, int q_heads, int head_dim, int max_seq_len, int n_query,
                            int window) {
  size_t need = 0;
  for (int paged = 0; paged < 2; ++paged) {
    const DecodePlan p = plan_decode(batch, kv_heads, q_heads, head_dim, max_seq_len, max_seq_len, false, false,
                                     paged != 0, n_query, window);
    const WsLayout w = ws_layout(batch * kv_heads * p.head_tiles * p.tok_tiles, p.rows, head_dim, p.max_chunks);
    need = std::max(need, w.total);
  }
  return need;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t s) {
  if (a.head_dim == 128) return launch_decode_d<128>(a, p, s);
  if (a.head_dim == 256) return launch_decode_d<256>(a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq_impl
