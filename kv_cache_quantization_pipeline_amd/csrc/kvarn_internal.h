// Kernel launchers behind the libkvarn C-ABI (host-side declarations).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvarn {

// ng: quantisation groups per token (128 / group size): 1, 2 or 4.
hipError_t launch_quantize_tiles(const _Float16* k, const _Float16* v, const int32_t* dst_pages, uint8_t* cache,
                                 int64_t page_stride, int num_tiles, int num_kv_heads, int kb, int vb, int ng,
                                 int iters, hipStream_t stream);

hipError_t launch_append(const _Float16* k_new, const _Float16* v_new, int32_t* seq_lens, _Float16* tail_k,
                         _Float16* tail_v, const int32_t* page_table, int max_pages, uint8_t* cache,
                         int64_t page_stride, int num_seqs, int num_kv_heads, int kb, int vb, int ng, int iters,
                         hipStream_t stream);

// Split-K decode plan: the grid is (num_seqs*num_kv_heads, n_splits) workgroups of 4 waves, n_splits
// sized for max_pages_per_seq (groups_per_split groups of pages_per_group pages per split at that
// length).  The kernel shares each sequence's actual groups evenly among its n_splits workgroups.
struct DecodePlan {
  int pages_per_group;
  int groups_per_split;
  int n_splits;
  // 0: the fp16 tail is shared out among all n_splits splits; T > 0: splits 0 .. T-1 own the tail
  // and no pages, splits T .. n_splits-1 own the pages
  int tail_splits;
};
// ng: quantisation groups per token (1, 2, 4); group_size: query heads per kv head.
int decode_pages_per_step(int kb, int vb, int ng, int group_size);
DecodePlan plan_decode(int kb, int vb, int ng, int num_seqs, int num_kv_heads, int group_size, int max_pages_per_seq);

// Decode workspace: one int32 arrival counter per (sequence, kv head), padded to 256 bytes, then
// kPartialFloats floats per (sequence, query head, split): running max, running sum, a flag (1 if
// the split owns fp16 tail tokens), a pad float, 128 rotated-domain accumulators and 128 raw-domain
// tail accumulators (written only with the flag set).  The counters must be zero when a launch
// starts; every launch leaves them zero.
constexpr int kPartialFloats = 260;

// The append kernel counts the arrivals of a sequence's kv-head workgroups in the bits of
// seq_lens[s] from this one up, so lengths stay below 2^24 tokens and kv heads at most 64.
constexpr int kArrivalShift = 24;
constexpr int kMaxAppendKvHeads = 64;
inline size_t decode_counter_bytes(int num_seqs, int num_kv_heads) {
  return (static_cast<size_t>(num_seqs) * num_kv_heads * sizeof(int32_t) + 255) / 256 * 256;
}

bool decode_supported(int kb, int vb, int ng, int group_size);

hipError_t launch_decode(int kb, int vb, int ng, int group_size, const _Float16* q, const uint8_t* cache,
                         int64_t page_stride, const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                         const _Float16* tail_k, const _Float16* tail_v, float sm_scale, _Float16* out,
                         float* workspace, int* counters, int num_seqs, int num_q_heads, int num_kv_heads,
                         const DecodePlan& plan, hipStream_t stream);
// The kernels of one group count (ng = 1, 2, 4), each in its own object.
#define KVARN_DECL_LAUNCHER(N)                                                                                \
  hipError_t launch_decode_ng##N(int kb, int vb, int group_size, const _Float16* q, const uint8_t* cache,     \
                                 int64_t page_stride, const int32_t* page_table, int max_pages,               \
                                 const int32_t* seq_lens, const _Float16* tail_k, const _Float16* tail_v,     \
                                 float sm_scale, _Float16* out, float* workspace, int* counters, int num_seqs, \
                                 int num_q_heads, int num_kv_heads, const DecodePlan& plan, hipStream_t stream);
KVARN_DECL_LAUNCHER(1)
KVARN_DECL_LAUNCHER(2)
KVARN_DECL_LAUNCHER(4)
#undef KVARN_DECL_LAUNCHER


// Chunked prefill (one quantisation group per token): grid (num_seqs * num_kv_heads, row blocks of
// 64 (query token, query head) rows).
bool prefill_supported(int kb, int vb, int ng, int group_size);
int prefill_row_blocks(int max_q, int group_size);
hipError_t launch_prefill(int kb, int vb, int group_size, const _Float16* q, const int32_t* q_lens, int max_q,
                          const uint8_t* cache, int64_t page_stride, const int32_t* page_table, int max_pages,
                          const int32_t* seq_lens, const _Float16* tail_k, const _Float16* tail_v, float sm_scale,
                          _Float16* out, int num_seqs, int num_q_heads, int num_kv_heads, hipStream_t stream);

}  // namespace kvarn
