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

// Split-K decode plan: the page kernel's grid is (num_seqs * num_kv_heads, tail_splits + page_splits)
// workgroups of 4 waves.  Split i < tail_splits of a (sequence, kv head) pair attends over tail tokens
// 128 i / tail_splits .. 128 (i + 1) / tail_splits - 1 (1 or kMaxTailSplits splits); split tail_splits + j streams
// page groups 4 j .. 4 j + 3 (one group of pages_per_group pages per wave), sized for
// max_pages_per_seq.  A merge kernel of num_seqs * num_q_heads workgroups follows.
struct DecodePlan {
  int pages_per_group;
  int tail_splits;
  int page_splits;
};
constexpr int kMaxTailSplits = 8;
// One partial result: 128 per-channel sums, the running max (log2 units), the running sum, 2 pad floats.
constexpr int kPartFloats = 132;

// ng: quantisation groups per token (1, 2, 4); group_size: query heads per kv head.
int decode_pages_per_step(int kb, int vb, int ng, int group_size);
DecodePlan plan_decode(int kb, int vb, int ng, int num_seqs, int num_kv_heads, int group_size, int max_pages_per_seq);

// Decode workspace: the split partials [seq][q head][tail_splits + page_splits][kPartFloats], written by the
// page kernel and read by the merge kernel of the same call; nothing is kept between calls.
struct DecodeWorkspace {
  float* part;
};
size_t decode_workspace_bytes(const DecodePlan& plan, int num_seqs, int num_q_heads, int num_kv_heads);
DecodeWorkspace decode_workspace_layout(void* workspace, const DecodePlan& plan, int num_seqs, int num_q_heads,
                                        int num_kv_heads);

// The append kernel counts the arrivals of a sequence's kv-head workgroups in the bits of
// seq_lens[s] from this one up, so lengths stay below 2^24 tokens and kv heads at most 64.
constexpr int kArrivalShift = 24;
constexpr int kMaxAppendKvHeads = 64;

bool decode_supported(int kb, int vb, int ng, int group_size);

hipError_t launch_decode(int kb, int vb, int ng, int group_size, const _Float16* q, const uint8_t* cache,
                         int64_t page_stride, const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                         const _Float16* tail_k, const _Float16* tail_v, float sm_scale, _Float16* out,
                         const DecodeWorkspace& ws, int num_seqs, int num_q_heads, int num_kv_heads,
                         const DecodePlan& plan, hipStream_t stream);
// The kernels of one group count (ng = 1, 2, 4), each in its own object.
#define KVARN_DECL_LAUNCHER(N)                                                                                \
  hipError_t launch_decode_ng##N(int kb, int vb, int group_size, const _Float16* q, const uint8_t* cache,     \
                                 int64_t page_stride, const int32_t* page_table, int max_pages,               \
                                 const int32_t* seq_lens, const _Float16* tail_k, const _Float16* tail_v,     \
                                 float sm_scale, _Float16* out, const DecodeWorkspace& ws, int num_seqs,     \
                                 int num_q_heads, int num_kv_heads, const DecodePlan& plan, hipStream_t stream);
KVARN_DECL_LAUNCHER(1)
KVARN_DECL_LAUNCHER(2)
KVARN_DECL_LAUNCHER(4)
#undef KVARN_DECL_LAUNCHER


// Chunked prefill: grid (num_seqs * num_kv_heads, row blocks of 64 (query token, query head) rows);
// ng quantisation groups per token (1, 2, 4).
bool prefill_supported(int kb, int vb, int ng, int group_size);
int prefill_row_blocks(int max_q, int group_size);
hipError_t launch_prefill(int kb, int vb, int ng, int group_size, const _Float16* q, const int32_t* q_lens, int max_q,
                          const uint8_t* cache, int64_t page_stride, const int32_t* page_table, int max_pages,
                          const int32_t* seq_lens, const _Float16* tail_k, const _Float16* tail_v, float sm_scale,
                          _Float16* out, int num_seqs, int num_q_heads, int num_kv_heads, hipStream_t stream);
// The prefill kernels of one group count, each in its own object.
#define KVARN_DECL_PF_LAUNCHER(N)                                                                                 \
  hipError_t launch_prefill_ng##N(int kb, int vb, int group_size, const _Float16* q, const int32_t* q_lens,       \
                                  int max_q, const uint8_t* cache, int64_t page_stride, const int32_t* page_table, \
                                  int max_pages, const int32_t* seq_lens, const _Float16* tail_k,                 \
                                  const _Float16* tail_v, float qscale, float rawscale, _Float16* out,            \
                                  int num_seqs, int num_kv_heads, int num_q_heads, int row_blocks,                \
                                  hipStream_t stream);
KVARN_DECL_PF_LAUNCHER(1)
KVARN_DECL_PF_LAUNCHER(2)
KVARN_DECL_PF_LAUNCHER(4)
#undef KVARN_DECL_PF_LAUNCHER

}  // namespace kvarn
