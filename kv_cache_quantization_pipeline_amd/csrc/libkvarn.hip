// libkvarn C-ABI: argument validation and kernel launches (see include/libkvarn.h).
#include "../../include/libkvarn.h"

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "kvarn_device.h"
#include "kvarn_internal.h"

namespace {

bool bits_ok(int b) { return b == 2 || b == 4 || b == 8; }

kvarn_status check_format(const kvarn_format* f) {
  if (f == nullptr) return KVARN_E_INVALID_ARG;
  if (!bits_ok(f->k_bits) || !bits_ok(f->v_bits)) return KVARN_E_UNSUPPORTED;
  if (f->head_dim != 128 || f->block_size != 128) return KVARN_E_UNSUPPORTED;
  if (f->group != 128 && f->group != 64 && f->group != 32) return KVARN_E_UNSUPPORTED;
  if (f->sinkhorn_iters < 0 || f->sinkhorn_iters > 64) return KVARN_E_INVALID_ARG;
  return KVARN_OK;
}

// parse a decimal integer at *p, advancing p; false if none
bool parse_int(const char*& p, int* out) {
  if (*p < '0' || *p > '9') return false;
  long v = 0;
  while (*p >= '0' && *p <= '9') {
    v = v * 10 + (*p - '0');
    if (v > 1000000) return false;
    ++p;
  }
  *out = static_cast<int>(v);
  return true;
}

kvarn_status hip_status(hipError_t e) { return e == hipSuccess ? KVARN_OK : KVARN_E_HIP; }

// quantisation groups per token
int n_groups(const kvarn_format* f) { return 128 / f->group; }

int64_t record_bytes(const kvarn_format* f) { return kvarn::record_bytes(f->k_bits, f->v_bits, n_groups(f)); }

// Fixed decode workspace of kvarn_decode_attention_noalloc: one copy per GPU, held until the process
// ends.  In host code `scratch` only names the symbol; its device address on the current GPU comes
// from hipGetSymbolAddress, taken once per device and kept in scratch_ptr.
constexpr int kMaxDevices = 256;
static __device__ __align__(256) float scratch[(64u << 20) / sizeof(float)];
std::atomic<void*> scratch_ptr[kMaxDevices];

kvarn_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVARN_E_HIP;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // with device `dev` current: the address of that device's copy of the array
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return KVARN_E_HIP;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return KVARN_OK;
}

// Argument checks shared by both decode entry points (everything but the workspace).
kvarn_status decode_check(const kvarn_format* f, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          const void* q, const void* cache, int64_t page_stride_bytes, const int32_t* page_table,
                          int32_t max_pages_per_seq, const int32_t* seq_lens, const void* tail_k, const void* tail_v,
                          const void* out) {
  const kvarn_status st = check_format(f);
  if (st != KVARN_OK) return st;
  if (num_seqs < 0 || num_kv_heads <= 0 || num_q_heads <= 0 || max_pages_per_seq < 0) return KVARN_E_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return KVARN_E_INVALID_ARG;
  const int G = num_q_heads / num_kv_heads;
  if (!kvarn::decode_supported(f->k_bits, f->v_bits, n_groups(f), G)) return KVARN_E_UNSUPPORTED;
  if (num_seqs == 0) return KVARN_OK;
  if (q == nullptr || cache == nullptr || page_table == nullptr || seq_lens == nullptr || tail_k == nullptr ||
      tail_v == nullptr || out == nullptr)
    return KVARN_E_INVALID_ARG;
  const int64_t R = record_bytes(f);
  if (page_stride_bytes < R * num_kv_heads || page_stride_bytes % 16 != 0) return KVARN_E_INVALID_ARG;
  if (static_cast<int64_t>(num_seqs) * num_kv_heads > 0x7fffffffLL) return KVARN_E_INVALID_ARG;
  const kvarn::DecodePlan plan =
      kvarn::plan_decode(f->k_bits, f->v_bits, n_groups(f), num_seqs, num_kv_heads, G, max_pages_per_seq);
  if (plan.tail_splits + plan.page_splits > 65535) return KVARN_E_UNSUPPORTED;
  if (static_cast<int64_t>(num_seqs) * num_q_heads > 0x7fffffffLL) return KVARN_E_INVALID_ARG;
  return KVARN_OK;
}

kvarn_status decode_launch(const kvarn_format* f, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           const void* q, const void* cache, int64_t page_stride_bytes, const int32_t* page_table,
                           int32_t max_pages_per_seq, const int32_t* seq_lens, const void* tail_k, const void* tail_v,
                           float sm_scale, void* out, void* workspace, hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  const kvarn::DecodePlan plan =
      kvarn::plan_decode(f->k_bits, f->v_bits, n_groups(f), num_seqs, num_kv_heads, G, max_pages_per_seq);
  return hip_status(kvarn::launch_decode(f->k_bits, f->v_bits, n_groups(f), G, static_cast<const _Float16*>(q),
                                         static_cast<const uint8_t*>(cache), page_stride_bytes, page_table,
                                         max_pages_per_seq, seq_lens, static_cast<const _Float16*>(tail_k),
                                         static_cast<const _Float16*>(tail_v), sm_scale, static_cast<_Float16*>(out),
                                         kvarn::decode_workspace_layout(workspace, plan, num_seqs, num_q_heads,
                                                                        num_kv_heads),
                                         num_seqs, num_q_heads, num_kv_heads, plan, stream));
}

}  // namespace

extern "C" {

kvarn_status kvarn_format_parse(const char* name, kvarn_format* out) {
  if (name == nullptr || out == nullptr) return KVARN_E_INVALID_ARG;
  const char* p = name;
  const char* prefix = "kvarn_k";
  if (std::strncmp(p, prefix, std::strlen(prefix)) != 0) return KVARN_E_INVALID_ARG;
  p += std::strlen(prefix);
  int kb, vb, g;
  if (!parse_int(p, &kb)) return KVARN_E_INVALID_ARG;
  if (*p++ != 'v') return KVARN_E_INVALID_ARG;
  if (!parse_int(p, &vb)) return KVARN_E_INVALID_ARG;
  if (*p++ != '_' || *p++ != 'g') return KVARN_E_INVALID_ARG;
  if (!parse_int(p, &g)) return KVARN_E_INVALID_ARG;
  if (*p != '\0') return KVARN_E_INVALID_ARG;
  kvarn_format f{kb, vb, g, 128, 128, 8};
  const kvarn_status st = check_format(&f);
  if (st != KVARN_OK) return st;
  *out = f;
  return KVARN_OK;
}

kvarn_status kvarn_format_check(const kvarn_format* f) { return check_format(f); }

size_t kvarn_record_bytes(const kvarn_format* f) {
  if (check_format(f) != KVARN_OK) return 0;
  return static_cast<size_t>(record_bytes(f));
}

size_t kvarn_decode_workspace_bytes(const kvarn_format* f, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t max_pages_per_seq) {
  if (check_format(f) != KVARN_OK || num_seqs < 0 || num_kv_heads <= 0 || num_q_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || max_pages_per_seq < 0)
    return 0;
  const int G = num_q_heads / num_kv_heads;
  if (!kvarn::decode_supported(f->k_bits, f->v_bits, n_groups(f), G)) return 0;
  const kvarn::DecodePlan plan =
      kvarn::plan_decode(f->k_bits, f->v_bits, n_groups(f), num_seqs, num_kv_heads, G, max_pages_per_seq);
  return kvarn::decode_workspace_bytes(plan, num_seqs, num_q_heads, num_kv_heads);
}

kvarn_status kvarn_quantize_tiles(const kvarn_format* f, int32_t num_tiles, int32_t num_kv_heads, const void* k,
                                  const void* v, const int32_t* dst_pages, void* cache, int64_t page_stride_bytes,
                                  hipStream_t stream) {
  const kvarn_status st = check_format(f);
  if (st != KVARN_OK) return st;
  if (num_tiles < 0 || num_kv_heads <= 0) return KVARN_E_INVALID_ARG;
  if (num_tiles == 0) return KVARN_OK;
  if (k == nullptr || v == nullptr || dst_pages == nullptr || cache == nullptr) return KVARN_E_INVALID_ARG;
  const int64_t R = record_bytes(f);
  if (page_stride_bytes < R * num_kv_heads || page_stride_bytes % 16 != 0) return KVARN_E_INVALID_ARG;
  if (static_cast<int64_t>(num_tiles) * num_kv_heads > 0x3fffffffLL) return KVARN_E_INVALID_ARG;  // 2 WGs each
  return hip_status(kvarn::launch_quantize_tiles(static_cast<const _Float16*>(k), static_cast<const _Float16*>(v),
                                                 dst_pages, static_cast<uint8_t*>(cache), page_stride_bytes, num_tiles,
                                                 num_kv_heads, f->k_bits, f->v_bits, n_groups(f), f->sinkhorn_iters,
                                                 stream));
}

kvarn_status kvarn_append_token(const kvarn_format* f, int32_t num_seqs, int32_t num_kv_heads, const void* k_new,
                                const void* v_new, int32_t* seq_lens, void* tail_k, void* tail_v,
                                const int32_t* page_table, int32_t max_pages_per_seq, void* cache,
                                int64_t page_stride_bytes, hipStream_t stream) {
  const kvarn_status st = check_format(f);
  if (st != KVARN_OK) return st;
  if (num_seqs < 0 || num_kv_heads <= 0 || max_pages_per_seq <= 0) return KVARN_E_INVALID_ARG;
  if (num_kv_heads > kvarn::kMaxAppendKvHeads) return KVARN_E_UNSUPPORTED;
  if (num_seqs == 0) return KVARN_OK;
  if (k_new == nullptr || v_new == nullptr || seq_lens == nullptr || tail_k == nullptr || tail_v == nullptr ||
      page_table == nullptr || cache == nullptr)
    return KVARN_E_INVALID_ARG;
  const int64_t R = record_bytes(f);
  if (page_stride_bytes < R * num_kv_heads || page_stride_bytes % 16 != 0) return KVARN_E_INVALID_ARG;
  if (static_cast<int64_t>(num_seqs) * num_kv_heads > 0x7fffffffLL) return KVARN_E_INVALID_ARG;
  return hip_status(kvarn::launch_append(
      static_cast<const _Float16*>(k_new), static_cast<const _Float16*>(v_new), seq_lens,
      static_cast<_Float16*>(tail_k), static_cast<_Float16*>(tail_v), page_table, max_pages_per_seq,
      static_cast<uint8_t*>(cache), page_stride_bytes, num_seqs, num_kv_heads, f->k_bits, f->v_bits, n_groups(f),
      f->sinkhorn_iters, stream));
}

kvarn_status kvarn_decode_attention(const kvarn_format* f, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, const void* q, const void* cache, int64_t page_stride_bytes,
                                    const int32_t* page_table, int32_t max_pages_per_seq, const int32_t* seq_lens,
                                    const void* tail_k, const void* tail_v, float sm_scale, void* out,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const kvarn_status st = decode_check(f, num_seqs, num_q_heads, num_kv_heads, q, cache, page_stride_bytes,
                                       page_table, max_pages_per_seq, seq_lens, tail_k, tail_v, out);
  if (st != KVARN_OK || num_seqs == 0) return st;
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return KVARN_E_INVALID_ARG;
  if (workspace_bytes < kvarn_decode_workspace_bytes(f, num_seqs, num_q_heads, num_kv_heads, max_pages_per_seq))
    return KVARN_E_INVALID_ARG;
  return decode_launch(f, num_seqs, num_q_heads, num_kv_heads, q, cache, page_stride_bytes, page_table,
                       max_pages_per_seq, seq_lens, tail_k, tail_v, sm_scale, out, workspace, stream);
}

kvarn_status kvarn_decode_attention_noalloc(const kvarn_format* f, int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, const void* q, const void* cache,
                                            int64_t page_stride_bytes, const int32_t* page_table,
                                            int32_t max_pages_per_seq, const int32_t* seq_lens, const void* tail_k,
                                            const void* tail_v, float sm_scale, void* out, hipStream_t stream) {
  const kvarn_status st = decode_check(f, num_seqs, num_q_heads, num_kv_heads, q, cache, page_stride_bytes,
                                       page_table, max_pages_per_seq, seq_lens, tail_k, tail_v, out);
  if (st != KVARN_OK || num_seqs == 0) return st;
  if (kvarn_decode_workspace_bytes(f, num_seqs, num_q_heads, num_kv_heads, max_pages_per_seq) > sizeof(scratch))
    return KVARN_E_SCRATCH_LIMIT;
  void* ws = nullptr;
  const kvarn_status sst = scratch_address(&ws);
  if (sst != KVARN_OK) return sst;
  return decode_launch(f, num_seqs, num_q_heads, num_kv_heads, q, cache, page_stride_bytes, page_table,
                       max_pages_per_seq, seq_lens, tail_k, tail_v, sm_scale, out, ws, stream);
}

size_t kvarn_decode_noalloc_max_workspace_bytes(void) { return sizeof(scratch); }

kvarn_status kvarn_prefill_attention(const kvarn_format* f, int32_t num_seqs, int32_t max_q, int32_t num_q_heads,
                                     int32_t num_kv_heads, const void* q, const int32_t* q_lens, const void* cache,
                                     int64_t page_stride_bytes, const int32_t* page_table, int32_t max_pages_per_seq,
                                     const int32_t* seq_lens, const void* tail_k, const void* tail_v, float sm_scale,
                                     void* out, hipStream_t stream) {
  const kvarn_status st = check_format(f);
  if (st != KVARN_OK) return st;
  if (num_seqs < 0 || max_q < 0 || num_kv_heads <= 0 || num_q_heads <= 0 || max_pages_per_seq < 0)
    return KVARN_E_INVALID_ARG;
  if (num_q_heads % num_kv_heads != 0) return KVARN_E_INVALID_ARG;
  const int G = num_q_heads / num_kv_heads;
  if (!kvarn::prefill_supported(f->k_bits, f->v_bits, n_groups(f), G)) return KVARN_E_UNSUPPORTED;
  if (num_seqs == 0 || max_q == 0) return KVARN_OK;
  if (q == nullptr || q_lens == nullptr || cache == nullptr || page_table == nullptr || seq_lens == nullptr ||
      tail_k == nullptr || tail_v == nullptr || out == nullptr)
    return KVARN_E_INVALID_ARG;
  const int64_t R = record_bytes(f);
  if (page_stride_bytes < R * num_kv_heads || page_stride_bytes % 16 != 0) return KVARN_E_INVALID_ARG;
  if (static_cast<int64_t>(num_seqs) * num_kv_heads > 0x7fffffffLL) return KVARN_E_INVALID_ARG;
  if (kvarn::prefill_row_blocks(max_q, G) > 65535) return KVARN_E_UNSUPPORTED;
  return hip_status(kvarn::launch_prefill(f->k_bits, f->v_bits, n_groups(f), G, static_cast<const _Float16*>(q), q_lens,
                                          max_q,
                                          static_cast<const uint8_t*>(cache), page_stride_bytes, page_table,
                                          max_pages_per_seq, seq_lens, static_cast<const _Float16*>(tail_k),
                                          static_cast<const _Float16*>(tail_v), sm_scale, static_cast<_Float16*>(out),
                                          num_seqs, num_q_heads, num_kv_heads, stream));
}

const char* kvarn_status_string(int32_t status) {
  switch (status) {
    case KVARN_OK:
      return "ok";
    case KVARN_E_INVALID_ARG:
      return "invalid argument";
    case KVARN_E_UNSUPPORTED:
      return "unsupported";
    case KVARN_E_HIP:
      return "HIP error";
    case KVARN_E_SCRATCH_LIMIT:
      return "needs more workspace than the fixed scratch of the no-allocation entry point";
    case KVARN_E_OUT_OF_PAGES:
      return "page pool has too few free pages";
  }
  return "unknown status";
}

}  // extern "C"
