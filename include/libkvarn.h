/* libkvarn -- variance-normalised KV-cache quantisation (KVarN) for AMD MI355X (gfx950).
 *
 * Pages cited below (titles abbreviated):
 *   [HYPHO] blog.hypho.cn, "KV-cache 量化终于能跑生产了？KVarN 用方差归一化打破 vLLM 的吞吐量魔咒"
 *   [LEHUY] lehuy.net, "KVarN: Backend lượng tử hóa KV-cache gốc của Huawei giúp vLLM ..."
 *   [OPENAIHUB] openai-hub.net/news/593, "Huawei Cloud open-sources KVarN ..."
 *
 * The method (four stages per fixed token tile, [HYPHO] section "它怎么做到的：四步流水线",
 * [LEHUY] section "Cơ chế hoạt động: Chuẩn hóa phương sai"):
 *   1. take a raw fp16 K or V tile of 128 tokens x 128 channels,
 *   2. rotate every token along channels with the orthonormal Hadamard matrix Hn = H_128/sqrt(128),
 *   3. balance row (token) and column (channel) RMS by alternating Sinkhorn-style passes in
 *      log space (8 iterations, channels first),
 *   4. quantise each token's channels with asymmetric round-to-nearest at b bits, in groups of
 *      g contiguous (rotated) channels (keys 4 bits, values 2 bits, g = 128 by default:
 *      "kvarn_k4v2_g128"; g = 64 and 32 split a token into 2 or 4 groups), keeping the scales so
 *      that they can be folded back in when attention reads the cache.
 * The page size equals the tile size and must be 128 ([HYPHO] section "需要关注的几个问题", item 3).
 *
 * Conventions for every call:
 *   - Ownership: the caller owns and allocates every buffer (cache pool, tails, page table,
 *     lengths, workspace, outputs).  The library allocates nothing and keeps no per-call state;
 *     calls on different streams are independent.
 *   - Pointers marked (device) are device addresses; the call only enqueues work on `stream`
 *     and returns at once.  The host never reads device memory.
 *   - Errors detectable on the host (null pointer, unsupported format, bad sizes, workspace too
 *     small) return a status and launch nothing.  A failed launch returns KVARN_E_HIP.
 *     Device-side preconditions (valid page ids, pages allocated before a tile fills) are
 *     documented, not checked.
 *
 * Record layout (one record per (page, kv head), this library's own format; the pages fix
 * none of it).  T = 128 tokens, D = 128 channels, kb / vb = key / value bits:
 *   [0, 16*T*kb)            K codes, token-major.  Token t owns 16*kb bytes at t*16*kb.  Unit u
 *                           (0..15) of kb bytes at u*kb holds the codes of channels u + 16*e,
 *                           e = 0..7, code e at bit kb*e of the little-endian unit.
 *   [16*T*kb, +16*T*vb)     V codes.  Unit size U = 2*vb bytes (16 codes).  Unit
 *                           (nb, gr, nl, half) at ((nb*4 + gr)*16 + nl)*2*U + half*U holds channel
 *                           j = 16*nb + nl for tokens t = 64*half + 16*mb + 4*gr + i (mb, i = 0..3),
 *                           the code of (mb, i) at bit vb*(4*mb + i).
 *   then the scales, float32: the K half then the V half, each c[128], s'[ng][128], m'[ng][128]
 *                           with ng = 128 / g groups per token (group gi of token t at [gi][t]);
 *                           for g = 128 these are six float32[128]: c_K, s'_K, m'_K, c_V, s'_V, m'_V.
 * For a token t of one half, with Y = X Hn, log-scales (u, v) from step 3 and the statistics
 * mn_{t,gi}, s_{t,gi} of group gi of Z_t = Y_t exp(-u_t - v):  c_j = exp(v_j),
 * s'_{t,gi} = exp(u_t) s_{t,gi},  m'_{t,gi} = exp(u_t) mn_{t,gi}, and the value read back is
 * xhat_t = Hn yhat_t with yhat_tj = c_j (m'_{t,g(j)} + s'_{t,g(j)} q_tj), g(j) = j / g.
 * Record size: 15360 bytes for k4v2 g128, 17408 for g64, 21504 for g32; 35840 for k8v8 g128
 * (vs 65536 for fp16 K+V: 4.27x capacity for k4v2 g128).
 */
#ifndef LIBKVARN_H_
#define LIBKVARN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVARN_OK = 0,
  KVARN_E_INVALID_ARG = 1, /* null pointer, negative size, inconsistent sizes */
  KVARN_E_UNSUPPORTED = 2, /* a format, block size, head size or GQA ratio this library does not run */
  KVARN_E_HIP = 3,         /* a HIP launch or runtime call failed */
  KVARN_E_SCRATCH_LIMIT = 4, /* kvarn_decode_attention_noalloc: the call needs more workspace than its
                                fixed scratch holds (kvarn_decode_noalloc_max_workspace_bytes) */
  KVARN_E_OUT_OF_PAGES = 5   /* kvarn_page_pool_reserve: the pool has fewer free pages than the batch needs */
} kvarn_status;

/* kv-cache dtype string "kvarn_k{K}v{V}_g{G}" ([HYPHO] section "工程实践：一行配置启用";
 * [LEHUY] section "Dễ dàng tích hợp và sử dụng").  head_dim and block_size are 128; sinkhorn_iters
 * is 8 (one iteration = one channel pass + one token pass). */
typedef struct {
  int32_t k_bits, v_bits, group, head_dim, block_size, sinkhorn_iters;
} kvarn_format;

/* Parse a dtype string.  "kvarn_k4v2_g128" -> {4, 2, 128, 128, 128, 8}.  Bits must be 2, 4 or 8 and
 * the group 128, 64 or 32 (else KVARN_E_UNSUPPORTED); malformed strings KVARN_E_INVALID_ARG. */
kvarn_status kvarn_format_parse(const char* name, kvarn_format* out);

/* Check a format struct filled by hand: same rules as kvarn_format_parse, plus head_dim and
 * block_size 128 and 0 <= sinkhorn_iters <= 64. */
kvarn_status kvarn_format_check(const kvarn_format* f);

/* Bytes of one record (one page of one kv head); 0 if the format is invalid. */
size_t kvarn_record_bytes(const kvarn_format* f);

/* Workspace bytes kvarn_decode_attention needs for these sizes: the split-K partial results, per
 * (sequence, query head, split) 128 per-channel sums, a running max, a running sum and two pad floats
 * (528 bytes), for the fp16-tail splits and for every page split.  There is one page split per 4 groups
 * of pages (a group being 2 pages, or 1 for 16 query heads per kv head, 8-bit codes or groups below 128
 * channels) of the longest possible sequence, and 1 tail split, or 8 (16 tail tokens each) where
 * num_seqs * num_kv_heads * page splits is below 1024.  The split counts depend on the page table's
 * width max_pages_per_seq and on the number of (sequence, kv head) pairs, which is why those are
 * arguments (rather than a maximum context length).  0 for an unsupported format or shape. */
size_t kvarn_decode_workspace_bytes(const kvarn_format* f, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t max_pages_per_seq);

/* Bulk tile quantisation (prefill): stages 1-4 on num_tiles x num_kv_heads tiles.
 *   k, v       (device) fp16 [num_tiles][128 tokens][num_kv_heads][head_dim]
 *   dst_pages  (device) int32 [num_tiles]: physical page of each tile
 *   cache      (device) pool; tile i of head h is written at
 *              cache + dst_pages[i]*page_stride_bytes + h*kvarn_record_bytes(f)
 *   page_stride_bytes >= num_kv_heads*record_bytes and a multiple of 16.
 * Each tile's record depends only on that tile's K and V (no calibration, [HYPHO] section
 * "KVarN 是什么"). */
kvarn_status kvarn_quantize_tiles(const kvarn_format* f, int32_t num_tiles, int32_t num_kv_heads,
                                  const void* k, const void* v, const int32_t* dst_pages, void* cache,
                                  int64_t page_stride_bytes, hipStream_t stream);

/* Append one token per sequence (decode step).  With len = seq_lens[s] before the call:
 * tail_k/v[s][h][len % 128] <- k_new/v_new[s][h] (raw fp16); if (len + 1) % 128 == 0 the whole
 * tail tile of every head is quantised into page page_table[s*max_pages_per_seq + len/128];
 * finally seq_lens[s] = len + 1.
 *   k_new, v_new  (device) fp16 [num_seqs][num_kv_heads][head_dim]
 *   seq_lens      (device) int32 [num_seqs], read then incremented
 *   tail_k/tail_v (device) fp16 [num_seqs][num_kv_heads][128][head_dim]
 *   page_table    (device) int32 [num_seqs][max_pages_per_seq]
 * The page for a filling tile must be allocated in page_table before the call
 * (kvarn_page_pool_reserve for the length after the call does that).
 * The pages fix the per-tile quantiser but not when a decode step's new token is quantised; keeping
 * a tile's newest tokens in fp16 and quantising the tile once its 128th token arrives (so every
 * record is a whole tile, as the bulk path writes it) is this library's reading.
 * One launch reads and advances the lengths: while it runs, seq_lens[s] holds the number of kv
 * heads already appended in its bits 24 and up, so lengths must stay below 2^24 tokens, at most
 * 64 kv heads are supported (more return KVARN_E_UNSUPPORTED), and nothing else may read seq_lens
 * until the call's work has completed (calls on one stream are ordered). */
kvarn_status kvarn_append_token(const kvarn_format* f, int32_t num_seqs, int32_t num_kv_heads,
                                const void* k_new, const void* v_new, int32_t* seq_lens, void* tail_k,
                                void* tail_v, const int32_t* page_table, int32_t max_pages_per_seq,
                                void* cache, int64_t page_stride_bytes, hipStream_t stream);

/* Decode attention over the quantised cache (every step reads all cached tokens, [HYPHO] section
 * "论文的核心发现：推理场景的误差累积"), with the scales folded in on read ([LEHUY] section
 * "Cơ chế hoạt động", stage 4): channel scales into the rotated query, token scales into the
 * logits and the softmax weights, the inverse rotation applied once to the output.
 * For sequence s with L = seq_lens[s] tokens: full pages 0 .. L/128-1 come from the cache, the
 * L % 128 newest tokens from the fp16 tail.  Query head hq uses kv head hq / (Hq/Hkv).
 *   out[s][hq] = softmax(sm_scale * q . K^T) V  (fp16; all zeros when L = 0)
 *   q, out     (device) fp16 [num_seqs][num_q_heads][head_dim]
 *   page_table (device) int32 [num_seqs][max_pages_per_seq]; seq_lens (device) int32 [num_seqs]
 *              with seq_lens[s] < 128*(max_pages_per_seq + 1); max_pages_per_seq sizes the
 *              split-K grid and the workspace
 *   workspace  (device) >= kvarn_decode_workspace_bytes(...) bytes, 16-byte aligned, owned by the
 *              caller.  The call's first kernel writes the split partials there and its second kernel
 *              merges them, so its contents before and after a call do not matter (no initialisation);
 *              calls that may run at the same time (different streams) need separate workspaces.
 * Supported query heads per kv head: 1, 2, 4, 8 and 16. */
kvarn_status kvarn_decode_attention(const kvarn_format* f, int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, const void* q, const void* cache,
                                    int64_t page_stride_bytes, const int32_t* page_table,
                                    int32_t max_pages_per_seq, const int32_t* seq_lens,
                                    const void* tail_k, const void* tail_v,
                                    float sm_scale, void* out, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* kvarn_decode_attention without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The split
 * partials go to a fixed array of kvarn_decode_noalloc_max_workspace_bytes() bytes (64 MiB) that the
 * library holds on each GPU it runs on until the process ends; the call allocates nothing and takes
 * that array's address once per device (with the device current) on its first call there.
 * Arguments and results as for kvarn_decode_attention.  A call whose
 * kvarn_decode_workspace_bytes(...) exceeds the array returns KVARN_E_SCRATCH_LIMIT and launches
 * nothing.  Every call on one GPU shares the array: calls that may overlap on one GPU (different
 * streams, or different host threads without ordering) race and must not be issued; calls on one
 * stream are ordered and safe.  The array holds nothing between calls (no initialisation needed). */
kvarn_status kvarn_decode_attention_noalloc(const kvarn_format* f, int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, const void* q, const void* cache,
                                            int64_t page_stride_bytes, const int32_t* page_table,
                                            int32_t max_pages_per_seq, const int32_t* seq_lens,
                                            const void* tail_k, const void* tail_v, float sm_scale, void* out,
                                            hipStream_t stream);

/* Bytes of the fixed scratch array of kvarn_decode_attention_noalloc (64 MiB). */
size_t kvarn_decode_noalloc_max_workspace_bytes(void);

/* Chunked prefill attention over the quantised cache: many queries per kv head at once, the phase
 * before decoding ([HYPHO] section "它怎么做到的：四步流水线" for the cache it reads; scales folded
 * in on read as for decode, [LEHUY] section "Cơ chế hoạt động", stage 4).
 * Sequence s holds L = seq_lens[s] tokens (full pages from the cache, the L % 128 newest from the
 * fp16 tail, as for decode), the last n = q_lens[s] of which are this chunk's queries; their keys
 * and values must already be in the cache / tail (appended before the call).  Query i < n sits at
 * position L - n + i and attends causally to positions 0 .. L - n + i:
 *   out[s][i][hq] = softmax_{t <= L-n+i}(sm_scale * q[s][i][hq] . k_t) V   (fp16)
 *   q, out    (device) fp16 [num_seqs][max_q][num_q_heads][head_dim]; rows i >= q_lens[s] of out
 *             are not written
 *   q_lens    (device) int32 [num_seqs], 0 <= q_lens[s] <= min(max_q, seq_lens[s]) (larger values
 *             are clamped to that)
 *   page_table, seq_lens, tail_k, tail_v as for decode.
 * No workspace.  Supported: one quantisation group per token (g128), query heads per kv head
 * 1, 2, 4, 8 or 16; other formats return KVARN_E_UNSUPPORTED. */
kvarn_status kvarn_prefill_attention(const kvarn_format* f, int32_t num_seqs, int32_t max_q,
                                     int32_t num_q_heads, int32_t num_kv_heads, const void* q,
                                     const int32_t* q_lens, const void* cache, int64_t page_stride_bytes,
                                     const int32_t* page_table, int32_t max_pages_per_seq,
                                     const int32_t* seq_lens, const void* tail_k, const void* tail_v,
                                     float sm_scale, void* out, hipStream_t stream);

/* Host-side page pool for the paged cache (block_size 128, [HYPHO] section "工程实践：一行配置启用";
 * [LEHUY] section "Dễ dàng tích hợp và sử dụng").  It hands out physical page ids 0 .. num_pages-1 of
 * the caller's cache pool (page_stride_bytes each) and fills the host copy of the page table that the
 * caller then uploads; it touches no device memory and makes no HIP call.  A sequence of length L
 * needs pages for its full tiles 0 .. L/128 - 1 only (the L % 128 newest tokens are in the fp16 tail).
 * Calls on one pool may come from several host threads (each call holds the pool's lock). */
typedef struct kvarn_page_pool kvarn_page_pool;

/* New pool of num_pages free pages (num_pages >= 0); *pool receives it.  KVARN_E_INVALID_ARG for a null
 * out pointer, a negative count or a failed host allocation. */
kvarn_status kvarn_page_pool_create(int32_t num_pages, kvarn_page_pool** pool);

/* Free the pool (null is ignored).  Page tables filled from it keep their ids. */
void kvarn_page_pool_destroy(kvarn_page_pool* pool);

/* Free pages left; -1 for a null pool. */
int32_t kvarn_page_pool_num_free(kvarn_page_pool* pool);

/* Give every sequence of a batch the pages its new length needs.  For each s, the row
 * page_table[s*max_pages_per_seq ...] (host) holds num_owned[s] (host, in/out) pages owned by the
 * sequence in entries 0 .. num_owned[s]-1; entries num_owned[s] .. new_lens[s]/128 - 1 receive new
 * pages and num_owned[s] becomes new_lens[s]/128 when that is larger (a shorter length keeps its
 * pages).  All or nothing: on KVARN_E_OUT_OF_PAGES (too few free pages for the whole batch) or
 * KVARN_E_INVALID_ARG (negative sizes, num_owned[s] > max_pages_per_seq, new_lens[s]/128 >
 * max_pages_per_seq) nothing changes.  For decode steps replayed without returning to the host (a
 * captured graph), reserve for the length after the last replayed step. */
kvarn_status kvarn_page_pool_reserve(kvarn_page_pool* pool, int32_t num_seqs, const int32_t* new_lens,
                                     int32_t* page_table, int32_t max_pages_per_seq, int32_t* num_owned);

/* Return the *num_owned pages of one sequence's row (host) to the pool, set those entries to -1 and
 * *num_owned to 0.  KVARN_E_INVALID_ARG, changing nothing, if an entry is not a page this pool handed
 * out and has not taken back, or appears twice. */
kvarn_status kvarn_page_pool_release(kvarn_page_pool* pool, int32_t* page_table_row, int32_t max_pages_per_seq,
                                     int32_t* num_owned);

/* Human-readable name of a status value (any int: values that are no kvarn_status give "unknown status"). */
const char* kvarn_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* LIBKVARN_H_ */
