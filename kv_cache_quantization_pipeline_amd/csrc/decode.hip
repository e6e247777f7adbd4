// KVarN decode attention over the packed cache, for gfx950.
//
// Scales are folded in on read ([LEHUY] section "Cơ chế hoạt động", stage 4;
// [HYPHO] section "它怎么做到的：四步流水线", step 4).  With the record of one
// page, xhat_t = Hn (c ⊙ (m'_t + s'_t q_t)) and Hn symmetric:
//   q . khat_t = s'_t (q'' . q_t) + m'_t sigma,   q' = Hn q, q'' = c_K ⊙ q', sigma = sum_j q''_j
//   sum_t p_t vhat_t = Hn ( c_V ⊙ ( sum_t (p_t s'_t) q_t + sum_t p_t m'_t ) )
// so channel scales go into the rotated query, token scales into the logits and
// the softmax weights, and Hn is applied once, to the merged output.  Logits are kept in the log2 domain (q' is pre-scaled by
// sm_scale * log2 e) so the softmax uses exp2.
//
// Work split: grid (sequence * kv head, split), 4 waves per workgroup, each wave
// a run of page groups.  A group is P = 16/G pages (G query heads per kv head)
// so that the 16 MFMA columns are all used: for QK the A operand is the codes
// of token rows (16 per M block), K runs over (page, channel) and the B
// operand is block-diagonal (lane column n = (page e, head g) holds q''_e,g for
// page e's k-steps, zero elsewhere); for PV the A operand is the weights
// (row (e, g), K over (page, token)), the B operand the V codes.  Codes become
// exact fp16 integers in registers (4-bit: bytes read as fp8 e4m3, scaled by 2^9;
// 2-bit: nibbles read as fp4 e2m1, scaled by 2; 8-bit: 0x6400 | byte minus
// 1024).  Each wave keeps one
// running (max, sum, acc) per MFMA row, i.e. per (page parity, head); the
// workgroup merges its 4 waves x P streams in LDS and writes one split-K
// partial per query head.
//
// The fp16 tail (the len % 128 newest tokens) goes to the first splits of a (sequence, kv head):
// four tail-only splits where the grid has room for them, else a share of every page split; it
// enters raw-domain sums of their partials.  The workgroups of a pair count their arrivals
// on a device-scope counter in the workspace; the last one to arrive merges the partials and
// applies the inverse rotation (combine_head), one wave per query head.

#include <algorithm>

#include "kvarn_codes.h"
#include "kvarn_device.h"
#include "kvarn_internal.h"

// This file is compiled once per number of quantisation groups per token: KVARN_DECODE_NG = 1 (the
// default; also holds the host-side planning and dispatch), 2 or 4.  Each object holds the kernels
// of its group count, with internal linkage, and one launcher for them.
#ifndef KVARN_DECODE_NG
#define KVARN_DECODE_NG 1
#endif

namespace kvarn {

namespace {


// Stores and loads of the split-K partials that are coherent across the device (the L2 caches of
// all XCDs) on their own: relaxed atomics at agent scope.  No cache-wide write-back or
// invalidation is needed around the arrival counter then.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float2 load_agent2(const float* p) {
  return __builtin_bit_cast(float2, __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT));
}

// Sum over the 64 lanes of x[t] for 16 values t per lane, transposed: lane l returns the sum for
// t = l & 15 (four exchange-and-add steps that halve the values a lane keeps, then lanes l ^ 16 and
// l ^ 32).
__device__ __forceinline__ float transpose_sum16(float (&x)[16], int lane) {
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1) {
    const bool up = lane & w;
#pragma unroll
    for (int i = 0; i < w; ++i) {
      const float keep = up ? x[w + i] : x[i];
      const float send = up ? x[i] : x[w + i];
      x[i] = keep + __shfl_xor(send, w);
    }
  }
  const float y = x[0] + __shfl_xor(x[0], 16);
  return y + __shfl_xor(y, 32);
}

// Attention over the fp16 tail (raw domain) for the HW query heads g0, g0 + 4, ... (those below G) of
// one wave, over n >= 1 tail tokens t0 .. t0+n-1 (n <= 128) of their kv head.  Lane l owns channels
// 2l, 2l + 1: it reads those two channels of every key and value row (coalesced 256-byte rows) and
// of each query row, so a head's query costs two registers; the logits are summed across lanes 16
// tokens at a time (token t of a chunk ends in lanes t, t + 16, t + 32, t + 48).  Rows past the last
// token are clamped to it (in bounds) and masked.  Per head: mt = max_t lg_t (log2 units;
// lg = q . k * sm_log2e), lt = sum_t exp2(lg_t - mt), raw = sum_t exp2(lg_t - mt) v_t in the lane's
// two channels.
template <int HW, int G>
__device__ __forceinline__ void tail_heads(const _Float16* __restrict__ q0, int g0, const _Float16* __restrict__ tk,
                                           const _Float16* __restrict__ tv, int t0, int n, float sm_log2e,
                                           float (&mt)[HW], float (&lt)[HW], float (&raw)[HW][2], int lane) {
  constexpr int C = 16;  // tokens per chunk
  float qx[HW], qy[HW], m[HW];
#pragma unroll
  for (int hh = 0; hh < HW; ++hh) {
    const int g = min(g0 + 4 * hh, G - 1);
    const f16x2 qq = *reinterpret_cast<const f16x2*>(q0 + g * kCh + 2 * lane);
    qx[hh] = static_cast<float>(qq[0]) * sm_log2e;
    qy[hh] = static_cast<float>(qq[1]) * sm_log2e;
    m[hh] = -INFINITY;
    lt[hh] = 0.f;
    raw[hh][0] = raw[hh][1] = 0.f;
  }
  // online softmax over the chunks: running max m, sum lt and raw sums rescaled when m grows (the
  // planner shares the tail out so that a split's share is usually one chunk)
  for (int c = 0; c < n; c += C) {
    f16x2 kk[C], vv[C];
#pragma unroll
    for (int u = 0; u < C; ++u) {
      const int row = t0 + min(c + u, n - 1);
      kk[u] = *reinterpret_cast<const f16x2*>(tk + row * kCh + 2 * lane);
      vv[u] = *reinterpret_cast<const f16x2*>(tv + row * kCh + 2 * lane);
    }
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
      float x[C];
#pragma unroll
      for (int u = 0; u < C; ++u)
        x[u] = fmaf(qx[hh], static_cast<float>(kk[u][0]), qy[hh] * static_cast<float>(kk[u][1]));
      const float d = transpose_sum16(x, lane);
      const float lg = c + (lane & 15) < n ? d : -INFINITY;
      float cm = lg;
#pragma unroll
      for (int b = 8; b >= 1; b >>= 1) cm = fmaxf(cm, __shfl_xor(cm, b));
      const float mn = fmaxf(m[hh], cm);
      const float scale = m[hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hh] - mn);
      m[hh] = mn;
      const float p = lg != -INFINITY ? __builtin_amdgcn_exp2f(lg - mn) : 0.f;
      float ps = p;
#pragma unroll
      for (int b = 8; b >= 1; b >>= 1) ps += __shfl_xor(ps, b);
      lt[hh] = lt[hh] * scale + ps;
      float w0 = raw[hh][0] * scale, w1 = raw[hh][1] * scale;
#pragma unroll
      for (int u = 0; u < C; ++u) {
        // weight of token c + u: lane u holds it (0 past the last token)
        const float pw = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), u));
        w0 = fmaf(pw, static_cast<float>(vv[u][0]), w0);
        w1 = fmaf(pw, static_cast<float>(vv[u][1]), w1);
      }
      raw[hh][0] = w0;
      raw[hh][1] = w1;
    }
  }
#pragma unroll
  for (int hh = 0; hh < HW; ++hh) mt[hh] = m[hh];
}

// Merge the split-K partials of one (sequence, query head), apply Hn once, normalise and store.
// One wave; lane l owns output channels 2l and 2l + 1.  With M the largest running maximum (log2
// units) over the splits and f_k = exp2(M_k - M):
//   L = sum_k f_k L_k,  rot = sum_k f_k rot_k (rotated domain),  raw = sum_k f_k raw_k (the fp16 tail,
//   raw domain, only in the first n_tail splits, which own tail tokens),  out = (Hn rot + raw) / L,
// all zero for an empty sequence.  part: the n_splits partials of this head.  The split loops are
// unrolled deeply and their loads do not depend on earlier loads, so the rows of many splits are in
// flight at once (a long sequence with few (sequence, kv head) pairs has ~70 splits).
__device__ __forceinline__ void combine_head(const float* __restrict__ part, int n_splits, int n_tail,
                                             _Float16* __restrict__ o, int lane) {
  float M = -INFINITY;
  for (int k = lane; k < n_splits; k += 64) M = fmaxf(M, load_agent(part + k * kPartialFloats));
#pragma unroll
  for (int b = 32; b >= 1; b >>= 1) M = fmaxf(M, __shfl_xor(M, b));

  float L = 0.f, r[2] = {0.f, 0.f}, w[2] = {0.f, 0.f};
  if (M != -INFINITY) {
    // an empty split holds (-inf, 0, 0...): its factor exp2(-inf) is 0.  The first n_tail splits
    // own tail tokens (a split's share is at least one token) and carry raw-domain sums too.
#pragma unroll 8
    for (int k = 0; k < n_tail; ++k) {
      const float* pk = part + k * kPartialFloats;
      const float2 ml = load_agent2(pk);
      const float2 a = load_agent2(pk + 4 + 2 * lane);
      const float2 b = load_agent2(pk + 4 + kCh + 2 * lane);
      const float f = __builtin_amdgcn_exp2f(ml.x - M);
      L = fmaf(ml.y, f, L);
      r[0] = fmaf(a.x, f, r[0]);
      r[1] = fmaf(a.y, f, r[1]);
      w[0] = fmaf(b.x, f, w[0]);
      w[1] = fmaf(b.y, f, w[1]);
    }
#pragma unroll 32
    for (int k = n_tail; k < n_splits; ++k) {
      const float* pk = part + k * kPartialFloats;
      const float2 ml = load_agent2(pk);
      const float2 a = load_agent2(pk + 4 + 2 * lane);
      const float f = __builtin_amdgcn_exp2f(ml.x - M);
      L = fmaf(ml.y, f, L);
      r[0] = fmaf(a.x, f, r[0]);
      r[1] = fmaf(a.y, f, r[1]);
    }
  }
  // Hn over the rotated-domain sum: one stage in registers, six across lanes
  {
    const float a0 = r[0] + r[1], a1 = r[0] - r[1];
    r[0] = a0;
    r[1] = a1;
  }
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const bool upper = (lane >> b) & 1;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float x = __shfl_xor(r[c], 1 << b);
      r[c] = upper ? x - r[c] : r[c] + x;
    }
  }
  const float inv_l = L > 0.f ? 1.0f / L : 0.f;
  constexpr float kInvSqrt128 = 0.08838834764831845f;
  *reinterpret_cast<f16x2*>(o + 2 * lane) =
      f16x2{static_cast<_Float16>((r[0] * kInvSqrt128 + w[0]) * inv_l),
            static_cast<_Float16>((r[1] * kInvSqrt128 + w[1]) * inv_l)};
}

// Pages per wave step P: the 16 MFMA columns are (page, head) pairs.  G = 16 fills them with one
// page; otherwise a step is two pages (the most whose codes fit the registers of two waves per
// SIMD), or one for 8-bit K or V codes, and the columns beyond P*G are masked.
template <int KB, int VB, int G, int NG>
__host__ __device__ constexpr int decode_pages_per_step() {
  return (G >= 16 || NG > 1) ? 1 : ((KB == 8 || VB == 8) ? 1 : 2);
}

template <int KB, int VB, int G, int NG>
__global__ __launch_bounds__(256, 2) void decode_kernel(const _Float16* __restrict__ q, const uint8_t* __restrict__ cache,
                                                        int64_t page_stride, const int32_t* __restrict__ page_table,
                                                        int max_pages, const int32_t* __restrict__ seq_lens,
                                                        int num_q_heads, int num_kv_heads, float qscale,
                                                        float* __restrict__ ws, int* __restrict__ counters,
                                                        int n_splits, int tail_splits,
                                                        const _Float16* __restrict__ tail_k,
                                                        const _Float16* __restrict__ tail_v, float sm_log2e,
                                                        _Float16* __restrict__ out) {
  constexpr int P = decode_pages_per_step<KB, VB, G, NG>();
  constexpr int R = record_bytes(KB, VB, NG);
  constexpr int HS = half_scale_floats(NG);   // floats of one half's scales: c, s'[NG], m'[NG]
  constexpr int SC = 2 * HS;                   // floats of scales per page
  static_assert(NG == 1 || P == 1, "grouped formats take one page per step");
  constexpr int MRG = 130;      // floats per merged row

  __shared__ __attribute__((aligned(16))) float qrot[G][kCh];
  // Per wave, the scales of the current group and of the next one (P pages each): two stages, so
  // that the next group's scales are copied in while this group is computed.  They are separate
  // arrays, so that the compiler tells the copy into one from the reads of the other.  The final
  // merge reuses them (waves 0-1 in the first, 2-3 in the second).
  constexpr int STAGE_FLOATS = 4 * P * SC;
  constexpr int MERGE_HALF = 2 * 16 * MRG;
  constexpr int BUF = STAGE_FLOATS > MERGE_HALF ? STAGE_FLOATS : MERGE_HALF;
  __shared__ __attribute__((aligned(16))) float stage0[BUF];
  __shared__ __attribute__((aligned(16))) float stage1[BUF];

  const int sh = blockIdx.x;
  const int s = sh / num_kv_heads;
  const int h = sh - s * num_kv_heads;
  const int sp = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, gr = lane >> 4;

  const int len = seq_lens[s];
  const int n_pages = len >> 7;
  const int n_groups = (n_pages + P - 1) / P;

  // ---- q' = Hn q * sm_scale * log2(e): 32 threads per head, 4 channels each --------------
  for (int base = 0; base < G * 32; base += 256) {
    const int idx = base + tid;
    if (idx < G * 32) {
      const int g = idx >> 5, r = idx & 31;
      const _Float16* qp = q + (static_cast<int64_t>(s) * num_q_heads + h * G + g) * kCh + 4 * r;
      float x0 = qp[0], x1 = qp[1], x2 = qp[2], x3 = qp[3];
      float a0 = x0 + x1, a1 = x0 - x1, a2 = x2 + x3, a3 = x2 - x3;
      float v[4] = {a0 + a2, a1 + a3, a0 - a2, a1 - a3};
#pragma unroll
      for (int b = 0; b < 5; ++b) {
        const bool upper = (r >> b) & 1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float o = __shfl_xor(v[c], 1 << b, 32);
          v[c] = upper ? o - v[c] : v[c] + o;
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) qrot[g][4 * r + c] = v[c] * qscale;
    }
  }
  __syncthreads();

  // this lane's QK column / PV row n = nl: page e_own of the group, head g_own.  With P*G < 16
  // the columns of pages e_own >= P are unused: zero B operand, masked logits, zero weights.
  const int e_own = nl / G;
  const int g_own = nl - e_own * G;
  const bool col_ok = e_own < P;
  const int e_oc = col_ok ? e_own : 0;
  // page of the PV result row 4*gr + i held by this lane (one page for all four rows when G >= 4)
  // (for G >= 4 the four rows of a lane are one page: only index 0 is used then)
  int e_row[4], e_rc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e_row[i] = G >= 4 ? (4 * gr) / G : (4 * gr + i) / G;
    e_rc[i] = e_row[i] < P ? e_row[i] : 0;
  }

  f16x8 ONES;
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) ONES[sl] = static_cast<_Float16>(1.0f);
  f16x8 C0N;
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) C0N[sl] = static_cast<_Float16>(-0.5f * ((1 << VB) - 1));

  float m_run = -INFINITY;   // column nl (QK layout)
  float l_part = 0.f;        // this lane's tokens only; rows merged at the end
  float acc[8][4];           // PV layout: row 4*gr + i, channel 16*nb + nl
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[nb][i] = 0.f;

  // this sequence's groups split evenly over the page splits of the pair (all n_splits workgroups,
  // or those after the tail_splits tail-only ones; the grid is sized for the longest sequence), then
  // over the 4 waves of each
  const int nps = n_splits - tail_splits;
  const int gps = (n_groups + nps - 1) / nps;
  const int gpw = (gps + 3) / 4;
  // a tail-only split (sp < tail_splits) takes the empty group range [n_groups, n_groups)
  const int base = sp >= tail_splits ? (sp - tail_splits) * gps : n_groups;
  const int s_end = min(base + gps, n_groups);
  const int g_begin = base + wave * gpw;
  const int g_end = min(g_begin + gpw, s_end);
  const int64_t pt_row = static_cast<int64_t>(s) * max_pages;
  const int64_t head_off = static_cast<int64_t>(h) * R;

  // Physical page ids of this wave's groups: one vector load for 64 pages at a time (lane l holds
  // page base * P + l, clamped to the last page: a missing second page of a group is masked),
  // read out with readlane.
  int ids_base = g_begin, ids = 0;
  auto load_ids = [&](int g0) {
    ids_base = g0;
    const int pg = min(g0 * P + lane, n_pages - 1);
    ids = page_table[pt_row + pg];
  };
  auto recs = [&](int gi, const uint8_t* (&rec)[P]) {
    if ((gi - ids_base) * P + P > 64) load_ids(gi);
#pragma unroll
    for (int e = 0; e < P; ++e) {
      const int phys = __builtin_amdgcn_readlane(ids, (gi - ids_base) * P + e);
      rec[e] = cache + static_cast<int64_t>(phys) * page_stride + head_off;
    }
  };

  // One group, software-pipelined over the groups of the wave.  On entry the K codes of token
  // blocks 0-3 (kpre) and the scales (LDS stage sb) are in flight or arrived, issued at the end of
  // the previous group.  The wave issues blocks 4-7, builds the B operand, computes QK, loads the
  // V codes into the registers of the consumed K codes, computes softmax and PV, then issues the
  // next group's blocks 0-3 and copies its scales into the other stage (sb_next).
  auto step = [&](int gi, const KHalf<KB, P>& kpre, KHalf<KB, P>& kpre_next, const float* sb, float* sb_next,
                  const uint8_t* const (&rec)[P], const uint8_t* (&rec_next)[P]) {
    __amdgpu_buffer_rsrc_t rs[P];
#pragma unroll
    for (int e = 0; e < P; ++e) rs[e] = record_rsrc(rec[e], R);
    KHalf<KB, P> khi;
    load_k_half<KB, P>(khi, rs, 1, lane);
    // Vector memory operations complete in order: waiting until only the loads just issued are
    // outstanding means the scale copy into sb (and kpre) issued at the end of the previous group
    // has landed.  The compiler's own tracking of LDS copies does not see it through this loop.
    vmcnt_wait<P * 4 * (KB == 8 ? 2 : 1)>();

    const bool valid_own = col_ok && gi * P + e_own < n_pages;
    const float* sown = sb + e_oc * SC;

    // q'' = c_K ⊙ q' for this lane's page, as the QK B operand, split into fp16 hi + lo parts
    // (q'' = hi + lo to ~22 bits) so that rounding q'' does not perturb the logits
    f16x8 bqh[4], bql[4];
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const float4 c4 = *reinterpret_cast<const float4*>(sown + 4 * gr + 16 * e8);
      const float4 q4 = *reinterpret_cast<const float4*>(&qrot[g_own][4 * gr + 16 * e8]);
      const float x[4] = {col_ok ? c4.x * q4.x : 0.f, col_ok ? c4.y * q4.y : 0.f, col_ok ? c4.z * q4.z : 0.f,
                          col_ok ? c4.w * q4.w : 0.f};
      if constexpr (NG == 1) {
#pragma unroll
        for (int sl = 0; sl < 8; ++sl)
          if (keperm<KB>(sl) == e8) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              const float hi = f16_trunc(x[kb]);
              bqh[kb][sl] = static_cast<_Float16>(hi);
              bql[kb][sl] = static_cast<_Float16>(x[kb] - hi);
            }
          }
      } else {
        // k-step e8 / 2 holds code e8 of the four units in slots kg_slot(ui, e8 % 2)
#pragma unroll
        for (int ui = 0; ui < 4; ++ui) {
          const float hi = f16_trunc(x[ui]);
          bqh[e8 >> 1][kg_slot<KB>(ui, e8 & 1)] = static_cast<_Float16>(hi);
          bql[e8 >> 1][kg_slot<KB>(ui, e8 & 1)] = static_cast<_Float16>(x[ui] - hi);
        }
      }
    }

    // sigma_n = sum_j q''_nj over each quantisation group (all rows of the result equal); group g
    // is k-steps 4g/NG .. 4(g+1)/NG - 1
    float sigma[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 4 * g / NG; kb < 4 * (g + 1) / NG; ++kb) {
        d = mfma16(ONES, bqh[kb], d);
        d = mfma16(ONES, bql[kb], d);
      }
      sigma[g] = d[0];
    }

    // QK: one accumulator per page; the lane keeps its own page's column
    float lg[8][4];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      if constexpr (NG > 1) {
        // one accumulator per group, each scaled by its own (s', m') of the token
        f32x4 dg[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) dg[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f16x8 a = dequant_k_grouped<KB>(mb < 4 ? kpre.k[0][mb] : khi.k[0][mb - 4], kb);
          dg[kb * NG / 4] = mfma16(a, bqh[kb], dg[kb * NG / 4]);
          dg[kb * NG / 4] = mfma16(a, bql[kb], dg[kb * NG / 4]);
        }
        float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const float4 sk = *reinterpret_cast<const float4*>(sown + kCh + kCh * g + 16 * mb + 4 * gr);
          const float4 mk = *reinterpret_cast<const float4*>(sown + kCh * (1 + NG) + kCh * g + 16 * mb + 4 * gr);
          l4[0] += fmaf(sk.x, dg[g][0], mk.x * sigma[g]);
          l4[1] += fmaf(sk.y, dg[g][1], mk.y * sigma[g]);
          l4[2] += fmaf(sk.z, dg[g][2], mk.z * sigma[g]);
          l4[3] += fmaf(sk.w, dg[g][3], mk.w * sigma[g]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) lg[mb][i] = l4[i];
        continue;
      }
      f32x4 d[P];
#pragma unroll
      for (int e = 0; e < P; ++e) {
        d[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f16x8 a = dequant_k<KB>(mb < 4 ? kpre.k[e][mb] : khi.k[e][mb - 4], kb);
          d[e] = mfma16(a, bqh[kb], d[e]);
          d[e] = mfma16(a, bql[kb], d[e]);
        }
      }
      f32x4 dd = d[0];
#pragma unroll
      for (int e = 1; e < P; ++e) dd = (e_own == e) ? d[e] : dd;
      const float4 sk = *reinterpret_cast<const float4*>(sown + 128 + 16 * mb + 4 * gr);
      const float4 mk = *reinterpret_cast<const float4*>(sown + 256 + 16 * mb + 4 * gr);
      lg[mb][0] = fmaf(sk.x, dd[0], mk.x * sigma[0]);
      lg[mb][1] = fmaf(sk.y, dd[1], mk.y * sigma[0]);
      lg[mb][2] = fmaf(sk.z, dd[2], mk.z * sigma[0]);
      lg[mb][3] = fmaf(sk.w, dd[3], mk.w * sigma[0]);
    }

    __builtin_amdgcn_sched_barrier(0);
    VAll<VB, P> vc;
    load_v_all<KB, VB, P>(vc, rs, lane);

    // online softmax for column nl
    float mloc = -INFINITY;
    if (valid_own) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, lg[mb][i]);
    }
    mloc = rows_max4(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = m_new;

    if constexpr (NG == 1) {
      // PV weights w_t = p_t s'_t go to the MFMA in fp16 (w~).  u_j = sum_t w_t q_tj + sum_t p_t m'_t
      // is computed as sum_t w~_t (q_tj - c0) + (sum_t p_t m'_t + c0 sum_t w_t) with c0 = (2^b - 1)/2,
      // so that the rounding error sum_t (w~_t - w_t)(q_tj - c0) multiplies centred codes; the term
      // -c0 sum_t w~_t comes from the MFMA itself (weights against a constant operand).
      constexpr float c0 = 0.5f * ((1 << VB) - 1);
      f16x8 aw[4];
      float msum = 0.f, psum = 0.f, wexact = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float wv[2][4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int mb = 2 * kb + hh;
          const float4 sv = *reinterpret_cast<const float4*>(sown + 4 * 128 + 16 * mb + 4 * gr);
          const float4 mv = *reinterpret_cast<const float4*>(sown + 5 * 128 + 16 * mb + 4 * gr);
          const float svv[4] = {sv.x, sv.y, sv.z, sv.w};
          const float mvv[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = (live && valid_own) ? __builtin_amdgcn_exp2f(lg[mb][i] - m_new) : 0.f;
            psum += p;
            msum = fmaf(p, mvv[i], msum);
            wv[hh][i] = p * svv[i];
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          aw[kb][vslot<VB>(0, r)] = static_cast<_Float16>(wv[0][r]);
          aw[kb][vslot<VB>(1, r)] = static_cast<_Float16>(wv[1][r]);
          wexact += wv[0][r] + wv[1][r];
        }
      }
      l_part = l_part * alpha + psum;
      // the per-row constant of the PV result: -c0 sum_t w~_t (one MFMA per k-step against -c0) plus
      // sum_t p_t m'_t + c0 sum_t w_t as one extra k-step (fp16 hi + lo)
      const f32x4 corr = pv_zero_point<VB>(aw, fmaf(c0, wexact, msum), C0N);

      // alpha of the PV rows 4*gr + i lives in lane 4*gr + i (any row of lanes)
      float arow[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) arow[i] = __shfl(alpha, 4 * gr + i);
      const float* srow[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) srow[i] = sb + e_rc[G >= 4 ? 0 : i] * SC;

      // PV: one accumulator per page; the lane keeps its rows' page
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        f32x4 d[P];
#pragma unroll
        for (int e = 0; e < P; ++e) {
          d[e] = corr;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) d[e] = mfma16(aw[kb], dequant_v<VB>(vc.v[e][nb], kb), d[e]);
        }
        f32x4 dd = d[0];
#pragma unroll
        for (int e = 1; e < P; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) dd[i] = (e_row[G >= 4 ? 0 : i] == e) ? d[e][i] : dd[i];
        float cv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cv[i] = (G >= 4 || i == 0) ? srow[i][3 * 128 + 16 * nb + nl] : cv[0];
        if constexpr (G < 4) {
#pragma unroll
          for (int i = 1; i < 4; ++i) cv[i] = srow[i][3 * 128 + 16 * nb + nl];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nb][i] = fmaf(acc[nb][i], arow[i], cv[i] * dd[i]);
      }
    } else {
      // Quantisation groups (one page per step): the softmax numerators once, then per V group gv
      // (channel blocks nb = EV gv .. EV gv + EV - 1) its weights p_t s'_{t,gv} and zero-point sum.
      constexpr float c0 = 0.5f * ((1 << VB) - 1);
      constexpr int EV = 8 / NG;
      float pr[8][4];
      float psum = 0.f;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[mb][i] = (live && valid_own) ? __builtin_amdgcn_exp2f(lg[mb][i] - m_new) : 0.f;
          psum += pr[mb][i];
        }
      l_part = l_part * alpha + psum;
      float arow[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) arow[i] = __shfl(alpha, 4 * gr + i);
#pragma unroll
      for (int gv = 0; gv < NG; ++gv) {
        f16x8 aw[4];
        float msum = 0.f, wexact = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          float wv[2][4];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int mb = 2 * kb + hh;
            const float4 sv = *reinterpret_cast<const float4*>(sown + HS + kCh + kCh * gv + 16 * mb + 4 * gr);
            const float4 mv =
                *reinterpret_cast<const float4*>(sown + HS + kCh * (1 + NG) + kCh * gv + 16 * mb + 4 * gr);
            const float svv[4] = {sv.x, sv.y, sv.z, sv.w};
            const float mvv[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              msum = fmaf(pr[mb][i], mvv[i], msum);
              wv[hh][i] = pr[mb][i] * svv[i];
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            aw[kb][vslot<VB>(0, r)] = static_cast<_Float16>(wv[0][r]);
            aw[kb][vslot<VB>(1, r)] = static_cast<_Float16>(wv[1][r]);
            wexact += wv[0][r] + wv[1][r];
          }
        }
        const f32x4 corr = pv_zero_point<VB>(aw, fmaf(c0, wexact, msum), C0N);
#pragma unroll
        for (int nb = EV * gv; nb < EV * gv + EV; ++nb) {
          f32x4 d = corr;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) d = mfma16(aw[kb], dequant_v<VB>(vc.v[0][nb], kb), d);
          const float cv = sown[HS + 16 * nb + nl];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[nb][i] = fmaf(acc[nb][i], arow[i], cv * d[i]);
        }
      }
    }
    // the next group's K codes of blocks 0-3 and its scales, in flight while the next step starts
    __builtin_amdgcn_sched_barrier(0);
    if (gi + 1 < g_end) {
      recs(gi + 1, rec_next);
      __amdgpu_buffer_rsrc_t rs_n[P];
#pragma unroll
      for (int e = 0; e < P; ++e) rs_n[e] = record_rsrc(rec_next[e], R);
      load_k_half<KB, P>(kpre_next, rs_n, 0, lane);
      copy_scales<KB, VB, NG, P>(sb_next, rec_next, lane);
    }
    __builtin_amdgcn_wave_barrier();
  };

  if (g_begin < g_end) {
    float* const sb0 = stage0 + wave * (P * SC);
    float* const sb1 = stage1 + wave * (P * SC);
    KHalf<KB, P> ka, kb2;
    const uint8_t* ra[P];
    const uint8_t* rb[P];
    load_ids(g_begin);
    recs(g_begin, ra);
    {
      __amdgpu_buffer_rsrc_t rs[P];
#pragma unroll
      for (int e = 0; e < P; ++e) rs[e] = record_rsrc(ra[e], R);
      load_k_half<KB, P>(ka, rs, 0, lane);
      copy_scales<KB, VB, NG, P>(sb0, ra, lane);
    }
    for (int gi = g_begin; gi < g_end; gi += 2) {
      __builtin_amdgcn_sched_barrier(0);
      step(gi, ka, kb2, sb0, sb1, ra, rb);
      __builtin_amdgcn_sched_barrier(0);
      if (gi + 1 < g_end) step(gi + 1, kb2, ka, sb1, sb0, rb, ra);
    }
  }

  // ---- merge the 4 waves x P streams of each head, write one partial per head ----------
  const float l_col = rows_sum4(l_part);
  __syncthreads();  // the stages and qrot are reused below
  float* mrg = (wave < 2 ? stage0 : stage1) + (wave & 1) * 16 * MRG;
  if (gr == 0) {
    mrg[nl * MRG + 0] = m_run;
    mrg[nl * MRG + 1] = l_col;
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) mrg[(4 * gr + i) * MRG + 2 + 16 * nb + nl] = acc[nb][i];

  // This split's share of the fp16 tail (the len % 128 newest tokens): tokens t0 .. t1-1, for the
  // wave's query heads (wave, wave + 4, ...); raw-domain sums into qrot, (max, sum) into tail_ml.
  constexpr int HW = (G + 3) / 4;
  __shared__ float tail_ml[2][G];
  const int nt = len & (kTok - 1);
  // the tail owners: the first tail_splits splits, or all of them (then a split's share is small)
  const int owners = tail_splits > 0 ? tail_splits : n_splits;
  const int tps = (nt + owners - 1) / owners;
  const int t0 = min(nt, sp * tps), t1 = min(nt, t0 + tps);
  const bool has_tail = t1 > t0;
  if (has_tail && wave < G) {
    const int64_t tail_off = static_cast<int64_t>(sh) * kTok * kCh;
    float tmt[HW], tlt[HW], traw[HW][2];
    tail_heads<HW, G>(q + (static_cast<int64_t>(s) * num_q_heads + h * G) * kCh, wave, tail_k + tail_off,
                      tail_v + tail_off, t0, t1 - t0, sm_log2e, tmt, tlt, traw, lane);
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
      const int g = wave + 4 * hh;
      if (g < G) {
        qrot[g][2 * lane] = traw[hh][0];
        qrot[g][2 * lane + 1] = traw[hh][1];
        if (lane == 0) {
          tail_ml[0][g] = tmt[hh];
          tail_ml[1][g] = tlt[hh];
        }
      }
    }
  }
  __syncthreads();

  // partial of (head g, this split): [M, L, has tail, 0, rot[128], raw[128] (with a tail only)]
  for (int idx = tid; idx < G * kCh; idx += 256) {
    const int g = idx >> 7, j = idx & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int e = 0; e < P; ++e) M = fmaxf(M, (w < 2 ? stage0 : stage1)[((w & 1) * 16 + e * G + g) * MRG]);
    const float mt = has_tail ? tail_ml[0][g] : -INFINITY;
    M = fmaxf(M, mt);
    float L = 0.f, A = 0.f, W = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int e = 0; e < P; ++e) {
          const float* row = (w < 2 ? stage0 : stage1) + ((w & 1) * 16 + e * G + g) * MRG;
          const float f = __builtin_amdgcn_exp2f(row[0] - M);
          L = fmaf(row[1], f, L);
          A = fmaf(row[2 + j], f, A);
        }
      if (has_tail) {
        const float f = __builtin_amdgcn_exp2f(mt - M);
        L = fmaf(tail_ml[1][g], f, L);
        W = qrot[g][j] * f;
      }
    }
    float* po = ws + ((static_cast<int64_t>(s) * num_q_heads + h * G + g) * n_splits + sp) * kPartialFloats;
    if (j == 0) {
      store_agent(po, M);
      store_agent(po + 1, L);
      store_agent(po + 2, has_tail ? 1.0f : 0.0f);
      store_agent(po + 3, 0.0f);
    }
    store_agent(po + 4 + j, A);
    if (has_tail) store_agent(po + 4 + kCh + j, W);
  }

  // ---- the last workgroup of this (sequence, kv head) to finish merges the splits ----------
  // The partials were stored device-coherent; each thread waits until its stores have completed
  // before the workgroup counts its arrival, so the workgroup that counts the last arrival finds
  // every split's partial in place (and reads them device-coherent too).  It sets the counter back
  // to zero (no other workgroup of this launch touches it any more), so the workspace's counters
  // are zero again when the launch ends.
  __shared__ int last_wg;
  vmcnt_wait<0>();
  __syncthreads();
  if (tid == 0) last_wg = atomicAdd(counters + sh, 1) == n_splits - 1;
  __syncthreads();
  if (!last_wg) return;
  if (tid == 0) __hip_atomic_store(counters + sh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // splits that own tail tokens: the first ceil(nt / tps) (split sp owns tokens sp*tps .. sp*tps+tps-1)
  const int n_tail = tps > 0 ? (nt + tps - 1) / tps : 0;
  for (int g = wave; g < G; g += 4) {
    const int64_t sq = static_cast<int64_t>(s) * num_q_heads + h * G + g;
    combine_head(ws + sq * n_splits * kPartialFloats, n_splits, n_tail, out + sq * kCh, lane);
  }
}

template <int KB, int VB, int G, int NG>
static hipError_t launch_decode_t(const _Float16* q, const uint8_t* cache, int64_t page_stride,
                                  const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                                  const _Float16* tail_k, const _Float16* tail_v, float sm_scale, _Float16* out,
                                  float* workspace, int* counters, int num_seqs, int num_q_heads, int num_kv_heads,
                                  const DecodePlan& plan, hipStream_t stream) {
  const float qscale = sm_scale * kLog2e * 0.08838834764831845f;
  hipLaunchKernelGGL((decode_kernel<KB, VB, G, NG>), dim3(num_seqs * num_kv_heads, plan.n_splits), dim3(256), 0, stream,
                     q, cache, page_stride, page_table, max_pages, seq_lens, num_q_heads, num_kv_heads, qscale,
                     workspace, counters, plan.n_splits, plan.tail_splits, tail_k, tail_v, sm_scale * kLog2e, out);
  return hipGetLastError();
}

}  // namespace

#define KVARN_LAUNCHER_NAME2(N) launch_decode_ng##N
#define KVARN_LAUNCHER_NAME(N) KVARN_LAUNCHER_NAME2(N)
hipError_t KVARN_LAUNCHER_NAME(KVARN_DECODE_NG)(int kb, int vb, int group_size, const _Float16* q, const uint8_t* cache,
                                               int64_t page_stride, const int32_t* page_table, int max_pages,
                                               const int32_t* seq_lens, const _Float16* tail_k, const _Float16* tail_v,
                                               float sm_scale, _Float16* out, float* workspace, int* counters, int num_seqs,
                                               int num_q_heads, int num_kv_heads, const DecodePlan& plan,
                                               hipStream_t stream) {
  constexpr int NG = KVARN_DECODE_NG;
#define KVARN_DECODE_CASE(KB_, VB_, G_)                                                                           \
  if (kb == KB_ && vb == VB_ && group_size == G_)                                                                 \
    return launch_decode_t<KB_, VB_, G_, NG>(q, cache, page_stride, page_table, max_pages, seq_lens, tail_k, tail_v, \
                                             sm_scale, out, workspace, counters, num_seqs, num_q_heads, num_kv_heads, plan,  \
                                             stream);
#define KVARN_DECODE_BITS(G_)                                                                               \
  KVARN_DECODE_CASE(2, 2, G_) KVARN_DECODE_CASE(2, 4, G_) KVARN_DECODE_CASE(2, 8, G_)                       \
  KVARN_DECODE_CASE(4, 2, G_) KVARN_DECODE_CASE(4, 4, G_) KVARN_DECODE_CASE(4, 8, G_)                       \
  KVARN_DECODE_CASE(8, 2, G_) KVARN_DECODE_CASE(8, 4, G_) KVARN_DECODE_CASE(8, 8, G_)
  KVARN_DECODE_BITS(1)
  KVARN_DECODE_BITS(2)
  KVARN_DECODE_BITS(4)
  KVARN_DECODE_BITS(8)
  KVARN_DECODE_BITS(16)
#undef KVARN_DECODE_BITS
#undef KVARN_DECODE_CASE
  return hipErrorInvalidValue;
}

#if KVARN_DECODE_NG == 1
int decode_pages_per_step(int kb, int vb, int ng, int group_size) {
  if (group_size >= 16 || ng > 1) return 1;
  return (kb == 8 || vb == 8) ? 1 : 2;
}

DecodePlan plan_decode(int kb, int vb, int ng, int num_seqs, int num_kv_heads, int group_size, int max_pages_per_seq) {
  DecodePlan p;
  p.pages_per_group = decode_pages_per_step(kb, vb, ng, group_size);
  const int groups_max = (max_pages_per_seq + p.pages_per_group - 1) / p.pages_per_group;
  const int units = num_seqs * num_kv_heads;
  // 2 workgroups per CU on 256 CUs; 1 per CU with 8-bit codes, whose pages carry 2-3x the bytes
  // (longer runs per wave pipeline better there: 109 against 118 us for k8v8 at B 32 x 16K)
  const int target_wgs = (kb == 8 || vb == 8) ? 256 : 512;
  int splits0 = units > 0 ? (target_wgs + units - 1) / units : 1;
  if (splits0 < 1) splits0 = 1;
  // groups per split: a multiple of 4, so that each of the 4 waves of a workgroup gets the same count
  int gps = groups_max > 0 ? (groups_max + splits0 - 1) / splits0 : 1;
  gps = (gps + 3) / 4 * 4;
  p.groups_per_split = gps;
  const int page_splits = groups_max > 0 ? (groups_max + gps - 1) / gps : 1;
  constexpr int kTailSplits = 4;
  if (static_cast<int64_t>(units) * (page_splits + kTailSplits) <= target_wgs) {
    // few (sequence, kv head) pairs with long page runs: the fp16 tail (up to 127 tokens) goes to 4
    // workgroups of its own that own no pages, so its work overlaps the page stream instead of
    // lengthening the workgroups that stream pages (4 x 128K at 1 kv head: 47 -> 38 us with a tail)
    p.tail_splits = kTailSplits;
    p.n_splits = page_splits + kTailSplits;
  } else {
    // the grid is full: the tail is shared out among the page splits, at least 8 of them where the
    // grid has room, so that a split's share is about one 16-token chunk
    p.tail_splits = 0;
    p.n_splits = std::max(page_splits, std::min(8, splits0));
  }
  return p;
}

bool decode_supported(int kb, int vb, int ng, int group_size) {
  return (kb == 2 || kb == 4 || kb == 8) && (vb == 2 || vb == 4 || vb == 8) && (ng == 1 || ng == 2 || ng == 4) &&
         (group_size == 1 || group_size == 2 || group_size == 4 || group_size == 8 || group_size == 16);
}

hipError_t launch_decode(int kb, int vb, int ng, int group_size, const _Float16* q, const uint8_t* cache,
                         int64_t page_stride, const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                         const _Float16* tail_k, const _Float16* tail_v, float sm_scale, _Float16* out,
                         float* workspace, int* counters, int num_seqs, int num_q_heads, int num_kv_heads, const DecodePlan& plan,
                         hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  auto* fn = ng == 1 ? launch_decode_ng1 : ng == 2 ? launch_decode_ng2 : ng == 4 ? launch_decode_ng4 : nullptr;
  if (fn == nullptr) return hipErrorInvalidValue;
  return fn(kb, vb, group_size, q, cache, page_stride, page_table, max_pages, seq_lens, tail_k, tail_v, sm_scale, out,
            workspace, counters, num_seqs, num_q_heads, num_kv_heads, plan, stream);
}
#endif

}  // namespace kvarn
