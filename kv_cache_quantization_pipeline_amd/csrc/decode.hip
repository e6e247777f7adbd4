// KVarN decode attention over the packed cache, for gfx950.
//
// Scales are folded in on read ([LEHUY] section "Cơ chế hoạt động", stage 4;
// [HYPHO] section "它怎么做到的：四步流水线", step 4).  With the record of one
// page, xhat_t = Hn (c ⊙ (m'_t + s'_t q_t)) and Hn symmetric:
//   q . khat_t = s'_t (q'' . q_t) + m'_t sigma,   q' = Hn q, q'' = c_K ⊙ q', sigma = sum_j q''_j
//   sum_t p_t vhat_t = Hn ( c_V ⊙ ( sum_t (p_t s'_t) q_t + sum_t p_t m'_t ) )
// so channel scales go into the rotated query, token scales into the logits and the softmax
// weights, and Hn is applied once, to the merged output.  Logits are kept in the log2 domain (q' is
// pre-scaled by sm_scale * log2 e) so the softmax uses exp2.
//
// Work split.  Grid (sequence * kv head, split).  Split 0 of a (sequence, kv head) pair attends over
// the fp16 tail (the len % 128 newest tokens, raw domain); every other split is a workgroup of 4
// waves, and each wave takes exactly one group of P pages (P = 2 where the 16 MFMA columns hold two
// pages' query heads, else 1).  A wave issues all loads of its group at once (scales into LDS by
// global_load_lds, codes into registers) and keeps about 130-150 VGPRs, so 3-4 waves share each
// SIMD: the latency of one wave's loads is covered by the arithmetic of the others, and the many
// small workgroups balance the CUs.
//
// MFMA mapping (v_mfma_f32_16x16x32_f16).  Lane (gr = lane / 16, nl = lane % 16) owns query column
// n = nl = (page e, head g) of the group (n = e * G + g; columns past P * G are unused).
//   QK: A = the codes of 16 tokens (rows), K over channels; B = q'' of each column, split into fp16
//       hi + lo parts (two MFMAs per k-step, so that rounding q'' does not reach the logits).  The
//       result of page e is kept by the lanes whose column belongs to page e.
//   PV: A = the V codes (rows = 16 channels, K over tokens), B = the fp16 weights of each column,
//       zero in the columns of the other page, so both pages accumulate into one result; lane
//       (gr, nl) ends with channels 16 nb + 4 gr + i of its own column, whose softmax state (max,
//       sum) is its own too.  The weights' rounding error multiplies centred codes: the MFMA sums
//       w~ (q - c0), c0 = (2^b - 1) / 2, and sum_t p_t (m'_t + c0 s'_t) is added in fp32.
// Codes become exact fp16 integers in registers (4-bit: bytes read as fp8 e4m3, scaled by 2^9;
// 2-bit: nibbles read as fp4 e2m1, scaled by 2; 8-bit: 0x6400 | byte minus 1024).
//
// Merge.  Each page workgroup merges its 4 waves x P streams per query head in LDS and writes one
// partial (128 rotated-domain sums, running max in log2 units, running sum); the tail split writes
// one raw-domain partial per head.  A second kernel, one workgroup per (sequence, query head), merges
// the partials of all splits, applies Hn and writes fp16.  The kernel boundary orders the partials'
// stores before their loads, so the page workgroups end as soon as their stores are issued: no
// arrival counters, no waits for store completion, and no state kept in the workspace between calls.

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
// one wave, over the n tail tokens 0 .. n-1 (0 <= n <= 127) of their kv head.  Lane l owns channels
// 2l, 2l + 1: it reads those two channels of every key and value row (coalesced 256-byte rows) and
// of each query row, so a head's query costs two registers; the logits are summed across lanes 16
// tokens at a time (token t of a chunk ends in lanes t, t + 16, t + 32, t + 48).  Rows past the last
// token are clamped to it (in bounds) and masked.  Per head: mt = max_t lg_t (log2 units;
// lg = q . k * sm_log2e), lt = sum_t exp2(lg_t - mt), raw = sum_t exp2(lg_t - mt) v_t in the lane's
// two channels (-inf, 0, 0 for n = 0).
template <int HW, int G>
__device__ __forceinline__ void tail_heads(const _Float16* __restrict__ q0, int g0, const _Float16* __restrict__ tk,
                                           const _Float16* __restrict__ tv, int n, float sm_log2e,
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
  // online softmax over the chunks: running max m, sum lt and raw sums rescaled when m grows
  for (int c = 0; c < n; c += C) {
    f16x2 kk[C], vv[C];
#pragma unroll
    for (int u = 0; u < C; ++u) {
      const int row = min(c + u, n - 1);
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

// One partial: 128 sums (one per channel), then the running max (log2 units) and the running sum.
constexpr int kSumOff = 128;

// Per-format constants of the decode kernel.
template <int KB, int VB, int G, int NG>
struct DecodeCfg {
  // pages per wave group: the 16 MFMA columns are (page, head) pairs.  G = 16 fills them with one
  // page; otherwise two pages, except where 8-bit codes of two pages would crowd the registers and
  // for quantisation groups below 128 channels (their scale blocks are 5 or 9 KB per page).
  static constexpr int P = (G >= 16 || NG > 1 || KB == 8 || VB == 8) ? 1 : 2;
  static constexpr int R = record_bytes(KB, VB, NG);
  static constexpr int HS = half_scale_floats(NG);  // floats of one half's scales: c, s'[NG], m'[NG]
  static constexpr int SC = 2 * HS;                 // floats of scales per page
  static constexpr int SO = SC / 256;               // 1 KB LDS copies per page of scales
  // waves per SIMD the register budget is sized for
  // (four where the register budget of 128 holds without spilling: 2-bit V, one group, at most 8 query
  // heads, and 2-bit K or exactly 8 query heads; checked by the build's resource-usage report)
  static constexpr int OCC = (KB == 8 || VB == 8 || NG == 4)                            ? 2
                             : (VB == 2 && NG == 1 && G <= 8 && (KB == 2 || G == 8)) ? 4
                                                                                    : 3;
};

template <int KB>
struct PageK {
  KRegs<KB> k[8];  // token block mb: token 16 mb + nl, units 4 gr .. 4 gr + 3
};
template <int VB>
struct PageV {
  VRegs<VB> v[8];  // channel block nb: channel 16 nb + nl, tokens with (t >> 2) & 3 == gr
};

template <int KB>
__device__ __forceinline__ void load_page_k(PageK<KB>& d, __amdgpu_buffer_rsrc_t rs, int lane) {
  const uint32_t lo = static_cast<uint32_t>((lane & 15) * 16 * KB + 4 * (lane >> 4) * KB);
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const int off = mb * 16 * 16 * KB;
    if constexpr (KB == 2) {
      d.k[mb].w = bload64(rs, lo, off);
    } else if constexpr (KB == 4) {
      d.k[mb].w = bload128(rs, lo, off);
    } else {
      d.k[mb].w[0] = bload128(rs, lo, off);
      d.k[mb].w[1] = bload128(rs, lo, off + 16);
    }
  }
}

template <int KB, int VB>
__device__ __forceinline__ void load_page_v(PageV<VB>& d, __amdgpu_buffer_rsrc_t rs, int lane) {
  const uint32_t lo = static_cast<uint32_t>(lane * 4 * VB);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int off = k_code_bytes(KB) + nb * 64 * 4 * VB;
    if constexpr (VB == 2) {
      d.v[nb].w = bload64(rs, lo, off);
    } else if constexpr (VB == 4) {
      d.v[nb].w = bload128(rs, lo, off);
    } else {
      d.v[nb].w[0] = bload128(rs, lo, off);
      d.v[nb].w[1] = bload128(rs, lo, off + 16);
    }
  }
}

template <int KB, int VB, int G, int NG>
__global__ __launch_bounds__(256, (DecodeCfg<KB, VB, G, NG>::OCC)) void decode_kernel(
    const _Float16* __restrict__ q, const uint8_t* __restrict__ cache, int64_t page_stride,
    const int32_t* __restrict__ page_table, int max_pages, const int32_t* __restrict__ seq_lens, int num_q_heads,
    int num_kv_heads, float qscale, float* __restrict__ part, int tail_splits, int page_splits,
    const _Float16* __restrict__ tail_k,
    const _Float16* __restrict__ tail_v, float sm_log2e) {
  using Cfg = DecodeCfg<KB, VB, G, NG>;
  constexpr int P = Cfg::P;
  constexpr int R = Cfg::R;
  constexpr int HS = Cfg::HS;
  constexpr int SC = Cfg::SC;
  constexpr int MRG = kPartFloats;                 // floats per merged row in LDS (16-byte rows)
  constexpr int STAGE_FLOATS = 4 * P * SC;         // the 4 waves' scale blocks
  constexpr int MERGE_FLOATS = 4 * 16 * MRG;       // the 4 waves' 16 columns
  constexpr int BUF = STAGE_FLOATS > MERGE_FLOATS ? STAGE_FLOATS : MERGE_FLOATS;
  __shared__ __attribute__((aligned(16))) float qrot[G][kCh];
  __shared__ __attribute__((aligned(16))) float buf[BUF];

  const int sh = blockIdx.x;
  const int s = sh / num_kv_heads;
  const int h = sh - s * num_kv_heads;
  const int sp = blockIdx.y;
  const int n_splits = tail_splits + page_splits;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, gr = lane >> 4;
  const int len = seq_lens[s];
  // partials of (pair sh, head g): split k at part + ((sh * G + g) * n_splits + k) * kPartFloats
  const int64_t head0 = static_cast<int64_t>(sh) * G;

  if (sp < tail_splits) {
    // ---- the fp16 tail: raw-domain attention of every head of the pair, over this tail split's
    //      share of the tokens (128 / tail_splits consecutive ones) ----------------------------------
    constexpr int HW = (G + 3) / 4;
    const int share = kTok / tail_splits;
    const int t0 = sp * share;
    const int nt = min(max((len & (kTok - 1)) - t0, 0), share);
    const int64_t tail_off = (static_cast<int64_t>(sh) * kTok + t0) * kCh;
    if (wave < G) {
      float tmt[HW], tlt[HW], traw[HW][2];
      tail_heads<HW, G>(q + (static_cast<int64_t>(s) * num_q_heads + h * G) * kCh, wave, tail_k + tail_off,
                        tail_v + tail_off, nt, sm_log2e, tmt, tlt, traw, lane);
#pragma unroll
      for (int hh = 0; hh < HW; ++hh) {
        const int g = wave + 4 * hh;
        if (g < G) {
          float* po = part + ((head0 + g) * n_splits + sp) * kPartFloats;
          *reinterpret_cast<float2*>(po + 2 * lane) = make_float2(traw[hh][0], traw[hh][1]);
          if (lane == 0) *reinterpret_cast<float2*>(po + kSumOff) = make_float2(tmt[hh], tlt[hh]);
        }
      }
    }
  } else {
    // ---- a page split: one group of P pages per wave -------------------------------------------
    // The loads go out first, in this order: the query rows (for q'), then the group's scales (into
    // LDS) and codes.  Memory operations complete in order, so the q' rotation below waits for the
    // query rows only, while the page data is still in flight.
    constexpr int QI = (G * 32 + 255) / 256;  // query chunks of 4 channels per thread
    f16x4 qv[QI];
#pragma unroll
    for (int it = 0; it < QI; ++it) {
      const int idx = tid + 256 * it;
      if (idx < G * 32) {
        const int g = idx >> 5, r = idx & 31;
        qv[it] = *reinterpret_cast<const f16x4*>(q + (static_cast<int64_t>(s) * num_q_heads + h * G + g) * kCh + 4 * r);
      }
    }

    // this lane's column n = nl: page e_own of the group, head g_own; columns past P * G are unused
    const int e_own = nl / G;
    const int g_own = nl - e_own * G;
    const bool col_ok = e_own < P;
    const int e_oc = col_ok ? e_own : 0;

    const int n_pages = len >> 7;
    const int n_groups = (n_pages + P - 1) / P;
    const int gi = (sp - tail_splits) * 4 + wave;
    const bool has_group = gi < n_groups;

    float m_col = -INFINITY;   // running max of the column (log2 units), the same in its 4 lanes
    float l_lane = 0.f;        // softmax sum over this lane's tokens of the column
    float acc[8][4];           // channel 16 nb + 4 gr + i of the column, rotated domain, c_V applied
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[nb][i] = 0.f;

    // physical pages of the group (a missing second page is clamped to the last page and masked)
    const uint8_t* rec[P];
    __amdgpu_buffer_rsrc_t rs[P];
    float* const stg = buf + wave * (P * SC);
    PageK<KB> K[1];
    if (has_group) {
      const int64_t pt_row = static_cast<int64_t>(s) * max_pages;
      const int64_t head_off = static_cast<int64_t>(h) * R;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const int phys = page_table[pt_row + min(gi * P + e, n_pages - 1)];
        rec[e] = cache + static_cast<int64_t>(phys) * page_stride + head_off;
        rs[e] = record_rsrc(rec[e], R);
      }
      copy_scales<KB, VB, NG, P>(stg, rec, lane);
      __builtin_amdgcn_sched_barrier(0);
      load_page_k<KB>(K[0], rs[0], lane);
      __builtin_amdgcn_sched_barrier(0);
    }

    // q' = Hn q * sm_scale * log2(e) / sqrt(128): 32 threads per head, 4 channels each
#pragma unroll
    for (int it = 0; it < QI; ++it) {
      const int idx = tid + 256 * it;
      if (idx < G * 32) {
        const int g = idx >> 5, r = idx & 31;
        const float x0 = qv[it][0], x1 = qv[it][1], x2 = qv[it][2], x3 = qv[it][3];
        const float a0 = x0 + x1, a1 = x0 - x1, a2 = x2 + x3, a3 = x2 - x3;
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

    if (has_group) {
      // the scale copy into the stage has landed once only the code loads are outstanding (the
      // compiler does not track the LDS copy itself)
      vmcnt_wait<(KB == 8 ? 16 : 8)>();

      const bool valid_own = col_ok && gi * P + e_own < n_pages;
      const float* const sown = stg + e_oc * SC;

      // q'' = c_K ⊙ q' of this lane's column as the QK B operand, split into fp16 hi + lo parts
      // (q'' = hi + lo to ~22 bits; hi is exact fp16, so the split does not depend on how the
      // compiler converts)
      f16x8 bqh[4], bql[4];
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const float4 c4 = *reinterpret_cast<const float4*>(sown + 4 * gr + 16 * e8);
        const float4 q4 = *reinterpret_cast<const float4*>(&qrot[g_own][4 * gr + 16 * e8]);
        const float x[4] = {col_ok ? c4.x * q4.x : 0.f, col_ok ? c4.y * q4.y : 0.f, col_ok ? c4.z * q4.z : 0.f,
                            col_ok ? c4.w * q4.w : 0.f};
        if constexpr (NG == 1) {
          // slot sl of k-step kb holds channel 4 gr + kb + 16 keperm(sl)
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

      f16x8 ONES;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) ONES[sl] = static_cast<_Float16>(1.0f);
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

      // QK, page by page; lg[mb][i]: token 16 mb + 4 gr + i of the lane's column (its own page).
      // The V codes of a page are issued once its K codes are consumed.
      float lg[8][4];
      PageV<VB> V[P];
#pragma unroll
      for (int e = 0; e < P; ++e) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          float v4[4];
          if constexpr (NG == 1) {
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              const f16x8 a = dequant_k<KB>(K[0].k[mb], kb);
              d = mfma16(a, bqh[kb], d);
              d = mfma16(a, bql[kb], d);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) v4[i] = d[i];
          } else {
            // one accumulator per group, each scaled by its own (s', m') of the token (P = 1)
            f32x4 dg[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) dg[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              const f16x8 a = dequant_k_grouped<KB>(K[0].k[mb], kb);
              dg[kb * NG / 4] = mfma16(a, bqh[kb], dg[kb * NG / 4]);
              dg[kb * NG / 4] = mfma16(a, bql[kb], dg[kb * NG / 4]);
            }
            // the groups' terms summed from the first one (no 0 + x, which the compiler must keep)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
              const float4 sk = *reinterpret_cast<const float4*>(sown + kCh + kCh * g + 16 * mb + 4 * gr);
              const float4 mk = *reinterpret_cast<const float4*>(sown + kCh * (1 + NG) + kCh * g + 16 * mb + 4 * gr);
              const float t[4] = {fmaf(sk.x, dg[g][0], mk.x * sigma[g]), fmaf(sk.y, dg[g][1], mk.y * sigma[g]),
                                  fmaf(sk.z, dg[g][2], mk.z * sigma[g]), fmaf(sk.w, dg[g][3], mk.w * sigma[g])};
#pragma unroll
              for (int i = 0; i < 4; ++i) v4[i] = g == 0 ? t[i] : v4[i] + t[i];
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) lg[mb][i] = (e == 0 || e_own == e) ? v4[i] : lg[mb][i];
        }
        __builtin_amdgcn_sched_barrier(0);
        if (e + 1 < P) load_page_k<KB>(K[0], rs[e + 1], lane);
        load_page_v<KB, VB>(V[e], rs[e], lane);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NG == 1) {
        // logits: s'_t (q'' . q_t) + m'_t sigma
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          const float4 sk = *reinterpret_cast<const float4*>(sown + kCh + 16 * mb + 4 * gr);
          const float4 mk = *reinterpret_cast<const float4*>(sown + 2 * kCh + 16 * mb + 4 * gr);
          lg[mb][0] = fmaf(sk.x, lg[mb][0], mk.x * sigma[0]);
          lg[mb][1] = fmaf(sk.y, lg[mb][1], mk.y * sigma[0]);
          lg[mb][2] = fmaf(sk.z, lg[mb][2], mk.z * sigma[0]);
          lg[mb][3] = fmaf(sk.w, lg[mb][3], mk.w * sigma[0]);
        }
      }

      // softmax of the column over the group's tokens (one group per wave: no earlier state)
      float mloc = -INFINITY;
      if (valid_own) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, lg[mb][i]);
      }
      m_col = rows_max4(mloc);
      const bool live = valid_own && m_col != -INFINITY;
      // The weights w_t = p_t s'_t go to the MFMA in fp16.  So that they stay in fp16's normal range
      // whatever the magnitude of V, the softmax of the column is taken against m + E, with 2^E the
      // power of two at or below the page's largest V token scale: then w_t <= 2.  The column's state
      // (m + E, sum_t p_t 2^-E, sums 2^-E) is the same online-softmax state with a shifted reference.
      int e_pow[P];
#pragma unroll
      for (int e = 0; e < P; ++e) {
        const float* sv = stg + e * SC + HS + kCh;  // s'_V of page e, NG x 128 floats
        float smax = 0.f;
#pragma unroll
        for (int k = 0; k < 2 * NG; ++k) smax = fmaxf(smax, sv[lane + 64 * k]);
        smax = rows_max4(row_max16(smax));
        const int ex = smax > 0.f ? __builtin_amdgcn_frexp_expf(smax) - 1 : 0;
        e_pow[e] = min(max(ex, -100), 100);
      }
      int e_col = e_pow[0];
#pragma unroll
      for (int e = 1; e < P; ++e) e_col = e_oc == e ? e_pow[e] : e_col;
      const float m_ref = m_col + static_cast<float>(e_col);

      f16x8 C0N;
      constexpr float c0 = 0.5f * ((1 << VB) - 1);
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) C0N[sl] = static_cast<_Float16>(-c0);

      // numerators p_t (the lane's tokens of its column); a column with no live token subtracts +inf,
      // so that every exponent is -inf and every p_t 0 without a select per token
      const float m_sub = live ? m_ref : INFINITY;
      float pr[8][4];
      float psum = 0.f;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[mb][i] = __builtin_amdgcn_exp2f(lg[mb][i] - m_sub);
          psum += pr[mb][i];
        }
      l_lane = psum;

      // Per V quantisation group gv (channel blocks EV gv .. EV gv + EV - 1): the weights
      // w_t = p_t s'_t as fp16 B operand (slot vslot(h, i) of k-step kb: token 32 kb + 16 h + 4 gr + i),
      // and the per-column constant sum_t p_t m'_t + c0 sum_t w_t - c0 sum_t w~_t, the last sum taken
      // by the MFMA itself from the fp16 weights it multiplies.
      constexpr int EV = 8 / NG;
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
            const float4 mv = *reinterpret_cast<const float4*>(sown + HS + kCh * (1 + NG) + kCh * gv + 16 * mb + 4 * gr);
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
        const float bracket = rows_sum4(fmaf(c0, wexact, msum));
        f32x4 z = {bracket, bracket, bracket, bracket};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) z = mfma16(C0N, aw[kb], z);

        // the weights as the B operand of each page: zero in the columns of the other page
        f16x8 bw[P][4];
#pragma unroll
        for (int e = 0; e < P; ++e)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) bw[e][kb] = (P == 1 || e_own == e) ? aw[kb] : zero8();

#pragma unroll
        for (int nb = EV * gv; nb < EV * gv + EV; ++nb) {
          f32x4 c = z;
#pragma unroll
          for (int e = 0; e < P; ++e)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) c = mfma16(dequant_v<VB>(V[e].v[nb], kb), bw[e][kb], c);
          const float4 cv = *reinterpret_cast<const float4*>(sown + HS + 16 * nb + 4 * gr);
          acc[nb][0] = cv.x * c[0];
          acc[nb][1] = cv.y * c[1];
          acc[nb][2] = cv.z * c[2];
          acc[nb][3] = cv.w * c[3];
        }
      }
      m_col = m_ref;  // the reference the column's sums are taken against
    }

    // ---- merge the 4 waves x P streams of each head, write one partial per head ----------------
    const float l_col = rows_sum4(l_lane);
    __syncthreads();  // every wave is done with its scale stage (the merge rows reuse the buffer)
    {
      float* row = buf + (wave * 16 + nl) * MRG;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        *reinterpret_cast<float4*>(row + 16 * nb + 4 * gr) = make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
      if (gr == 0) *reinterpret_cast<float2*>(row + kSumOff) = make_float2(m_col, l_col);
    }
    __syncthreads();
    for (int idx = tid; idx < G * (kCh / 2); idx += 256) {
      const int g = idx >> 6, j = 2 * (idx & 63);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int e = 0; e < P; ++e) M = fmaxf(M, buf[(w * 16 + e * G + g) * MRG + kSumOff]);
      float L = 0.f, A0 = 0.f, A1 = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int e = 0; e < P; ++e) {
            const float* row = buf + (w * 16 + e * G + g) * MRG;
            const float f = __builtin_amdgcn_exp2f(row[kSumOff] - M);
            const float2 a = *reinterpret_cast<const float2*>(row + j);
            L = fmaf(row[kSumOff + 1], f, L);
            A0 = fmaf(a.x, f, A0);
            A1 = fmaf(a.y, f, A1);
          }
      }
      float* po = part + ((head0 + g) * n_splits + sp) * kPartFloats;
      *reinterpret_cast<float2*>(po + j) = make_float2(A0, A1);
      if (j == 0) *reinterpret_cast<float2*>(po + kSumOff) = make_float2(M, L);
    }
  }
}

// Merge of the split partials of one (sequence, query head) per workgroup of W waves (8 waves with 8
// rows in flight each, or 16 with 16 for over 64 page splits and few workgroups): splits 0 ..
// tail_splits - 1 are the tail's (raw domain), the rest the pages' (rotated domain).  Wave w folds page
// splits tail_splits + w, tail_splits + W + w, ... with an online rescale, B splits' rows in flight at a
// time; wave 0 also folds the tail splits, whose rows it loads before its first batch and folds after
// issuing it, so both are in flight together.  With M the largest running max and f_k = exp2(M_k - M):
// L = sum_k f_k L_k, out = (Hn sum_{page k} f_k rot_k + sum_{tail k} f_k raw_k) / L; all zero for an
// empty sequence.  Lane l owns output channels 2l, 2l + 1.
template <int W, int B>
__global__ __launch_bounds__(64 * W) void decode_merge_kernel(const float* __restrict__ part, int tail_splits,
                                                              int n_splits, _Float16* __restrict__ out) {
  constexpr int kBatch = B, kW = W;
  __shared__ float2 wacc[kW][64];
  __shared__ float2 wml[kW];
  const int hq = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float* ph = part + static_cast<int64_t>(hq) * n_splits * kPartFloats;
  // the tail splits' rows (at most kMaxTailSplits), wave 0 only
  float2 tl_ml[kMaxTailSplits], tl_a[kMaxTailSplits];
  if (wave == 0) {
#pragma unroll
    for (int k = 0; k < kMaxTailSplits; ++k) {
      if (k < tail_splits) {
        tl_ml[k] = *reinterpret_cast<const float2*>(ph + k * kPartFloats + kSumOff);
        tl_a[k] = *reinterpret_cast<const float2*>(ph + k * kPartFloats + 2 * lane);
      } else {
        tl_ml[k] = make_float2(-INFINITY, 0.f);
        tl_a[k] = make_float2(0.f, 0.f);
      }
    }
  }
  bool tail_pending = wave == 0;  // every call has a page split, so wave 0 enters the loop below
  float2 tml = make_float2(-INFINITY, 0.f), traw = make_float2(0.f, 0.f);

  float M = -INFINITY, L = 0.f, r0 = 0.f, r1 = 0.f;
  for (int k0 = tail_splits + wave; k0 < n_splits; k0 += kW * kBatch) {
    float2 ml[kBatch], a[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int k = k0 + kW * u;
      if (k < n_splits) {
        ml[u] = *reinterpret_cast<const float2*>(ph + k * kPartFloats + kSumOff);
        a[u] = *reinterpret_cast<const float2*>(ph + k * kPartFloats + 2 * lane);
      } else {
        ml[u] = make_float2(-INFINITY, 0.f);
        a[u] = make_float2(0.f, 0.f);
      }
    }
    if (tail_pending) {
      // fold the tail splits into one raw-domain partial
      tail_pending = false;
      float Mr = tl_ml[0].x;
#pragma unroll
      for (int k = 1; k < kMaxTailSplits; ++k) Mr = fmaxf(Mr, tl_ml[k].x);
      if (Mr != -INFINITY) {
        tml = make_float2(Mr, 0.f);
#pragma unroll
        for (int k = 0; k < kMaxTailSplits; ++k) {
          const float f = __builtin_amdgcn_exp2f(tl_ml[k].x - Mr);
          tml.y = fmaf(tl_ml[k].y, f, tml.y);
          traw.x = fmaf(tl_a[k].x, f, traw.x);
          traw.y = fmaf(tl_a[k].y, f, traw.y);
        }
      }
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) Mb = fmaxf(Mb, ml[u].x);
    if (Mb != -INFINITY) {
      const float fo = __builtin_amdgcn_exp2f(M - Mb);  // 0 while M is still -inf
      L *= fo;
      r0 *= fo;
      r1 *= fo;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float f = __builtin_amdgcn_exp2f(ml[u].x - Mb);
        L = fmaf(ml[u].y, f, L);
        r0 = fmaf(a[u].x, f, r0);
        r1 = fmaf(a[u].y, f, r1);
      }
      M = Mb;
    }
  }
  wacc[wave][lane] = make_float2(r0, r1);
  if (lane == 0) wml[wave] = make_float2(M, L);
  __syncthreads();
  if (wave != 0) return;

  float Mt = tml.x;
#pragma unroll
  for (int w = 0; w < kW; ++w) Mt = fmaxf(Mt, wml[w].x);
  float Lt = 0.f, r[2] = {0.f, 0.f}, raw[2] = {0.f, 0.f};
  if (Mt != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const float f = __builtin_amdgcn_exp2f(wml[w].x - Mt);
      Lt = fmaf(wml[w].y, f, Lt);
      r[0] = fmaf(wacc[w][lane].x, f, r[0]);
      r[1] = fmaf(wacc[w][lane].y, f, r[1]);
    }
    const float ft = __builtin_amdgcn_exp2f(tml.x - Mt);
    Lt = fmaf(tml.y, ft, Lt);
    raw[0] = traw.x * ft;
    raw[1] = traw.y * ft;
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
  const float inv_l = Lt > 0.f ? 1.0f / Lt : 0.f;
  constexpr float kInvSqrt128 = 0.08838834764831845f;
  *reinterpret_cast<f16x2*>(out + static_cast<int64_t>(hq) * kCh + 2 * lane) =
      f16x2{static_cast<_Float16>((r[0] * kInvSqrt128 + raw[0]) * inv_l),
            static_cast<_Float16>((r[1] * kInvSqrt128 + raw[1]) * inv_l)};
}

template <int KB, int VB, int G, int NG>
static hipError_t launch_decode_t(const _Float16* q, const uint8_t* cache, int64_t page_stride,
                                  const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                                  const _Float16* tail_k, const _Float16* tail_v, float sm_scale, _Float16* out,
                                  const DecodeWorkspace& ws, int num_seqs, int num_q_heads, int num_kv_heads,
                                  const DecodePlan& plan, hipStream_t stream) {
  const float qscale = sm_scale * kLog2e * 0.08838834764831845f;
  hipLaunchKernelGGL((decode_kernel<KB, VB, G, NG>), dim3(num_seqs * num_kv_heads, plan.tail_splits + plan.page_splits),
                     dim3(256), 0,
                     stream, q, cache, page_stride, page_table, max_pages, seq_lens, num_q_heads, num_kv_heads, qscale,
                     ws.part, plan.tail_splits, plan.page_splits, tail_k, tail_v, sm_scale * kLog2e);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 16 waves only where the splits outnumber one 8-wave batch and the (sequence, query head)
  // workgroups are too few to fill the chip anyway
  if (plan.page_splits > 8 * 8 && static_cast<int64_t>(num_seqs) * num_q_heads < 512)
    hipLaunchKernelGGL((decode_merge_kernel<16, 16>), dim3(num_seqs * num_q_heads), dim3(1024), 0, stream, ws.part,
                       plan.tail_splits, plan.tail_splits + plan.page_splits, out);
  else
    hipLaunchKernelGGL((decode_merge_kernel<8, 8>), dim3(num_seqs * num_q_heads), dim3(512), 0, stream, ws.part,
                       plan.tail_splits, plan.tail_splits + plan.page_splits, out);
  return hipGetLastError();
}

}  // namespace

#define KVARN_LAUNCHER_NAME2(N) launch_decode_ng##N
#define KVARN_LAUNCHER_NAME(N) KVARN_LAUNCHER_NAME2(N)
hipError_t KVARN_LAUNCHER_NAME(KVARN_DECODE_NG)(int kb, int vb, int group_size, const _Float16* q, const uint8_t* cache,
                                               int64_t page_stride, const int32_t* page_table, int max_pages,
                                               const int32_t* seq_lens, const _Float16* tail_k, const _Float16* tail_v,
                                               float sm_scale, _Float16* out, const DecodeWorkspace& ws, int num_seqs,
                                               int num_q_heads, int num_kv_heads, const DecodePlan& plan,
                                               hipStream_t stream) {
  constexpr int NG = KVARN_DECODE_NG;
#define KVARN_DECODE_CASE(KB_, VB_, G_)                                                                             \
  if (kb == KB_ && vb == VB_ && group_size == G_)                                                                   \
    return launch_decode_t<KB_, VB_, G_, NG>(q, cache, page_stride, page_table, max_pages, seq_lens, tail_k, tail_v, \
                                             sm_scale, out, ws, num_seqs, num_q_heads, num_kv_heads, plan, stream);
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
  // one group per wave, 4 waves per page split; at least one page split
  p.page_splits = std::max(1, (groups_max + 3) / 4);
  // The fp16 tail (up to 127 tokens of every head of a pair) is one split's work, or eight splits' of
  // one 16-token chunk each where the pages leave the grid with few workgroups: the tail walk is then
  // on the critical path of the call.
  const int64_t page_wgs = static_cast<int64_t>(num_seqs) * num_kv_heads * p.page_splits;
  p.tail_splits = page_wgs < 1024 ? kMaxTailSplits : 1;
  return p;
}

size_t decode_workspace_bytes(const DecodePlan& plan, int num_seqs, int num_q_heads, int num_kv_heads) {
  (void)num_kv_heads;
  return static_cast<size_t>(num_seqs) * num_q_heads * (plan.tail_splits + plan.page_splits) * kPartFloats *
         sizeof(float);
}

DecodeWorkspace decode_workspace_layout(void* workspace, const DecodePlan& plan, int num_seqs, int num_q_heads,
                                        int num_kv_heads) {
  (void)plan;
  (void)num_seqs;
  (void)num_q_heads;
  (void)num_kv_heads;
  DecodeWorkspace w;
  w.part = static_cast<float*>(workspace);
  return w;
}

bool decode_supported(int kb, int vb, int ng, int group_size) {
  return (kb == 2 || kb == 4 || kb == 8) && (vb == 2 || vb == 4 || vb == 8) && (ng == 1 || ng == 2 || ng == 4) &&
         (group_size == 1 || group_size == 2 || group_size == 4 || group_size == 8 || group_size == 16);
}

hipError_t launch_decode(int kb, int vb, int ng, int group_size, const _Float16* q, const uint8_t* cache,
                         int64_t page_stride, const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                         const _Float16* tail_k, const _Float16* tail_v, float sm_scale, _Float16* out,
                         const DecodeWorkspace& ws, int num_seqs, int num_q_heads, int num_kv_heads,
                         const DecodePlan& plan, hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  auto* fn = ng == 1 ? launch_decode_ng1 : ng == 2 ? launch_decode_ng2 : ng == 4 ? launch_decode_ng4 : nullptr;
  if (fn == nullptr) return hipErrorInvalidValue;
  return fn(kb, vb, group_size, q, cache, page_stride, page_table, max_pages, seq_lens, tail_k, tail_v, sm_scale, out,
            ws, num_seqs, num_q_heads, num_kv_heads, plan, stream);
}
#endif

}  // namespace kvarn
