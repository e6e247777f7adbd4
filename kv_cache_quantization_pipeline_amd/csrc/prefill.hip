// KVarN chunked-prefill attention over the packed cache, for gfx950.
//
// Sequence s holds L = seq_lens[s] tokens: floor(L / 128) quantised pages and an fp16 tail of the
// L % 128 newest tokens.  Its last n = q_lens[s] tokens are this chunk's queries (their keys and
// values were appended before the call); query i sits at position L - n + i and attends causally
// to positions 0 .. L - n + i.  Prefill is the phase with many queries per kv head ([HYPHO] section
// "它怎么做到的：四步流水线" describes the cache it reads; the scales are folded in on read as in
// decode, [LEHUY] section "Cơ chế hoạt động", stage 4).
//
// Work split: grid (sequence * kv head, blocks of 64 query rows), a row being a (query token,
// query head of this kv head) pair, head fastest; 4 waves per workgroup, 16 rows per wave.  The 16
// MFMA columns of a wave are its 16 query rows.
//
// Per page, the workgroup converts the page's K and V codes to fp16 once, into LDS, in the MFMA
// operand layouts (each wave a quarter: token blocks 2w, 2w + 1 of K, channel blocks 2w, 2w + 1 of
// V), while the page's scale block goes to LDS by asynchronous copy; the next page's codes and
// scales are already being loaded while the current page is computed.  Each wave then does for its
// 16 rows what the decode kernel does for one page: QK with the K codes as the A operand and
// q'' = c_K ⊙ q' (fp16 hi + lo) as the B operand, one accumulator per quantisation group, logits
// sum_g s'_g (q''_g . codes) + m'_g sigma_g, the causal mask, an online softmax per row, and PV per
// V group with the fp16 weights p_t s'_t against the V codes (the zero-point sum through one MFMA,
// channel scale c_V on the result).  The fp16 tail is attended in the raw domain: raw q against raw
// K rows, then the weights against the tail V staged in LDS transposed; that accumulator is added
// once Hn has been applied to the rotated one.

#include "kvarn_codes.h"
#include "kvarn_device.h"
#include "kvarn_internal.h"

#ifndef KVARN_PREFILL_NG
#define KVARN_PREFILL_NG 1
#endif

namespace kvarn {

namespace {

constexpr int kRowsPerBlock = 64;  // 4 waves x 16 query rows
// Smallest divisor of a row's PV weights on one page (see the weight rescale below).
constexpr float kMinWeightScale = 1e-30f;

// Position of tail token t in a row of the transposed LDS copy of the tail V: k-step t / 32, lane
// row (t >> 2) & 3, slot 2 (t & 3) + ((t >> 4) & 1), the slot order of the PV weights below.
__device__ __forceinline__ int vt_pos(int t) {
  return (t >> 5) * 32 + ((t >> 2) & 3) * 8 + 2 * (t & 3) + ((t >> 4) & 1);
}

// The codes this wave converts for one page: K token blocks 2w, 2w + 1 and V channel blocks 2w, 2w + 1.
template <int KB, int VB>
struct PageShare {
  KRegs<KB> k[2];
  VRegs<VB> v[2];
};

template <int KB, int VB>
__device__ __forceinline__ void load_share(PageShare<KB, VB>& d, __amdgpu_buffer_rsrc_t rs, int wave, int lane) {
  const uint32_t klo = static_cast<uint32_t>((lane & 15) * 16 * KB + 4 * (lane >> 4) * KB);
  const uint32_t vlo = static_cast<uint32_t>(lane * 4 * VB);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int koff = (2 * wave + m) * 16 * 16 * KB;
    if constexpr (KB == 2) {
      d.k[m].w = bload64(rs, klo, koff);
    } else if constexpr (KB == 4) {
      d.k[m].w = bload128(rs, klo, koff);
    } else {
      d.k[m].w[0] = bload128(rs, klo, koff);
      d.k[m].w[1] = bload128(rs, klo, koff + 16);
    }
    const int voff = k_code_bytes(KB) + (2 * wave + m) * 64 * 4 * VB;
    if constexpr (VB == 2) {
      d.v[m].w = bload64(rs, vlo, voff);
    } else if constexpr (VB == 4) {
      d.v[m].w = bload128(rs, vlo, voff);
    } else {
      d.v[m].w[0] = bload128(rs, vlo, voff);
      d.v[m].w[1] = bload128(rs, vlo, voff + 16);
    }
  }
}

// This wave's 1 KB chunks (c = wave, wave + 4, ...) of a page's scale block into the LDS stage.
template <int KB, int VB, int NG>
__device__ __forceinline__ void copy_scale_share(float* stage, const uint8_t* rec, int wave, int lane) {
  constexpr int SC = 2 * half_scale_floats(NG);
  constexpr int CHUNKS = SC / 256;
  const uint8_t* sbase = rec + scale_offset(KB, VB);
  const uint32_t lo = static_cast<uint32_t>(lane * 16);
#pragma unroll
  for (int c0 = 0; c0 < CHUNKS; c0 += 4) {
    const int c = c0 + wave;
    if (c < CHUNKS)
      __builtin_amdgcn_global_load_lds(sbase + (lo + static_cast<uint32_t>(c * 1024)), stage + c * 256, 16, 0, 0);
  }
}

template <int KB, int VB, int G, int NG>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const _Float16* __restrict__ q,
                                                         const int32_t* __restrict__ q_lens, int max_q,
                                                         const uint8_t* __restrict__ cache, int64_t page_stride,
                                                         const int32_t* __restrict__ page_table, int max_pages,
                                                         const int32_t* __restrict__ seq_lens,
                                                         const _Float16* __restrict__ tail_k,
                                                         const _Float16* __restrict__ tail_v, int num_q_heads,
                                                         int num_kv_heads, float qscale, float rawscale,
                                                         _Float16* __restrict__ out) {
  constexpr int R = record_bytes(KB, VB, NG);
  constexpr int HS = half_scale_floats(NG);  // floats of one half's scales: c, s'[NG], m'[NG]
  constexpr int SC = 2 * HS;
  constexpr int EV = 8 / NG;                 // V channel blocks per quantisation group
  // Scale stages: two (the next page's scales copied while the current page is computed), or one for
  // four groups per token, whose 9 KB scale block would otherwise leave room for one workgroup per CU.
  constexpr int NSTAGE = NG == 4 ? 1 : 2;
  // LDS: the page's codes as fp16 operands (K [mb][kb][lane], V [nb][kb][lane]) and the scale stages.
  // The query rotation at the start and the tail's transposed V at the end reuse the K region.
  __shared__ __attribute__((aligned(16))) f16x8 kdq[8][4][64];
  __shared__ __attribute__((aligned(16))) f16x8 vdq[8][4][64];
  __shared__ __attribute__((aligned(16))) float stage[NSTAGE][SC];
  float(*qrot)[kCh] = reinterpret_cast<float(*)[kCh]>(&kdq[0][0][0]);
  _Float16(*vt)[kTok] = reinterpret_cast<_Float16(*)[kTok]>(&kdq[0][0][0]);
  static_assert(sizeof(kdq) >= kRowsPerBlock * kCh * sizeof(float), "query rows alias the K codes");
  static_assert(sizeof(kdq) >= kCh * kTok * sizeof(_Float16), "tail V aliases the K codes");

  const int sh = blockIdx.x;
  const int s = sh / num_kv_heads;
  const int h = sh - s * num_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15, gr = lane >> 4;
  const int L = seq_lens[s];
  const int n = min(min(q_lens[s], max_q), L);
  const int row0 = blockIdx.y * kRowsPerBlock;
  if (row0 >= n * G) return;  // the same for the whole workgroup
  const int full = L >> 7, nt = L & (kTok - 1);

  // ---- q' = Hn q * sm_scale * log2(e) for the block's 64 rows: 32 threads per row ------------------
  for (int base = 0; base < kRowsPerBlock * 32; base += 256) {
    const int idx = base + tid;
    const int r = idx >> 5, c = idx & 31;
    const int rg = row0 + r;
    const int i = rg / G, g = rg - (rg / G) * G;
    float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
    if (i < n) {
      const _Float16* qp = q + ((static_cast<int64_t>(s) * max_q + i) * num_q_heads + h * G + g) * kCh + 4 * c;
      x0 = qp[0];
      x1 = qp[1];
      x2 = qp[2];
      x3 = qp[3];
    }
    const float a0 = x0 + x1, a1 = x0 - x1, a2 = x2 + x3, a3 = x2 - x3;
    float v[4] = {a0 + a2, a1 + a3, a0 - a2, a1 - a3};
#pragma unroll
    for (int b = 0; b < 5; ++b) {
      const bool upper = (c >> b) & 1;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float o = __shfl_xor(v[k], 1 << b, 32);
        v[k] = upper ? o - v[k] : v[k] + o;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) qrot[r][4 * c + k] = v[k] * qscale;
  }
  __syncthreads();

  // this lane's QK column / PV weight row: row wave * 16 + nl of the block
  const int rg_own = row0 + wave * 16 + nl;
  const int i_own = rg_own / G;
  const int p_own = i_own < n ? L - n + i_own : -1;  // last key position the row sees
  int pm = p_own;
#pragma unroll
  for (int b = 1; b < 16; b <<= 1) pm = max(pm, __shfl_xor(pm, b));
  const int pmax = __builtin_amdgcn_readfirstlane(pm);  // over the wave's 16 rows

  // a row past the chunk keeps q' = 0 (its logits stay finite; it is never written)
  const bool col_ok = p_own >= 0;
  float4 qv[8];
#pragma unroll
  for (int e8 = 0; e8 < 8; ++e8) {
    const float4 v = *reinterpret_cast<const float4*>(&qrot[wave * 16 + nl][4 * gr + 16 * e8]);
    qv[e8] = col_ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  // the first key position not visible to every valid row of the wave: pages below it need no mask
  int pn = col_ok ? p_own : 0x7fffffff;
#pragma unroll
  for (int b = 1; b < 16; b <<= 1) pn = min(pn, __shfl_xor(pn, b));
  const int pmin = __builtin_amdgcn_readfirstlane(pn);
  __syncthreads();  // the query rows are in registers; the K region is free for the codes

  f16x8 ONES;
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) ONES[sl] = static_cast<_Float16>(1.0f);
  f16x8 C0N;
#pragma unroll
  for (int sl = 0; sl < 8; ++sl) C0N[sl] = static_cast<_Float16>(-0.5f * ((1 << VB) - 1));

  float m_run = -INFINITY;  // column nl (QK layout)
  float l_part = 0.f;       // this lane's keys only; rows merged at the end
  float acc[8][4];          // PV layout: row 4*gr + i, channel 16*nb + nl (rotated domain)
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[nb][i] = 0.f;

  // online-softmax step shared by the pages and the tail: new running max from lg, returns alpha
  auto softmax_step = [&](const float (&lg)[8][4], float& m_new_out, bool& live_out) {
    float mloc = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, lg[mb][i]);
    mloc = rows_max4(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = m_new;
    m_new_out = m_new;
    live_out = live;
    return alpha;
  };

  // ---- quantised pages --------------------------------------------------------------------------
  // The page count is the workgroup's (its last row sees the most keys), so that every wave takes
  // part in converting every page; a wave whose rows see none of a page skips its own arithmetic.
  int n_pages = 0;
  {
    const int i_last = min(n - 1, (row0 + kRowsPerBlock - 1) / G);
    const int p_last = L - n + i_last;
    n_pages = min(full, (p_last >> 7) + 1);
  }
  const int64_t pt_row = static_cast<int64_t>(s) * max_pages;
  const int64_t head_off = static_cast<int64_t>(h) * R;
  PageShare<KB, VB> share;
  if (n_pages > 0) {
    const uint8_t* rec = cache + static_cast<int64_t>(page_table[pt_row]) * page_stride + head_off;
    load_share<KB, VB>(share, record_rsrc(rec, R), wave, lane);
    copy_scale_share<KB, VB, NG>(stage[0], rec, wave, lane);
  }
  for (int p = 0; p < n_pages; ++p) {
    if constexpr (NSTAGE == 1) {
      // one stage: page p's scales are copied only now that page p - 1 is done with it
      if (p > 0)
        copy_scale_share<KB, VB, NG>(stage[0],
                                     cache + static_cast<int64_t>(page_table[pt_row + p]) * page_stride + head_off,
                                     wave, lane);
    }
    // this wave's share of page p: codes in registers, scales in the stage
    vmcnt_wait<0>();
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if constexpr (NG == 1)
          kdq[2 * wave + m][kb][lane] = dequant_k<KB>(share.k[m], kb);
        else
          kdq[2 * wave + m][kb][lane] = dequant_k_grouped<KB>(share.k[m], kb);
        vdq[2 * wave + m][kb][lane] = dequant_v<VB>(share.v[m], kb);
      }
    __syncthreads();  // page p complete in LDS
    if (p + 1 < n_pages) {
      // page p + 1 in flight while page p is computed; its stage was last read for page p - 1
      const uint8_t* rec = cache + static_cast<int64_t>(page_table[pt_row + p + 1]) * page_stride + head_off;
      load_share<KB, VB>(share, record_rsrc(rec, R), wave, lane);
      if constexpr (NSTAGE == 2) copy_scale_share<KB, VB, NG>(stage[(p + 1) & 1], rec, wave, lane);
    }
    const float* const sp = stage[p % NSTAGE];

    if (128 * p <= pmax) {
      // q'' = c_K ⊙ q' of this lane's row as the QK B operand, fp16 hi + lo
      f16x8 bqh[4], bql[4];
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const float4 c4 = *reinterpret_cast<const float4*>(sp + 4 * gr + 16 * e8);
        const float x[4] = {c4.x * qv[e8].x, c4.y * qv[e8].y, c4.z * qv[e8].z, c4.w * qv[e8].w};
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
      // sigma_g = sum_j q''_j over quantisation group g (k-steps 4g/NG .. 4(g+1)/NG - 1)
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

      // QK and the causal mask: key 128 p + 16 mb + 4 gr + i against the row's last position
      float lg[8][4];
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        f32x4 dg[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) dg[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f16x8 a = kdq[mb][kb][lane];
          dg[kb * NG / 4] = mfma16(a, bqh[kb], dg[kb * NG / 4]);
          dg[kb * NG / 4] = mfma16(a, bql[kb], dg[kb * NG / 4]);
        }
        // the groups' terms summed from the first one (no 0 + x, which the compiler must keep)
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const float4 sk = *reinterpret_cast<const float4*>(sp + kCh * (1 + g) + 16 * mb + 4 * gr);
          const float4 mk = *reinterpret_cast<const float4*>(sp + kCh * (1 + NG + g) + 16 * mb + 4 * gr);
          const float t[4] = {fmaf(sk.x, dg[g][0], mk.x * sigma[g]), fmaf(sk.y, dg[g][1], mk.y * sigma[g]),
                              fmaf(sk.z, dg[g][2], mk.z * sigma[g]), fmaf(sk.w, dg[g][3], mk.w * sigma[g])};
#pragma unroll
          for (int i = 0; i < 4; ++i) lg[mb][i] = g == 0 ? t[i] : lg[mb][i] + t[i];
        }
      }
      if (128 * p + 127 > pmin) {
        // the page reaches past some row's last visible key
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (128 * p + 16 * mb + 4 * gr + i > p_own) lg[mb][i] = -INFINITY;
      }

      float m_new;
      bool live;
      const float alpha = softmax_step(lg, m_new, live);
      // a row with no live key subtracts +inf: every exponent is -inf, every p_t 0, with no select per key
      const float m_sub = live ? m_new : INFINITY;

      // PV weights w_t = p_t s'_t (s' of the token's V group) go to the MFMA in fp16, divided by the
      // row's largest weight on this page over all groups (W) so that none of the weights that matter
      // falls into fp16's subnormal range (small token scales of 8-bit values, spread attention); the
      // row's PV result is multiplied back by W.  (W is bounded below: where every weight on the page
      // is that small, the page is negligible against the row's running sum, and 1 / W must not
      // overflow; the weights then round to fp16 zeros.)  With one group, lg keeps w_t after this loop.
      constexpr float c0 = 0.5f * ((1 << VB) - 1);
      float psum = 0.f, wmax = 0.f, msum1 = 0.f;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        float smax[4];
        if constexpr (NG == 1) {
          const float4 sv = *reinterpret_cast<const float4*>(sp + HS + kCh + 16 * mb + 4 * gr);
          const float4 mv = *reinterpret_cast<const float4*>(sp + HS + 2 * kCh + 16 * mb + 4 * gr);
          smax[0] = sv.x;
          smax[1] = sv.y;
          smax[2] = sv.z;
          smax[3] = sv.w;
          const float mvv[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pr = __builtin_amdgcn_exp2f(lg[mb][i] - m_sub);
            psum += pr;
            msum1 = fmaf(pr, mvv[i], msum1);
            lg[mb][i] = pr * smax[i];  // w_t
            wmax = fmaxf(wmax, lg[mb][i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) smax[i] = 0.f;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const float4 sv = *reinterpret_cast<const float4*>(sp + HS + kCh * (1 + g) + 16 * mb + 4 * gr);
            smax[0] = fmaxf(smax[0], sv.x);
            smax[1] = fmaxf(smax[1], sv.y);
            smax[2] = fmaxf(smax[2], sv.z);
            smax[3] = fmaxf(smax[3], sv.w);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            lg[mb][i] = __builtin_amdgcn_exp2f(lg[mb][i] - m_sub);  // p_t
            psum += lg[mb][i];
            wmax = fmaxf(wmax, lg[mb][i] * smax[i]);
          }
        }
      }
      wmax = rows_max4(wmax);
      const float wscale = fmaxf(wmax, kMinWeightScale);
      const float inv_ws = __builtin_amdgcn_rcpf(wscale);  // within 1 ulp; the result is multiplied by wscale
      l_part = l_part * alpha + psum;
      float arow[4], wrow[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        arow[i] = __shfl(alpha, 4 * gr + i);
        wrow[i] = __shfl(wscale, 4 * gr + i);
      }
#pragma unroll
      for (int gv = 0; gv < NG; ++gv) {
        f16x8 aw[4];
        float msum = msum1, wexact = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int mb = 2 * kb + hh;
            float wv[4];
            if constexpr (NG == 1) {
#pragma unroll
              for (int r = 0; r < 4; ++r) wv[r] = lg[mb][r] * inv_ws;
            } else {
              const float4 sv = *reinterpret_cast<const float4*>(sp + HS + kCh * (1 + gv) + 16 * mb + 4 * gr);
              const float4 mv = *reinterpret_cast<const float4*>(sp + HS + kCh * (1 + NG + gv) + 16 * mb + 4 * gr);
              const float svv[4] = {sv.x, sv.y, sv.z, sv.w};
              const float mvv[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                msum = fmaf(lg[mb][r], mvv[r], msum);
                wv[r] = lg[mb][r] * svv[r] * inv_ws;
              }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              aw[kb][vslot<VB>(hh, r)] = static_cast<_Float16>(wv[r]);
              wexact += wv[r];
            }
          }
        const f32x4 corr = pv_zero_point<VB>(aw, fmaf(c0, wexact, msum * inv_ws), C0N);
#pragma unroll
        for (int nb = EV * gv; nb < EV * gv + EV; ++nb) {
          f32x4 d = corr;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) d = mfma16(aw[kb], vdq[nb][kb][lane], d);
          const float cv = sp[HS + 16 * nb + nl];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[nb][i] = fmaf(acc[nb][i], arow[i], cv * wrow[i] * d[i]);
        }
      }
    }
    __syncthreads();  // every wave is done with page p's codes before page p + 1 overwrites them
  }

  // ---- the fp16 tail, raw domain ------------------------------------------------------------------
  float acc_raw[8][4];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_raw[nb][i] = 0.f;
  if (nt > 0) {
    // tail V transposed into LDS (channel-major, tokens in PV slot order); tokens >= nt are zeros
    const int64_t tbase = (static_cast<int64_t>(s) * num_kv_heads + h) * kTok * kCh;
    for (int task = tid; task < kTok * 16; task += 256) {
      const int t = task >> 4, c8 = task & 15;
      f16x8 v = zero8();
      if (t < nt) v = *reinterpret_cast<const f16x8*>(tail_v + tbase + static_cast<int64_t>(t) * kCh + 8 * c8);
      const int pos = vt_pos(t);
#pragma unroll
      for (int k = 0; k < 8; ++k) vt[8 * c8 + k][pos] = v[k];
    }
    __syncthreads();

    if (pmax >= 128 * full) {
      // raw q of this lane's row as the B operand, natural channel order (k-step kk: 32 kk + 8 gr + sl)
      f16x8 bq[4];
      const int g_own = rg_own - i_own * G;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) bq[kk] = zero8();
      if (col_ok) {
        const _Float16* qp = q + ((static_cast<int64_t>(s) * max_q + i_own) * num_q_heads + h * G + g_own) * kCh;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) bq[kk] = *reinterpret_cast<const f16x8*>(qp + 32 * kk + 8 * gr);
      }
      float lg[8][4];
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        if (16 * mb < nt) {
          const int kt = 16 * mb + nl;  // A operand row: tail token
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            f16x8 a = zero8();
            if (kt < nt) a = *reinterpret_cast<const f16x8*>(tail_k + tbase + static_cast<int64_t>(kt) * kCh + 32 * kk + 8 * gr);
            d = mfma16(a, bq[kk], d);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * mb + 4 * gr + i;
          lg[mb][i] = (t < nt && 128 * full + t <= p_own) ? d[i] * rawscale : -INFINITY;
        }
      }
      float m_new;
      bool live;
      const float alpha = softmax_step(lg, m_new, live);
      const float m_sub = live ? m_new : INFINITY;
      // weights in fp16 divided by the row's largest (as for the pages), multiplied back after PV
      float pr[8][4];
      float psum = 0.f, wmax = 0.f;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[mb][i] = __builtin_amdgcn_exp2f(lg[mb][i] - m_sub);
          psum += pr[mb][i];
          wmax = fmaxf(wmax, pr[mb][i]);
        }
      wmax = rows_max4(wmax);
      const float wscale = fmaxf(wmax, kMinWeightScale);
      const float inv_ws = __builtin_amdgcn_rcpf(wscale);
      f16x8 aw[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) aw[kb][2 * i + hh] = static_cast<_Float16>(pr[2 * kb + hh][i] * inv_ws);
      l_part = l_part * alpha + psum;
      float arow[4], wrow[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        arow[i] = __shfl(alpha, 4 * gr + i);
        wrow[i] = __shfl(wscale, 4 * gr + i);
      }
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          d = mfma16(aw[kb], *reinterpret_cast<const f16x8*>(&vt[16 * nb + nl][32 * kb + 8 * gr]), d);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[nb][i] *= arow[i];
          acc_raw[nb][i] = fmaf(acc_raw[nb][i], arow[i], wrow[i] * d[i]);
        }
      }
    }
  }

  // ---- out = (Hn acc + acc_raw) / l per row ----------------------------------------------------------
  const float l_col = rows_sum4(l_part);
  float lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lrow[i] = __shfl(l_col, 4 * gr + i);
  // Hadamard over channel j = 16 nb + nl: bits of nb in registers, bits of nl across lanes
#pragma unroll
  for (int b = 1; b < 8; b <<= 1)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      if (!(nb & b)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = acc[nb][i], c = acc[nb | b][i];
          acc[nb][i] = a + c;
          acc[nb | b][i] = a - c;
        }
      }
#pragma unroll
  for (int b = 1; b < 16; b <<= 1) {
    const bool upper = nl & b;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float o = __shfl_xor(acc[nb][i], b);
        acc[nb][i] = upper ? o - acc[nb][i] : acc[nb][i] + o;
      }
  }
  constexpr float kInvSqrt128 = 0.08838834764831845f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rg = row0 + wave * 16 + 4 * gr + i;
    const int it = rg / G, g = rg - (rg / G) * G;
    if (it < n) {
      const float inv_l = lrow[i] > 0.f ? 1.0f / lrow[i] : 0.f;
      _Float16* o = out + ((static_cast<int64_t>(s) * max_q + it) * num_q_heads + h * G + g) * kCh + nl;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        o[16 * nb] = static_cast<_Float16>((acc[nb][i] * kInvSqrt128 + acc_raw[nb][i]) * inv_l);
    }
  }
}

}  // namespace

#define KVARN_PF_NAME2(N) launch_prefill_ng##N
#define KVARN_PF_NAME(N) KVARN_PF_NAME2(N)
hipError_t KVARN_PF_NAME(KVARN_PREFILL_NG)(int kb, int vb, int group_size, const _Float16* q, const int32_t* q_lens,
                                           int max_q, const uint8_t* cache, int64_t page_stride,
                                           const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                                           const _Float16* tail_k, const _Float16* tail_v, float qscale,
                                           float rawscale, _Float16* out, int num_seqs, int num_kv_heads,
                                           int num_q_heads, int row_blocks, hipStream_t stream) {
  constexpr int NG = KVARN_PREFILL_NG;
  const dim3 grid(num_seqs * num_kv_heads, row_blocks);
#define KVARN_PREFILL_CASE(KB_, VB_, G_)                                                                         \
  if (kb == KB_ && vb == VB_ && group_size == G_) {                                                              \
    hipLaunchKernelGGL((prefill_kernel<KB_, VB_, G_, NG>), grid, dim3(256), 0, stream, q, q_lens, max_q, cache,  \
                       page_stride, page_table, max_pages, seq_lens, tail_k, tail_v, num_q_heads, num_kv_heads, \
                       qscale, rawscale, out);                                                                   \
    return hipGetLastError();                                                                                    \
  }
#define KVARN_PREFILL_BITS(G_)                                                                                  \
  KVARN_PREFILL_CASE(2, 2, G_) KVARN_PREFILL_CASE(2, 4, G_) KVARN_PREFILL_CASE(2, 8, G_)                        \
  KVARN_PREFILL_CASE(4, 2, G_) KVARN_PREFILL_CASE(4, 4, G_) KVARN_PREFILL_CASE(4, 8, G_)                        \
  KVARN_PREFILL_CASE(8, 2, G_) KVARN_PREFILL_CASE(8, 4, G_) KVARN_PREFILL_CASE(8, 8, G_)
  KVARN_PREFILL_BITS(1)
  KVARN_PREFILL_BITS(2)
  KVARN_PREFILL_BITS(4)
  KVARN_PREFILL_BITS(8)
  KVARN_PREFILL_BITS(16)
#undef KVARN_PREFILL_BITS
#undef KVARN_PREFILL_CASE
  return hipErrorInvalidValue;
}

#if KVARN_PREFILL_NG == 1
bool prefill_supported(int kb, int vb, int ng, int group_size) {
  return (kb == 2 || kb == 4 || kb == 8) && (vb == 2 || vb == 4 || vb == 8) && (ng == 1 || ng == 2 || ng == 4) &&
         (group_size == 1 || group_size == 2 || group_size == 4 || group_size == 8 || group_size == 16);
}

int prefill_row_blocks(int max_q, int group_size) {
  return static_cast<int>((static_cast<int64_t>(max_q) * group_size + kRowsPerBlock - 1) / kRowsPerBlock);
}

hipError_t launch_prefill(int kb, int vb, int ng, int group_size, const _Float16* q, const int32_t* q_lens, int max_q,
                          const uint8_t* cache, int64_t page_stride, const int32_t* page_table, int max_pages,
                          const int32_t* seq_lens, const _Float16* tail_k, const _Float16* tail_v, float sm_scale,
                          _Float16* out, int num_seqs, int num_q_heads, int num_kv_heads, hipStream_t stream) {
  if (num_seqs == 0 || max_q == 0) return hipSuccess;
  const float rawscale = sm_scale * kLog2e;
  const float qscale = rawscale * 0.08838834764831845f;
  auto* fn = ng == 1 ? launch_prefill_ng1 : ng == 2 ? launch_prefill_ng2 : ng == 4 ? launch_prefill_ng4 : nullptr;
  if (fn == nullptr) return hipErrorInvalidValue;
  return fn(kb, vb, group_size, q, q_lens, max_q, cache, page_stride, page_table, max_pages, seq_lens, tail_k, tail_v,
            qscale, rawscale, out, num_seqs, num_kv_heads, num_q_heads, prefill_row_blocks(max_q, group_size),
            stream);
}
#endif

}  // namespace kvarn
