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
// MFMA columns of a wave are its 16 query rows.  Per page the wave does what the decode kernel does
// for one page: QK with the K codes as the A operand and q'' = c_K ⊙ q' (fp16 hi + lo) as the B
// operand, logits s' (q'' . codes) + m' sigma, the causal mask, an online softmax per row, and PV
// with the fp16 weights p_t s'_t against the V codes (the zero-point sum as in decode, channel
// scale c_V on the result).  The fp16 tail is attended in the raw domain: raw q against raw K rows,
// then the weights against the tail V staged in LDS transposed; that accumulator is added once Hn
// has been applied to the rotated one.  Only one group per token (g128) is supported here.

#include "kvarn_codes.h"
#include "kvarn_device.h"
#include "kvarn_internal.h"

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

// lgkmcnt(0): every LDS read of this wave has returned (vmcnt and expcnt not waited for)
__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

template <int KB, int VB, int G>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const _Float16* __restrict__ q,
                                                         const int32_t* __restrict__ q_lens, int max_q,
                                                         const uint8_t* __restrict__ cache, int64_t page_stride,
                                                         const int32_t* __restrict__ page_table, int max_pages,
                                                         const int32_t* __restrict__ seq_lens,
                                                         const _Float16* __restrict__ tail_k,
                                                         const _Float16* __restrict__ tail_v, int num_q_heads,
                                                         int num_kv_heads, float qscale, float rawscale,
                                                         _Float16* __restrict__ out) {
  constexpr int R = record_bytes(KB, VB, 1);
  constexpr int SC = 2 * half_scale_floats(1);   // 768 floats of scales per page
  __shared__ __attribute__((aligned(16))) float qrot[kRowsPerBlock][kCh];
  __shared__ __attribute__((aligned(16))) float stage[4][SC];
  __shared__ __attribute__((aligned(16))) _Float16 vt[kCh][kTok];

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

  float4 qv[8];
#pragma unroll
  for (int e8 = 0; e8 < 8; ++e8) qv[e8] = *reinterpret_cast<const float4*>(&qrot[wave * 16 + nl][4 * gr + 16 * e8]);
  const bool col_ok = p_own >= 0;

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
  const int n_pages = pmax < 0 ? 0 : min(full, (pmax >> 7) + 1);
  const int64_t pt_row = static_cast<int64_t>(s) * max_pages;
  const int64_t head_off = static_cast<int64_t>(h) * R;
  float* const sown = stage[wave];
  for (int p = 0; p < n_pages; ++p) {
    const int phys = page_table[pt_row + p];
    const uint8_t* rec[1] = {cache + static_cast<int64_t>(phys) * page_stride + head_off};
    const __amdgpu_buffer_rsrc_t rs[1] = {record_rsrc(rec[0], R)};
    KHalf<KB, 1> klo, khi;
    VAll<VB, 1> vc;
    load_k_half<KB, 1>(klo, rs, 0, lane);
    load_k_half<KB, 1>(khi, rs, 1, lane);
    load_v_all<KB, VB, 1>(vc, rs, lane);
    lgkm_wait0();  // the previous page's scale reads are done before the stage is overwritten
    copy_scales<KB, VB, 1, 1>(sown, rec, lane);
    vmcnt_wait<0>();

    // q'' = c_K ⊙ q' of this lane's row as the QK B operand, fp16 hi + lo
    f16x8 bqh[4], bql[4];
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const float4 c4 = *reinterpret_cast<const float4*>(sown + 4 * gr + 16 * e8);
      const float x[4] = {col_ok ? c4.x * qv[e8].x : 0.f, col_ok ? c4.y * qv[e8].y : 0.f,
                          col_ok ? c4.z * qv[e8].z : 0.f, col_ok ? c4.w * qv[e8].w : 0.f};
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
    }
    float sigma;
    {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        d = mfma16(ONES, bqh[kb], d);
        d = mfma16(ONES, bql[kb], d);
      }
      sigma = d[0];
    }

    // QK and the causal mask: key 128 p + 16 mb + 4 gr + i against the row's last position
    float lg[8][4];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f16x8 a = dequant_k<KB>(mb < 4 ? klo.k[0][mb] : khi.k[0][mb - 4], kb);
        d = mfma16(a, bqh[kb], d);
        d = mfma16(a, bql[kb], d);
      }
      const float4 sk = *reinterpret_cast<const float4*>(sown + 128 + 16 * mb + 4 * gr);
      const float4 mk = *reinterpret_cast<const float4*>(sown + 256 + 16 * mb + 4 * gr);
      const float skk[4] = {sk.x, sk.y, sk.z, sk.w}, mkk[4] = {mk.x, mk.y, mk.z, mk.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 128 * p + 16 * mb + 4 * gr + i;
        lg[mb][i] = key <= p_own ? fmaf(skk[i], d[i], mkk[i] * sigma) : -INFINITY;
      }
    }

    float m_new;
    bool live;
    const float alpha = softmax_step(lg, m_new, live);

    // PV weights w_t = p_t s'_t go to the MFMA in fp16, divided by the row's largest weight on this
    // page (W) so that none of the weights that matter falls into fp16's subnormal range (small
    // token scales of 8-bit values, spread attention); the row's PV result is multiplied back by W.
    // The zero-point sum is carried as in decode (codes centred on c0 through one MFMA against -c0).
    constexpr float c0 = 0.5f * ((1 << VB) - 1);
    float wv[8][4];
    float msum = 0.f, psum = 0.f, wmax = 0.f;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const float4 sv = *reinterpret_cast<const float4*>(sown + 4 * 128 + 16 * mb + 4 * gr);
      const float4 mv = *reinterpret_cast<const float4*>(sown + 5 * 128 + 16 * mb + 4 * gr);
      const float svv[4] = {sv.x, sv.y, sv.z, sv.w};
      const float mvv[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = live ? __builtin_amdgcn_exp2f(lg[mb][i] - m_new) : 0.f;
        psum += pr;
        msum = fmaf(pr, mvv[i], msum);
        wv[mb][i] = pr * svv[i];
        wmax = fmaxf(wmax, wv[mb][i]);
      }
    }
    // (bounded below: where every weight on the page is that small, the page is negligible against
    // the row's running sum, and 1 / wmax must not overflow; the weights then round to fp16 zeros)
    wmax = rows_max4(wmax);
    const float wscale = fmaxf(wmax, kMinWeightScale);
    const float inv_ws = 1.0f / wscale;
    msum *= inv_ws;
    f16x8 aw[4];
    float wexact = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x0 = wv[2 * kb][r] * inv_ws, x1 = wv[2 * kb + 1][r] * inv_ws;
        aw[kb][vslot<VB>(0, r)] = static_cast<_Float16>(x0);
        aw[kb][vslot<VB>(1, r)] = static_cast<_Float16>(x1);
        wexact += x0 + x1;
      }
    }
    l_part = l_part * alpha + psum;
    const f32x4 corr = pv_zero_point<VB>(aw, fmaf(c0, wexact, msum), C0N);
    float arow[4], wrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      arow[i] = __shfl(alpha, 4 * gr + i);
      wrow[i] = __shfl(wscale, 4 * gr + i);
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      f32x4 d = corr;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) d = mfma16(aw[kb], dequant_v<VB>(vc.v[0][nb], kb), d);
      const float cv = sown[3 * 128 + 16 * nb + nl];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[nb][i] = fmaf(acc[nb][i], arow[i], cv * wrow[i] * d[i]);
    }
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
      // weights in fp16 divided by the row's largest (as for the pages), multiplied back after PV
      float pr[8][4];
      float psum = 0.f, wmax = 0.f;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[mb][i] = live ? __builtin_amdgcn_exp2f(lg[mb][i] - m_new) : 0.f;
          psum += pr[mb][i];
          wmax = fmaxf(wmax, pr[mb][i]);
        }
      wmax = rows_max4(wmax);
      const float wscale = fmaxf(wmax, kMinWeightScale);
      const float inv_ws = 1.0f / wscale;
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

bool prefill_supported(int kb, int vb, int ng, int group_size) {
  return (kb == 2 || kb == 4 || kb == 8) && (vb == 2 || vb == 4 || vb == 8) && ng == 1 &&
         (group_size == 1 || group_size == 2 || group_size == 4 || group_size == 8 || group_size == 16);
}

int prefill_row_blocks(int max_q, int group_size) {
  return static_cast<int>((static_cast<int64_t>(max_q) * group_size + kRowsPerBlock - 1) / kRowsPerBlock);
}

hipError_t launch_prefill(int kb, int vb, int group_size, const _Float16* q, const int32_t* q_lens, int max_q,
                          const uint8_t* cache, int64_t page_stride, const int32_t* page_table, int max_pages,
                          const int32_t* seq_lens, const _Float16* tail_k, const _Float16* tail_v, float sm_scale,
                          _Float16* out, int num_seqs, int num_q_heads, int num_kv_heads, hipStream_t stream) {
  if (num_seqs == 0 || max_q == 0) return hipSuccess;
  const float rawscale = sm_scale * kLog2e;
  const float qscale = rawscale * 0.08838834764831845f;
  const dim3 grid(num_seqs * num_kv_heads, prefill_row_blocks(max_q, group_size));
#define KVARN_PREFILL_CASE(KB_, VB_, G_)                                                                         \
  if (kb == KB_ && vb == VB_ && group_size == G_) {                                                              \
    hipLaunchKernelGGL((prefill_kernel<KB_, VB_, G_>), grid, dim3(256), 0, stream, q, q_lens, max_q, cache,      \
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

}  // namespace kvarn
