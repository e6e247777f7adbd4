// KVarN tile quantiser for gfx950.
//
// One workgroup of 128 threads (2 waves) handles one half (K or V) of one tile
// of one kv head, each wave 64 of the 128 tokens (the append kernel runs both
// halves in one 4-wave workgroup: waves 0-1 K, waves 2-3 V).
// Per tile half ([HYPHO] section "它怎么做到的：四步流水线", steps 1-4;
// [LEHUY] section "Cơ chế hoạt động: Chuẩn hóa phương sai"):
//   1. 128-bit loads of the fp16 tile straight into MFMA A operands,
//   2. rotation Ytilde = X H_128 on the matrix cores (v_mfma_f32_16x16x32_f16;
//      X is exact in fp16 and H is +-1, so the products are exact and only the
//      fp32 accumulation rounds),
//   3. log-space Sinkhorn on A = Ytilde^2 kept in registers: exp(-2u) and
//      exp(-2v) are carried as reciprocals of the row / column sums, so a pass
//      is one FMA per element plus lane reductions (DPP row rotations for the
//      16 lanes that share a token, permlane16/32 swaps for the 4 lane rows
//      that share a channel, LDS for the partner wave),
//   4. asymmetric RTN per token group (128, 64 or 32 contiguous channels) and sub-byte packing
//      straight from the MFMA result layout into the record layout.
// Scaling: with Ytilde = sqrt(128) Y the channel log-scales come out shifted by
// ln(128)/2 and the token log-scales unchanged; the stored values are
// corrected exactly (c_j = sqrt(S_j / 128)).  The token scale exp(u_t)
// cancels from the codes and from s'_t, m'_t (s'_t = e^{u_t} s_t with s_t
// proportional to e^{-u_t}), so the last token pass is not needed.

#include "kvarn_device.h"
#include "kvarn_internal.h"

namespace kvarn {

namespace {

// Per-wave LDS scratch for transposing per-token values across the 16 lanes of a lane row:
// tb[lane][*] holds a lane's per-token partials, wb[row][*] the per-token results broadcast back.
constexpr int kTbStride = 34;  // 32 values + 2 padding floats per lane (8-byte aligned rows)
struct WaveLds {
  float tb[64][kTbStride];
  float wb[4][32];
};

// C-layout of v_mfma_f32_16x16x32_f16 for this wave's 64 tokens x 128 channels:
// y[mb][nb][i] = Ytilde[t = 64*half + 16*mb + 4*gr + i][j = 16*nb + nl].
struct TileRegs {
  f32x4 y[4][8];
};

// All-gather over the 4 lane rows of a value held in the reduce-scatter layout
// (row r holds slot order[r] with order = {0, 2, 1, 3}): returns v[k] = slot k.
__device__ __forceinline__ void rows_allgather4(float s, float (&v)[4]) {
  float a = s, b = s;
  swap16(a, b);  // a: rows 0,1 <- slot 0, rows 2,3 <- slot 1; b: slots 2, 3
  float c = a, d = a;
  swap32(c, d);
  float f = b, g = b;
  swap32(f, g);
  v[0] = c;
  v[1] = d;
  v[2] = f;
  v[3] = g;
}

// Pack codes c = 0 .. N-1 (unrounded value f(c)) at bit BITS*c of the words w: code c goes to byte
// (BITS*c % 32) / 8 of sub-word (BITS*c % 8) / BITS through v_cvt_pk_u8_f32 (round to nearest,
// ties to even, clamp to [0, 255], insert as one byte), and the 8/BITS sub-words of a word are
// merged with shifts by BITS.
template <int BITS, int N, class F, int NW>
__device__ __forceinline__ void pack_codes(F f, uint32_t (&w)[NW]) {
  constexpr int NS = 8 / BITS;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    uint32_t d[NS];
#pragma unroll
    for (int sw = 0; sw < NS; ++sw) d[sw] = 0;
#pragma unroll
    for (int c = 0; c < N; ++c)
      if ((BITS * c) / 32 == k)
        d[(BITS * c % 8) / BITS] = __builtin_amdgcn_cvt_pk_u8_f32(f(c), (BITS * c % 32) / 8, d[(BITS * c % 8) / BITS]);
    uint32_t u = d[0];
#pragma unroll
    for (int sw = 1; sw < NS; ++sw) u |= d[sw] << (BITS * sw);
    w[k] = u;
  }
}

// Codes and stores for one tile half once the channel sums S~_j are known, one quantisation group
// per token (g128).  R holds Ytilde on entry and W = Ytilde exp(-v~) (= Y exp(-v)) afterwards.
template <int BITS>
__device__ __forceinline__ void quantize_store_g128(TileRegs& R, const float (&sfin)[8], uint8_t* rec, int code_off,
                                               int scale_off, bool is_v, int half, int gr, int nl, WaveLds& L) {
  constexpr int qmax = (1 << BITS) - 1;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const float b = __builtin_amdgcn_rsqf(sfin[nb]);  // exp(-v~_j)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) R.y[mb][nb] *= b;
  }

  float* sc = reinterpret_cast<float*>(rec + scale_off);
  const int lane = 16 * gr + nl;
  // per-token min / max: this lane's 8 channels, then the 16 lanes of the row through an LDS
  // transpose (lane nl of a row reduces token k = nl = 4*mb + i of that row)
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mn = R.y[mb][0][i], mx = mn;
#pragma unroll
      for (int nb = 1; nb < 8; ++nb) {
        mn = fminf(mn, R.y[mb][nb][i]);
        mx = fmaxf(mx, R.y[mb][nb][i]);
      }
      *reinterpret_cast<float2*>(&L.tb[lane][2 * (4 * mb + i)]) = make_float2(mn, mx);
    }
  __builtin_amdgcn_wave_barrier();
  float mn_own, mx_own;
  {
    const float2 v0 = *reinterpret_cast<const float2*>(&L.tb[16 * gr][2 * nl]);
    mn_own = v0.x;
    mx_own = v0.y;
#pragma unroll
    for (int l = 1; l < 16; ++l) {
      const float2 v = *reinterpret_cast<const float2*>(&L.tb[16 * gr + l][2 * nl]);
      mn_own = fminf(mn_own, v.x);
      mx_own = fmaxf(mx_own, v.y);
    }
  }
  {
    const float range = mx_own - mn_own;
    const float inv_own = range > 0.f ? qmax * fast_rcp(range) : 0.f;
    const int t = 64 * half + 16 * (nl >> 2) + 4 * gr + (nl & 3);
    sc[128 + t] = range * (1.0f / qmax);
    sc[256 + t] = mn_own;
    *reinterpret_cast<float2*>(&L.wb[gr][2 * nl]) = make_float2(mn_own, inv_own);
  }
  __builtin_amdgcn_wave_barrier();
  float inv[4][4], mnv[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const float4 v = *reinterpret_cast<const float4*>(&L.wb[gr][8 * mb + 4 * ii]);
      mnv[mb][2 * ii] = v.x;
      inv[mb][2 * ii] = v.y;
      mnv[mb][2 * ii + 1] = v.z;
      inv[mb][2 * ii + 1] = v.w;
    }
  if (half == 0 && gr == 0) {
    // c_j = sqrt(S~_j / 128) = S~_j rsq(S~_j) / sqrt(128), within 2 ulp; exactly 1 for S~_j = 128
    // (an all-zero channel)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const float c = sfin[nb] * __builtin_amdgcn_rsqf(sfin[nb]) * 0.08838834764831845f;
      sc[16 * nb + nl] = sfin[nb] == 128.0f ? 1.0f : c;
    }
  }

  // (W - mn) * inv as one FMA; v_cvt_pk_u8_f32 rounds it to the nearest integer (ties to even),
  // clamps to [0, 255] and inserts it as one byte of a word
  float nmi[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) nmi[mb][i] = -mnv[mb][i] * inv[mb][i];
  auto val = [&](int mb, int nb, int i) -> float { return fmaf(R.y[mb][nb][i], inv[mb][i], nmi[mb][i]); };

  if (!is_v) {
    // K unit of token t, lane nl: channels nl + 16e at bit BITS*e
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 64 * half + 16 * mb + 4 * gr + i;
        uint8_t* p = rec + code_off + t * 16 * BITS + nl * BITS;
        if constexpr (BITS == 8) {
          uint32_t w[2];
          pack_codes<BITS, 8>([&](int e) { return val(mb, e, i); }, w);
          *reinterpret_cast<u32x2*>(p) = u32x2{w[0], w[1]};
        } else {
          // 8 codes: 32 bits (4-bit) or the low 16 bits of a word (2-bit)
          uint32_t w[1];
          if constexpr (BITS == 4) {
            pack_codes<BITS, 8>([&](int e) { return val(mb, e, i); }, w);
            *reinterpret_cast<uint32_t*>(p) = w[0];
          } else {
            pack_codes<BITS, 8>([&](int e) { return val(mb, e, i); }, w);
            *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(w[0]);
          }
        }
      }
  } else {
    // V unit (nb, gr, nl, half): tokens (mb, i) at bit BITS*(4mb + i)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      uint8_t* p = rec + code_off + ((nb * 4 + gr) * 16 + nl) * 4 * BITS + half * 2 * BITS;
      constexpr int W = BITS / 2;  // 32-bit words per unit
      uint32_t u[W];
      pack_codes<BITS, 16>([&](int c) { return val(c >> 2, nb, c & 3); }, u);
      if constexpr (W == 1)
        *reinterpret_cast<uint32_t*>(p) = u[0];
      else if constexpr (W == 2)
        *reinterpret_cast<u32x2*>(p) = u32x2{u[0], u[1]};
      else
        *reinterpret_cast<u32x4*>(p) = u32x4{u[0], u[1], u[2], u[3]};
    }
  }
}

// Pack codes c = c0 .. c1-1 of N (unrounded value f(c)) at bit BITS*c of the words w, OR-ed into
// what w holds: code c goes to byte (BITS*c % 32) / 8 of sub-word (BITS*c % 8) / BITS through
// v_cvt_pk_u8_f32 (round to nearest, ties to even, clamp to [0, 255], insert as one byte), and the
// 8/BITS sub-words of a word are merged with shifts by BITS.  c0 and c1 are constants once the
// caller's loops are unrolled.
template <int BITS, int N, class F, int NW>
__device__ __forceinline__ void pack_codes_or(F f, int c0, int c1, uint32_t (&w)[NW]) {
  constexpr int NS = 8 / BITS;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    if ((BITS * c0) / 32 > k || (BITS * (c1 - 1)) / 32 < k) continue;
    uint32_t d[NS];
#pragma unroll
    for (int sw = 0; sw < NS; ++sw) d[sw] = 0;
#pragma unroll
    for (int c = 0; c < N; ++c)
      if (c >= c0 && c < c1 && (BITS * c) / 32 == k)
        d[(BITS * c % 8) / BITS] = __builtin_amdgcn_cvt_pk_u8_f32(f(c), (BITS * c % 32) / 8, d[(BITS * c % 8) / BITS]);
    uint32_t u = d[0];
#pragma unroll
    for (int sw = 1; sw < NS; ++sw) u |= d[sw] << (BITS * sw);
    w[k] |= u;
  }
}

// Codes and stores for one tile half once the channel sums S~_j are known, NG > 1 quantisation
// groups per token.  R holds Ytilde on entry and W = Ytilde exp(-v~) (= Y exp(-v)) afterwards.
// Each token's channels form NG groups of 128/NG contiguous channels (channel blocks nb = EG*gi .. EG*gi + EG - 1 of group gi), each with
// its own (mn, s); the groups are done one after the other so that only one group's per-token
// (mn, 1/s) is held in registers.
template <int BITS, int NG>
__device__ __forceinline__ void quantize_store(TileRegs& R, const float (&sfin)[8], uint8_t* rec, int code_off,
                                               int scale_off, bool is_v, int half, int gr, int nl, WaveLds& L) {
  constexpr int qmax = (1 << BITS) - 1;
  constexpr int EG = 8 / NG;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const float b = __builtin_amdgcn_rsqf(sfin[nb]);  // exp(-v~_j)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) R.y[mb][nb] *= b;
  }

  float* sc = reinterpret_cast<float*>(rec + scale_off);
  const int lane = 16 * gr + nl;
  // the token whose statistics this lane reduces: k = nl = 4*mb + i of its lane row
  const int t_own = 64 * half + 16 * (nl >> 2) + 4 * gr + (nl & 3);
  if (half == 0 && gr == 0) {
    // c_j = sqrt(S~_j / 128) = S~_j rsq(S~_j) / sqrt(128), within 2 ulp; exactly 1 for S~_j = 128
    // (an all-zero channel)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const float c = sfin[nb] * __builtin_amdgcn_rsqf(sfin[nb]) * 0.08838834764831845f;
      sc[16 * nb + nl] = sfin[nb] == 128.0f ? 1.0f : c;
    }
  }

  // K units of this lane's 16 tokens (channels nl + 16e, e = nb), filled group by group
  constexpr int KW = BITS == 8 ? 2 : 1;
  uint32_t kw[4][4][KW];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < KW; ++k) kw[mb][i][k] = 0;

#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    // per-(token, group) min / max: this lane's EG channels, then the 16 lanes of the row through
    // an LDS transpose (lane nl of a row reduces token k = nl = 4*mb + i of that row)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mn = R.y[mb][EG * gi][i], mx = mn;
#pragma unroll
        for (int nb = EG * gi + 1; nb < EG * gi + EG; ++nb) {
          mn = fminf(mn, R.y[mb][nb][i]);
          mx = fmaxf(mx, R.y[mb][nb][i]);
        }
        *reinterpret_cast<float2*>(&L.tb[lane][2 * (4 * mb + i)]) = make_float2(mn, mx);
      }
    __builtin_amdgcn_wave_barrier();
    float mn_own, mx_own;
    {
      const float2 v0 = *reinterpret_cast<const float2*>(&L.tb[16 * gr][2 * nl]);
      mn_own = v0.x;
      mx_own = v0.y;
#pragma unroll
      for (int l = 1; l < 16; ++l) {
        const float2 v = *reinterpret_cast<const float2*>(&L.tb[16 * gr + l][2 * nl]);
        mn_own = fminf(mn_own, v.x);
        mx_own = fmaxf(mx_own, v.y);
      }
    }
    {
      const float range = mx_own - mn_own;
      const float inv_own = range > 0.f ? qmax * fast_rcp(range) : 0.f;
      sc[kCh + kCh * gi + t_own] = range * (1.0f / qmax);
      sc[kCh + kCh * NG + kCh * gi + t_own] = mn_own;
      *reinterpret_cast<float2*>(&L.wb[gr][2 * nl]) = make_float2(mn_own, inv_own);
    }
    __builtin_amdgcn_wave_barrier();
    float inv[4][4], nmi[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const float4 v = *reinterpret_cast<const float4*>(&L.wb[gr][8 * mb + 4 * ii]);
        inv[mb][2 * ii] = v.y;
        nmi[mb][2 * ii] = -v.x * v.y;
        inv[mb][2 * ii + 1] = v.w;
        nmi[mb][2 * ii + 1] = -v.z * v.w;
      }
    __builtin_amdgcn_wave_barrier();

    // (W - mn) * inv as one FMA; v_cvt_pk_u8_f32 rounds it to the nearest integer (ties to even),
    // clamps to [0, 255] and inserts it as one byte of a word
    auto val = [&](int mb, int nb, int i) -> float { return fmaf(R.y[mb][nb][i], inv[mb][i], nmi[mb][i]); };
    if (!is_v) {
      // K unit of token t, lane nl: channels nl + 16e at bit BITS*e; stored with its last group
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pack_codes_or<BITS, 8>([&](int e) { return val(mb, e, i); }, EG * gi, EG * gi + EG, kw[mb][i]);
          if (gi == NG - 1) {
            const int t = 64 * half + 16 * mb + 4 * gr + i;
            uint8_t* p = rec + code_off + t * 16 * BITS + nl * BITS;
            if constexpr (BITS == 8)
              *reinterpret_cast<u32x2*>(p) = u32x2{kw[mb][i][0], kw[mb][i][1]};
            else if constexpr (BITS == 4)
              *reinterpret_cast<uint32_t*>(p) = kw[mb][i][0];
            else
              *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(kw[mb][i][0]);
          }
        }
    } else {
      // V unit (nb, gr, nl, half): tokens (mb, i) at bit BITS*(4mb + i)
#pragma unroll
      for (int nb = EG * gi; nb < EG * gi + EG; ++nb) {
        uint8_t* p = rec + code_off + ((nb * 4 + gr) * 16 + nl) * 4 * BITS + half * 2 * BITS;
        constexpr int W = BITS / 2;  // 32-bit words per unit
        uint32_t u[W];
#pragma unroll
        for (int k = 0; k < W; ++k) u[k] = 0;
        pack_codes_or<BITS, 16>([&](int c) { return val(c >> 2, nb, c & 3); }, 0, 16, u);
        if constexpr (W == 1)
          *reinterpret_cast<uint32_t*>(p) = u[0];
        else if constexpr (W == 2)
          *reinterpret_cast<u32x2*>(p) = u32x2{u[0], u[1]};
        else
          *reinterpret_cast<u32x4*>(p) = u32x4{u[0], u[1], u[2], u[3]};
      }
    }
  }
}

// MFMA A operands of this wave's 64 tokens: token 16*mb + nl, channels 32*k4 + 8*gr + s.
__device__ __forceinline__ void load_x(f16x8 (&xa)[4][4], const _Float16* __restrict__ x, int64_t row_stride,
                                       const _Float16* __restrict__ last_row, int half, int gr, int nl) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int t = 64 * half + 16 * mb + nl;
    const _Float16* row = (last_row != nullptr && t == kTok - 1) ? last_row : x + t * row_stride;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) xa[mb][k4] = *reinterpret_cast<const f16x8*>(row + 32 * k4 + 8 * gr);
  }
}

// Ytilde = X H_128 on the matrix cores.  Entry (k, n) of H is (-1)^popcount(k & n) with
// k = 32*k4 + 8*gr + s and n = 16*nb + nl; it splits into a lane pattern (s, gr bit 0, nl),
// a lane sign for odd nb (gr bit 1) and a sign uniform over the wave (popcount(k4 & (nb >> 1))).
__device__ __forceinline__ void rotate(const f16x8 (&xa)[4][4], TileRegs& R, int gr, int nl) {
  f16x8 P0, N0, P1, N1;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int par = __builtin_popcount(s & (nl & 7)) + (gr & 1) * (nl >> 3);
    P0[s] = (par & 1) ? static_cast<_Float16>(-1.0f) : static_cast<_Float16>(1.0f);
  }
  N0 = -P0;
  P1 = (gr >> 1) ? N0 : P0;
  N1 = -P1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const bool u = __builtin_popcount(k4 & (nb >> 1)) & 1;
        const f16x8 B = (nb & 1) ? (u ? N1 : P1) : (u ? N0 : P0);
        c = mfma16(xa[mb][k4], B, c);
      }
      R.y[mb][nb] = c;
    }
}

}  // namespace

// Quantise the tile half owned by this pair of waves and write its part of the
// record.  x: token 0, channel 0; row t at x + t*row_stride (halves); when
// last_row is non-null token 127 is read from there.  xch: LDS [2][4][64].
template <int KB, int VB, int NG>
__device__ __forceinline__ void quantize_tile_half(const _Float16* __restrict__ x, int64_t row_stride,
                                                   const _Float16* __restrict__ last_row, uint8_t* __restrict__ rec,
                                                   int iters, bool is_v, float2 (*xch)[4][64], WaveLds* wlds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = wave & 1;
  const int nl = lane & 15, gr = lane >> 4;
  WaveLds& L = wlds[wave];
  // Every row / column sum starts at kEps: a sum over an all-zero row or column stays positive, its
  // reciprocal only ever multiplies zeros, and no zero test is needed in the iterations.
  constexpr float kEps = 1e-30f;

  // 1-2. load the tile half and rotate it on the matrix cores; only A = Ytilde^2 is kept through
  //      the Sinkhorn iterations (Ytilde is recomputed afterwards, so a wave needs 128 values per lane
  //      and two waves fit on each SIMD)
  TileRegs R;
  {
    f16x8 xa[4][4];
    load_x(xa, x, row_stride, last_row, half, gr, nl);
    // all 16 loads in flight before the first MFMA waits on one
    __builtin_amdgcn_sched_barrier(0);
    rotate(xa, R, gr, nl);
  }
  auto& A = R.y;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) A[mb][nb] *= A[mb][nb];

  // 3. Sinkhorn.  w[mb][i] = exp(-2u_t)/128 (token weights), e[nb] = exp(-2v~_j).
  float w[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) w[mb][i] = 1.0f / 128.0f;
  float sfin[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) sfin[nb] = 128.0f;  // v~ = ln(128)/2 <=> v = 0 (no iterations)

  for (int it = 0; it < iters; ++it) {
    // channel pass: S~_j = sum_t A_tj w_t
    float p[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      float acc = 0.f;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(A[mb][nb][i], w[mb][i], acc);
      p[nb] = acc;
    }
    // reduce over the 4 lane rows: s0 holds nb = {0,2,1,3}[gr], s1 holds nb = {4,6,5,7}[gr]
    float s0 = red16(red32(p[0], p[1]), red32(p[2], p[3]));
    float s1 = red16(red32(p[4], p[5]), red32(p[6], p[7]));
    // and over the partner wave (tokens of the other 64-row half)
    float2(*buf)[64] = xch[it & 1];
    buf[wave][lane] = make_float2(s0, s1);
    __syncthreads();
    const float2 o = buf[wave ^ 1][lane];
    // own + partner is commutative, so both waves of the pair hold identical sums
    s0 += o.x;
    s1 += o.y;
    const bool last = (it == iters - 1);
    if (last) {
      // an all-zero channel (sum exactly 0) keeps log-scale 0: stored c_j = 1 <=> S~_j = 128
      float v[4];
      rows_allgather4(s0 > 0.f ? s0 : 128.0f, v);
#pragma unroll
      for (int k = 0; k < 4; ++k) sfin[k] = v[k];
      rows_allgather4(s1 > 0.f ? s1 : 128.0f, v);
#pragma unroll
      for (int k = 0; k < 4; ++k) sfin[4 + k] = v[k];
    } else {
    s0 += kEps;
    s1 += kEps;
    float e[8];
    {
      float v[4];
      rows_allgather4(fast_rcp(s0), v);
#pragma unroll
      for (int k = 0; k < 4; ++k) e[k] = v[k];
      rows_allgather4(fast_rcp(s1), v);
#pragma unroll
      for (int k = 0; k < 4; ++k) e[4 + k] = v[k];
    }
    // token pass: R_t = sum_j A_tj e_j.  Each lane forms 16 partials (its 8 channels); the 16 lanes
    // of a row are summed through an LDS transpose, lane nl owning token 4*mb + i = nl, whose
    // reciprocal is broadcast back to the row.
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          a0 = fmaf(A[mb][nb][2 * ii], e[nb], a0);
          a1 = fmaf(A[mb][nb][2 * ii + 1], e[nb], a1);
        }
        *reinterpret_cast<float2*>(&L.tb[lane][4 * mb + 2 * ii]) = make_float2(a0, a1);
      }
    __builtin_amdgcn_wave_barrier();
    {
      float r = kEps;
#pragma unroll
      for (int l = 0; l < 16; ++l) r += L.tb[16 * gr + l][nl];
      L.wb[gr][nl] = fast_rcp(r);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const float4 v = *reinterpret_cast<const float4*>(&L.wb[gr][4 * mb]);
      w[mb][0] = v.x;
      w[mb][1] = v.y;
      w[mb][2] = v.z;
      w[mb][3] = v.w;
    }
    }
  }

  // 4. Ytilde again (the tile is still in L2), then codes, scales, stores
  {
    f16x8 xa[4][4];
    load_x(xa, x, row_stride, last_row, half, gr, nl);
    rotate(xa, R, gr, nl);
  }
  // 4. codes, scales, stores
  const int code_off = is_v ? k_code_bytes(KB) : 0;
  const int scale_off = scale_offset(KB, VB) + (is_v ? half_scale_floats(NG) * 4 : 0);
  if constexpr (NG == 1) {
    if (is_v)
      quantize_store_g128<VB>(R, sfin, rec, code_off, scale_off, is_v, half, gr, nl, L);
    else
      quantize_store_g128<KB>(R, sfin, rec, code_off, scale_off, is_v, half, gr, nl, L);
  } else {
    if (is_v)
      quantize_store<VB, NG>(R, sfin, rec, code_off, scale_off, is_v, half, gr, nl, L);
    else
      quantize_store<KB, NG>(R, sfin, rec, code_off, scale_off, is_v, half, gr, nl, L);
  }
}

// One workgroup of 2 waves per (tile, kv head, half): the K and V halves of a tile are independent,
// so the per-pass barrier only couples the two waves that share a half.
template <int KB, int VB, int NG>
__global__ __launch_bounds__(128, 2) void quantize_tiles_kernel(const _Float16* __restrict__ k,
                                                                const _Float16* __restrict__ v,
                                                                const int32_t* __restrict__ dst_pages,
                                                                uint8_t* __restrict__ cache, int64_t page_stride,
                                                                int num_kv_heads, int iters) {
  __shared__ float2 xch[2][4][64];
  __shared__ WaveLds wlds[2];
  const int th = blockIdx.x >> 1;
  const bool is_v = blockIdx.x & 1;
  const int tile = th / num_kv_heads;
  const int h = th - tile * num_kv_heads;
  const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * kCh;
  const _Float16* src = (is_v ? v : k) + (static_cast<int64_t>(tile) * kTok * num_kv_heads + h) * kCh;
  uint8_t* rec = cache + static_cast<int64_t>(dst_pages[tile]) * page_stride +
                 static_cast<int64_t>(h) * record_bytes(KB, VB, NG);
  quantize_tile_half<KB, VB, NG>(src, row_stride, nullptr, rec, iters, is_v, xch, wlds);
}

// Token append: one workgroup per (sequence, kv head).  Writes the new token into
// the fp16 tail at len % 128 and, when that fills the tile, quantises the tail
// (token 127 read from the new token itself) into page_table[s][len / 128].
// The length is read and advanced in the same launch: each workgroup of sequence s adds
// 1 << kArrivalShift to seq_lens[s] and takes len from the low bits of the old value, and the one
// that counts the last arrival takes the count back out and adds the new token.  Every workgroup
// thus reads len before any change to the low bits (len < 2^kArrivalShift; at most 64 kv heads,
// so the word never overflows).
template <int KB, int VB, int NG>
__global__ __launch_bounds__(256, 2) void append_kernel(const _Float16* __restrict__ k_new,
                                                        const _Float16* __restrict__ v_new,
                                                        int32_t* __restrict__ seq_lens,
                                                        _Float16* __restrict__ tail_k, _Float16* __restrict__ tail_v,
                                                        const int32_t* __restrict__ page_table, int max_pages,
                                                        uint8_t* __restrict__ cache, int64_t page_stride,
                                                        int num_kv_heads, int iters) {
  __shared__ float2 xch[2][4][64];
  __shared__ WaveLds wlds[4];
  const int sh = blockIdx.x;
  const int s = sh / num_kv_heads;
  const int h = sh - s * num_kv_heads;
  __shared__ int len_sh;
  if (threadIdx.x == 0) {
    const int old = atomicAdd(seq_lens + s, 1 << kArrivalShift);
    len_sh = old & ((1 << kArrivalShift) - 1);
    if ((old >> kArrivalShift) == num_kv_heads - 1) atomicAdd(seq_lens + s, 1 - (num_kv_heads << kArrivalShift));
  }
  __syncthreads();
  const int len = len_sh;
  const int slot = len & (kTok - 1);
  const int64_t tail_base = static_cast<int64_t>(sh) * kTok * kCh;
  const int tid = threadIdx.x;
  if (tid < 32) {
    const bool isv = tid >= 16;
    const _Float16* src = (isv ? v_new : k_new) + static_cast<int64_t>(sh) * kCh + 8 * (tid & 15);
    _Float16* dst = (isv ? tail_v : tail_k) + tail_base + slot * kCh + 8 * (tid & 15);
    *reinterpret_cast<f16x8*>(dst) = *reinterpret_cast<const f16x8*>(src);
  }
  if (slot == kTok - 1) {
    const bool is_v = (tid >> 6) >= 2;
    const _Float16* x = (is_v ? tail_v : tail_k) + tail_base;
    const _Float16* last = (is_v ? v_new : k_new) + static_cast<int64_t>(sh) * kCh;
    const int page = page_table[static_cast<int64_t>(s) * max_pages + (len >> 7)];
    uint8_t* rec =
        cache + static_cast<int64_t>(page) * page_stride + static_cast<int64_t>(h) * record_bytes(KB, VB, NG);
    quantize_tile_half<KB, VB, NG>(x, kCh, last, rec, iters, is_v, xch, wlds);
  }
}

// (kb, vb, groups per token) -> the kernel instantiation for that format
#define KVARN_FOR_EACH_BITS(X, NG) \
  X(2, 2, NG) X(2, 4, NG) X(2, 8, NG) X(4, 2, NG) X(4, 4, NG) X(4, 8, NG) X(8, 2, NG) X(8, 4, NG) X(8, 8, NG)
#define KVARN_FOR_EACH_FORMAT(X) KVARN_FOR_EACH_BITS(X, 1) KVARN_FOR_EACH_BITS(X, 2) KVARN_FOR_EACH_BITS(X, 4)

hipError_t launch_quantize_tiles(const _Float16* k, const _Float16* v, const int32_t* dst_pages, uint8_t* cache,
                                 int64_t page_stride, int num_tiles, int num_kv_heads, int kb, int vb, int ng,
                                 int iters, hipStream_t stream) {
  if (num_tiles == 0) return hipSuccess;
#define KVARN_Q(KB_, VB_, NG_)                                                                                      \
  if (kb == KB_ && vb == VB_ && ng == NG_) {                                                                        \
    hipLaunchKernelGGL((quantize_tiles_kernel<KB_, VB_, NG_>), dim3(2 * num_tiles * num_kv_heads), dim3(128), 0,    \
                       stream,                                                                                       \
                       k, v, dst_pages, cache, page_stride, num_kv_heads, iters);                                   \
    return hipGetLastError();                                                                                       \
  }
  KVARN_FOR_EACH_FORMAT(KVARN_Q)
#undef KVARN_Q
  return hipErrorInvalidValue;
}

hipError_t launch_append(const _Float16* k_new, const _Float16* v_new, int32_t* seq_lens, _Float16* tail_k,
                         _Float16* tail_v, const int32_t* page_table, int max_pages, uint8_t* cache,
                         int64_t page_stride, int num_seqs, int num_kv_heads, int kb, int vb, int ng, int iters,
                         hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  hipError_t e = hipErrorInvalidValue;
#define KVARN_A(KB_, VB_, NG_)                                                                                     \
  if (kb == KB_ && vb == VB_ && ng == NG_) {                                                                       \
    hipLaunchKernelGGL((append_kernel<KB_, VB_, NG_>), dim3(num_seqs * num_kv_heads), dim3(256), 0, stream, k_new, \
                       v_new, seq_lens, tail_k, tail_v, page_table, max_pages, cache, page_stride, num_kv_heads,    \
                       iters);                                                                                     \
    e = hipGetLastError();                                                                                         \
  }
  KVARN_FOR_EACH_FORMAT(KVARN_A)
#undef KVARN_A
  return e;
}

}  // namespace kvarn
