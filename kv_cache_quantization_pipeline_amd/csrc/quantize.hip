// KVarN tile quantiser for gfx950.
//
// One workgroup of 256 threads (4 waves) handles one tile of one kv head:
// waves 0-1 the K half, waves 2-3 the V half, each wave 64 of the 128 tokens.
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
//   4. asymmetric RTN per token group of 128 channels and sub-byte packing
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

// C-layout of v_mfma_f32_16x16x32_f16 for this wave's 64 tokens x 128 channels:
// y[mb][nb][i] = Ytilde[t = 64*half + 16*mb + 4*gr + i][j = 16*nb + nl].
struct TileRegs {
  f32x4 y[4][8];
};

template <int BITS>
__device__ __forceinline__ void store_k_unit(uint8_t* p, const uint32_t (&q)[8]) {
  if constexpr (BITS == 4) {
    uint32_t u = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) u |= q[e] << (4 * e);
    *reinterpret_cast<uint32_t*>(p) = u;
  } else if constexpr (BITS == 8) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= q[e] << (8 * e);
      hi |= q[e + 4] << (8 * e);
    }
    *reinterpret_cast<u32x2*>(p) = u32x2{lo, hi};
  } else {  // 2 bits
    uint32_t u = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) u |= q[e] << (2 * e);
    *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(u);
  }
}

template <int BITS>
__device__ __forceinline__ void store_v_unit(uint8_t* p, const uint32_t (&q)[16]) {
  if constexpr (BITS == 2) {
    uint32_t u = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) u |= q[c] << (2 * c);
    *reinterpret_cast<uint32_t*>(p) = u;
  } else if constexpr (BITS == 4) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      lo |= q[c] << (4 * c);
      hi |= q[c + 8] << (4 * c);
    }
    *reinterpret_cast<u32x2*>(p) = u32x2{lo, hi};
  } else {  // 8 bits
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < 16; ++c) w[c >> 2] |= q[c] << (8 * (c & 3));
    *reinterpret_cast<u32x4*>(p) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

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

// Codes and stores for one tile half once the channel sums S~_j are known.
template <int BITS>
__device__ __forceinline__ void quantize_store(const TileRegs& R, const float (&sfin)[8], uint8_t* rec, int code_off,
                                               int scale_off, bool is_v, int half, int gr, int nl) {
  constexpr int qmax = (1 << BITS) - 1;
  float bsc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) bsc[nb] = __builtin_amdgcn_rsqf(sfin[nb]);  // exp(-v~_j)

  float inv[4][4], bias[4][4], sp[4][4], mp[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mn = R.y[mb][0][i] * bsc[0], mx = mn;
#pragma unroll
      for (int nb = 1; nb < 8; ++nb) {
        const float w = R.y[mb][nb][i] * bsc[nb];
        mn = fminf(mn, w);
        mx = fmaxf(mx, w);
      }
      mn = row_min16(mn);
      mx = row_max16(mx);
      const float range = mx - mn;
      sp[mb][i] = range * (1.0f / qmax);
      mp[mb][i] = mn;
      const float iv = range > 0.f ? qmax * fast_rcp(range) : 0.f;
      inv[mb][i] = iv;
      bias[mb][i] = -mn * iv;
    }

  auto code = [&](int mb, int nb, int i) -> uint32_t {
    const float w = R.y[mb][nb][i] * bsc[nb];
    const float t = __builtin_rintf(fmaf(w, inv[mb][i], bias[mb][i]));
    const uint32_t c = static_cast<uint32_t>(fmaxf(t, 0.f));
    return c > qmax ? qmax : c;
  };

  if (!is_v) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t q[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) q[nb] = code(mb, nb, i);
        const int t = 64 * half + 16 * mb + 4 * gr + i;
        store_k_unit<BITS>(rec + code_off + t * 16 * BITS + nl * BITS, q);
      }
  } else {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      uint32_t q[16];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) q[4 * mb + i] = code(mb, nb, i);
      store_v_unit<BITS>(rec + code_off + ((nb * 4 + gr) * 16 + nl) * 4 * BITS + half * 2 * BITS, q);
    }
  }

  float* sc = reinterpret_cast<float*>(rec + scale_off);
  if (half == 0 && gr == 0) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) sc[16 * nb + nl] = __builtin_sqrtf(sfin[nb] * (1.0f / 128.0f));
  }
  if (nl < 4) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const float s = nl == 0 ? sp[mb][0] : nl == 1 ? sp[mb][1] : nl == 2 ? sp[mb][2] : sp[mb][3];
      const float m = nl == 0 ? mp[mb][0] : nl == 1 ? mp[mb][1] : nl == 2 ? mp[mb][2] : mp[mb][3];
      const int t = 64 * half + 16 * mb + 4 * gr + nl;
      sc[128 + t] = s;
      sc[256 + t] = m;
    }
  }
}

}  // namespace

// Quantise the tile half owned by this pair of waves and write its part of the
// record.  x: token 0, channel 0; row t at x + t*row_stride (halves); when
// last_row is non-null token 127 is read from there.  xch: LDS [2][4][64].
__device__ void quantize_tile_half(const _Float16* __restrict__ x, int64_t row_stride,
                                   const _Float16* __restrict__ last_row, uint8_t* __restrict__ rec, int kb,
                                   int vb, int iters, float2 (*xch)[4][64]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = wave & 1;
  const bool is_v = wave >= 2;
  const int nl = lane & 15, gr = lane >> 4;

  // 1. MFMA A operands: token 16*mb + nl of this wave, channels 32*kb + 8*gr + s.
  f16x8 xa[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int t = 64 * half + 16 * mb + nl;
    const _Float16* row = (last_row != nullptr && t == kTok - 1) ? last_row : x + t * row_stride;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) xa[mb][k4] = *reinterpret_cast<const f16x8*>(row + 32 * k4 + 8 * gr);
  }

  // 2. B operands of H_128: entry (k, n) = (-1)^popcount(k & n) with k = 32*kb + 8*gr + s and
  //    n = 16*nb + nl splits into a lane pattern (s, gr bit 0, nl), a lane sign for odd nb
  //    (gr bit 1) and a sign uniform over the wave (popcount(kb & (nb >> 1))).
  f16x8 P0, N0, P1, N1;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int par = __builtin_popcount(s & (nl & 7)) + (gr & 1) * (nl >> 3);
    P0[s] = (par & 1) ? static_cast<_Float16>(-1.0f) : static_cast<_Float16>(1.0f);
  }
  N0 = -P0;
  P1 = (gr >> 1) ? N0 : P0;
  N1 = -P1;

  TileRegs R;
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

  // 3. Sinkhorn.  w[mb][i] = exp(-2u_t)/128 (token weights), e[nb] = exp(-2v~_j).
  float A[4][8][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) A[mb][nb][i] = R.y[mb][nb][i] * R.y[mb][nb][i];

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
    s0 += o.x;
    s1 += o.y;
    const bool last = (it == iters - 1);
    if (last) {
      float v[4];
      rows_allgather4(s0 > 0.f ? s0 : 128.0f, v);
#pragma unroll
      for (int k = 0; k < 4; ++k) sfin[k] = v[k];
      rows_allgather4(s1 > 0.f ? s1 : 128.0f, v);
#pragma unroll
      for (int k = 0; k < 4; ++k) sfin[4 + k] = v[k];
      break;
    }
    float e[8];
    {
      float v[4];
      rows_allgather4(s0 > 0.f ? fast_rcp(s0) : 1.0f / 128.0f, v);
#pragma unroll
      for (int k = 0; k < 4; ++k) e[k] = v[k];
      rows_allgather4(s1 > 0.f ? fast_rcp(s1) : 1.0f / 128.0f, v);
#pragma unroll
      for (int k = 0; k < 4; ++k) e[4 + k] = v[k];
    }
    // token pass: R_t = sum_j A_tj e_j over the 16 lanes of the row
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc = fmaf(A[mb][nb][i], e[nb], acc);
        acc = row_sum16(acc);
        w[mb][i] = acc > 0.f ? fast_rcp(acc) : 1.0f / 128.0f;
      }
  }

  // 4. codes, scales, stores
  const int bits = is_v ? vb : kb;
  const int code_off = is_v ? k_code_bytes(kb) : 0;
  const int scale_off = scale_offset(kb, vb) + (is_v ? 3 * 512 : 0);
  if (bits == 4)
    quantize_store<4>(R, sfin, rec, code_off, scale_off, is_v, half, gr, nl);
  else if (bits == 2)
    quantize_store<2>(R, sfin, rec, code_off, scale_off, is_v, half, gr, nl);
  else
    quantize_store<8>(R, sfin, rec, code_off, scale_off, is_v, half, gr, nl);
}

__global__ __launch_bounds__(256, 1) void quantize_tiles_kernel(const _Float16* __restrict__ k,
                                                                const _Float16* __restrict__ v,
                                                                const int32_t* __restrict__ dst_pages,
                                                                uint8_t* __restrict__ cache, int64_t page_stride,
                                                                int num_kv_heads, int kb, int vb, int iters) {
  __shared__ float2 xch[2][4][64];
  const int tile = blockIdx.x / num_kv_heads;
  const int h = blockIdx.x - tile * num_kv_heads;
  const bool is_v = (threadIdx.x >> 6) >= 2;
  const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * kCh;
  const _Float16* src = (is_v ? v : k) + (static_cast<int64_t>(tile) * kTok * num_kv_heads + h) * kCh;
  uint8_t* rec = cache + static_cast<int64_t>(dst_pages[tile]) * page_stride +
                 static_cast<int64_t>(h) * record_bytes(kb, vb);
  quantize_tile_half(src, row_stride, nullptr, rec, kb, vb, iters, xch);
}

// Token append: one workgroup per (sequence, kv head).  Writes the new token into
// the fp16 tail at len % 128 and, when that fills the tile, quantises the tail
// (token 127 read from the new token itself) into page_table[s][len / 128].
__global__ __launch_bounds__(256, 1) void append_kernel(const _Float16* __restrict__ k_new,
                                                        const _Float16* __restrict__ v_new,
                                                        const int32_t* __restrict__ seq_lens,
                                                        _Float16* __restrict__ tail_k, _Float16* __restrict__ tail_v,
                                                        const int32_t* __restrict__ page_table, int max_pages,
                                                        uint8_t* __restrict__ cache, int64_t page_stride,
                                                        int num_kv_heads, int kb, int vb, int iters) {
  __shared__ float2 xch[2][4][64];
  const int sh = blockIdx.x;
  const int s = sh / num_kv_heads;
  const int h = sh - s * num_kv_heads;
  const int len = seq_lens[s];
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
    uint8_t* rec = cache + static_cast<int64_t>(page) * page_stride + static_cast<int64_t>(h) * record_bytes(kb, vb);
    quantize_tile_half(x, kCh, last, rec, kb, vb, iters, xch);
  }
}

__global__ void seq_len_increment_kernel(int32_t* __restrict__ seq_lens, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) seq_lens[i] += 1;
}

hipError_t launch_quantize_tiles(const _Float16* k, const _Float16* v, const int32_t* dst_pages, uint8_t* cache,
                                 int64_t page_stride, int num_tiles, int num_kv_heads, int kb, int vb, int iters,
                                 hipStream_t stream) {
  if (num_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_tiles_kernel, dim3(num_tiles * num_kv_heads), dim3(256), 0, stream, k, v, dst_pages,
                     cache, page_stride, num_kv_heads, kb, vb, iters);
  return hipGetLastError();
}

hipError_t launch_append(const _Float16* k_new, const _Float16* v_new, int32_t* seq_lens, _Float16* tail_k,
                         _Float16* tail_v, const int32_t* page_table, int max_pages, uint8_t* cache,
                         int64_t page_stride, int num_seqs, int num_kv_heads, int kb, int vb, int iters,
                         hipStream_t stream) {
  if (num_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(num_seqs * num_kv_heads), dim3(256), 0, stream, k_new, v_new, seq_lens,
                     tail_k, tail_v, page_table, max_pages, cache, page_stride, num_kv_heads, kb, vb, iters);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(seq_len_increment_kernel, dim3((num_seqs + 255) / 256), dim3(256), 0, stream, seq_lens, num_seqs);
  return hipGetLastError();
}

}  // namespace kvarn
