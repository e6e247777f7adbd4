// Packed-code helpers shared by the attention kernels (decode and prefill) for gfx950: code ->
// fp16 conversions, the MFMA operand layouts of the K and V codes of a record, buffer loads of a
// record and the asynchronous copy of its scale block into LDS.
#pragma once

#include "kvarn_device.h"

namespace kvarn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <bool HI>
__device__ __forceinline__ f16x2 fp8b_to_f16(uint32_t w) {
  // bytes (0,1) or (2,3) of w, each a code 0..15, read as OCP e4m3 (value code * 2^-9) times 2^9
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 512.0f, HI);
}
template <int SEL>
__device__ __forceinline__ f16x2 fp4b_to_f16(uint32_t w) {
  // byte SEL of w read as two OCP fp4 (e2m1) values, low nibble first: nibbles 0..3 are exactly
  // 0, 0.5, 1, 1.5, so a 2-bit code alone in its nibble converts to code / 2, times 2
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, SEL);
}
__device__ __forceinline__ f16x2 u8pair_to_f16(uint32_t w) {
  // (w & 0x00ff00ff) are two bytes in 16-bit lanes: 0x6400 | b is the fp16 value 1024 + b
  const uint32_t x = (w & 0x00ff00ffu) | 0x64006400u;
  return __builtin_bit_cast(f16x2, x) - f16x2{static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
}
__device__ __forceinline__ f16x8 cat4(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// ---- K codes: token 16*mb + nl, units 4*gr .. 4*gr+3 -------------------------
template <int KB>
struct KRegs;
template <>
struct KRegs<2> {
  u32x2 w;
};
template <>
struct KRegs<4> {
  u32x4 w;
};
template <>
struct KRegs<8> {
  u32x4 w[2];
};

template <int KB>
__device__ __forceinline__ void load_k(KRegs<KB>& r, const uint8_t* p) {
  if constexpr (KB == 2) {
    r.w = *reinterpret_cast<const u32x2*>(p);
  } else if constexpr (KB == 4) {
    r.w = *reinterpret_cast<const u32x4*>(p);
  } else {
    r.w[0] = *reinterpret_cast<const u32x4*>(p);
    r.w[1] = *reinterpret_cast<const u32x4*>(p + 16);
  }
}

// Slot s of the MFMA operand at k-step kb holds code e = keperm(s) of unit 4*gr + kb,
// i.e. channel 4*gr + kb + 16*keperm(s).
template <int KB>
__host__ __device__ constexpr int keperm(int s) {
  return KB <= 4 ? (s < 4 ? 2 * s : 2 * (s - 4) + 1)              // 0 2 4 6 1 3 5 7
                 : ((s & 4) | ((s & 1) << 1) | ((s >> 1) & 1));   // 0 2 1 3 4 6 5 7
}

template <int KB>
__device__ __forceinline__ f16x8 dequant_k(const KRegs<KB>& r, int kb) {
  if constexpr (KB == 2) {
    // units 2j and 2j+1 share a dword (bytes 0-1 and 2-3); w & 0x33333333 leaves codes e = 0, 2 |
    // 4, 6 of each unit alone in the nibbles of its two bytes, (w >> 2) & 0x33333333 codes 1, 3 | 5, 7
    const uint32_t w = r.w[kb >> 1];
    const uint32_t m0 = w & 0x33333333u, m1 = (w >> 2) & 0x33333333u;
    if (kb & 1) return cat4(fp4b_to_f16<2>(m0), fp4b_to_f16<3>(m0), fp4b_to_f16<2>(m1), fp4b_to_f16<3>(m1));
    return cat4(fp4b_to_f16<0>(m0), fp4b_to_f16<1>(m0), fp4b_to_f16<0>(m1), fp4b_to_f16<1>(m1));
  } else if constexpr (KB == 4) {
    const uint32_t w = r.w[kb];
    const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
    return cat4(fp8b_to_f16<false>(lo), fp8b_to_f16<true>(lo), fp8b_to_f16<false>(hi), fp8b_to_f16<true>(hi));
  } else {
    const uint32_t d0 = r.w[kb >> 1][2 * (kb & 1)], d1 = r.w[kb >> 1][2 * (kb & 1) + 1];
    return cat4(u8pair_to_f16(d0), u8pair_to_f16(d0 >> 8), u8pair_to_f16(d1), u8pair_to_f16(d1 >> 8));
  }
}

// Quantisation groups below 128 channels (ng = 2 or 4 per token): k-step kk instead holds codes
// e = 2 kk, 2 kk + 1 of all four units 4*gr + ui, so that each k-step lies in one group
// (channel u + 16 e is in group e / (8 / ng)).  Slot kg_slot(ui, p) holds unit ui, code e = 2 kk + p.
template <int KB>
__host__ __device__ constexpr int kg_slot(int ui, int p) {
  return KB == 2 ? 2 * ui + p : ui + 4 * p;
}

template <int KB>
__device__ __forceinline__ f16x8 dequant_k_grouped(const KRegs<KB>& r, int kk) {
  if constexpr (KB == 2) {
    // byte kk / 2 of each 16-bit unit into one dword, its nibble kk % 2 low; then the two 2-bit codes
    // of each byte into separate nibbles for the fp4 conversion (unit ui in byte ui)
    const uint32_t b = static_cast<uint32_t>(kk >> 1);
    const uint32_t sel = b | ((2 + b) << 8) | ((4 + b) << 16) | ((6 + b) << 24);
    uint32_t x = __builtin_amdgcn_perm(r.w[1], r.w[0], sel);
    if (kk & 1) x >>= 4;
    const uint32_t y = (x & 0x03030303u) | ((x << 2) & 0x30303030u);
    return cat4(fp4b_to_f16<0>(y), fp4b_to_f16<1>(y), fp4b_to_f16<2>(y), fp4b_to_f16<3>(y));
  } else if constexpr (KB == 4) {
    // byte kk of the four unit dwords (codes 2 kk low nibble, 2 kk + 1 high nibble) into one dword
    const uint32_t k = static_cast<uint32_t>(kk);
    const uint32_t sel = k | ((4 + k) << 8) | 0x0c0c0000u;
    const uint32_t x = __builtin_amdgcn_perm(r.w[1], r.w[0], sel) | (__builtin_amdgcn_perm(r.w[3], r.w[2], sel) << 16);
    const uint32_t lo = x & 0x0f0f0f0fu, hi = (x >> 4) & 0x0f0f0f0fu;
    return cat4(fp8b_to_f16<false>(lo), fp8b_to_f16<true>(lo), fp8b_to_f16<false>(hi), fp8b_to_f16<true>(hi));
  } else {
    // bytes 2 kk, 2 kk + 1 of each unit (dword kk / 2 of the unit, half kk % 2): units 0, 1 into d0,
    // units 2, 3 into d1, as (u even e, u even e+1, u odd e, u odd e+1)
    const uint32_t h = 2u * static_cast<uint32_t>(kk & 1);
    const uint32_t sel = h | ((h + 1) << 8) | ((4 + h) << 16) | ((5 + h) << 24);
    const int dw = kk >> 1;
    const uint32_t d0 = __builtin_amdgcn_perm(r.w[0][2 + dw], r.w[0][dw], sel);
    const uint32_t d1 = __builtin_amdgcn_perm(r.w[1][2 + dw], r.w[1][dw], sel);
    return cat4(u8pair_to_f16(d0), u8pair_to_f16(d1), u8pair_to_f16(d0 >> 8), u8pair_to_f16(d1 >> 8));
  }
}

// ---- V codes: channel 16*nb + nl, tokens with (t >> 2) & 3 == gr ------------------
template <int VB>
struct VRegs;
template <>
struct VRegs<2> {
  u32x2 w;  // half 0, half 1
};
template <>
struct VRegs<4> {
  u32x4 w;  // half 0: w[0], w[1]; half 1: w[2], w[3]
};
template <>
struct VRegs<8> {
  u32x4 w[2];
};

template <int VB>
__device__ __forceinline__ void load_v(VRegs<VB>& r, const uint8_t* p) {
  if constexpr (VB == 2) {
    r.w = *reinterpret_cast<const u32x2*>(p);
  } else if constexpr (VB == 4) {
    r.w = *reinterpret_cast<const u32x4*>(p);
  } else {
    r.w[0] = *reinterpret_cast<const u32x4*>(p);
    r.w[1] = *reinterpret_cast<const u32x4*>(p + 16);
  }
}

// k-step kb covers tokens 32*kb + 16*h + 4*gr + i (h, i < 2, 4); slot vslot<VB>(h, i) of the
// MFMA operand holds token (h, i): for 2 and 4 bits the order the masks produce, slots
// (0 1 2 3 4 5 6 7) = (h,i) (0,0) (0,2) (1,0) (1,2) (0,1) (0,3) (1,1) (1,3); (2i + h) for 8 bits.
template <int VB>
__host__ __device__ constexpr int vslot(int h, int i) {
  return VB <= 4 ? (((i & 1) << 2) | (h << 1) | (i >> 1)) : (2 * i + h);
}

template <int VB, int WS>
__device__ __forceinline__ f16x8 dequant_v_ws(const VRegs<VB>& r, int half) {
  constexpr int ws = WS;
  const int kb = 2 * half + WS;
  if constexpr (VB == 4) {
    // dword 2 half + WS holds token (h, i) at bit 16 h + 4 i
    const uint32_t d = r.w[2 * half + WS];
    const uint32_t lo = d & 0x0f0f0f0fu, hi = (d >> 4) & 0x0f0f0f0fu;
    return cat4(fp8b_to_f16<false>(lo), fp8b_to_f16<true>(lo), fp8b_to_f16<false>(hi), fp8b_to_f16<true>(hi));
  } else if constexpr (VB == 2) {
    // byte mb of d holds tokens (mb, i = 0..3) at bits 2i: d & 0x33333333 leaves i = 0, 2 alone in
    // the nibbles, (d >> 2) & 0x33333333 i = 1, 3; bytes 2 WS, 2 WS + 1 are h = 0, 1
    const uint32_t d = r.w[half];
    const uint32_t m0 = d & 0x33333333u, m1 = (d >> 2) & 0x33333333u;
    return cat4(fp4b_to_f16<2 * WS>(m0), fp4b_to_f16<2 * WS + 1>(m0), fp4b_to_f16<2 * WS>(m1),
                fp4b_to_f16<2 * WS + 1>(m1));
  } else {
    const uint32_t D0 = r.w[kb >> 1][2 * ws], D1 = r.w[kb >> 1][2 * ws + 1];
    f16x2 o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // bytes D0.q and D1.q into 16-bit lanes 0 and 1
      const uint32_t sel = static_cast<uint32_t>(q) | 0x0c00u | (static_cast<uint32_t>(4 + q) << 16) | 0x0c000000u;
      o[q] = u8pair_to_f16(__builtin_amdgcn_perm(D1, D0, sel));
    }
    return cat4(o[0], o[1], o[2], o[3]);
  }
}
template <int VB>
__device__ __forceinline__ f16x8 dequant_v(const VRegs<VB>& r, int kb) {
  return (kb & 1) ? dequant_v_ws<VB, 1>(r, kb >> 1) : dequant_v_ws<VB, 0>(r, kb >> 1);
}

// K codes of token blocks mb = 4 h .. 4 h + 3 (h = 0, 1) of the P pages of a group
template <int KB, int P>
struct KHalf {
  KRegs<KB> k[P][4];
};
template <int VB, int P>
struct VAll {
  VRegs<VB> v[P][8];
};

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt not waited for), gfx9 encoding: vmcnt bits 3:0 and 15:14.
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Loads of one group go through buffer descriptors (one per page, base = the record): the lane's
// offset is one VGPR per operand kind and the block offset an SGPR, so no per-lane 64-bit address
// is computed or kept live across the group loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t record_rsrc(const uint8_t* rec, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(rec), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 bload64(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// K codes of token blocks 4h .. 4h+3: token 16 mb + nl, units 4 gr .. 4 gr + 3
template <int KB, int P>
__device__ __forceinline__ void load_k_half(KHalf<KB, P>& d, const __amdgpu_buffer_rsrc_t (&rs)[P], int h, int lane) {
  const uint32_t lo = static_cast<uint32_t>((lane & 15) * 16 * KB + 4 * (lane >> 4) * KB);
#pragma unroll
  for (int e = 0; e < P; ++e)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int off = 16 * (4 * h + m) * 16 * KB;
      if constexpr (KB == 2) {
        d.k[e][m].w = bload64(rs[e], lo, off);
      } else if constexpr (KB == 4) {
        d.k[e][m].w = bload128(rs[e], lo, off);
      } else {
        d.k[e][m].w[0] = bload128(rs[e], lo, off);
        d.k[e][m].w[1] = bload128(rs[e], lo, off + 16);
      }
    }
}

// V codes: unit (nb, gr, nl) of 4 VB bytes at k_code_bytes + (64 nb + lane) 4 VB
template <int KB, int VB, int P>
__device__ __forceinline__ void load_v_all(VAll<VB, P>& d, const __amdgpu_buffer_rsrc_t (&rs)[P], int lane) {
  const uint32_t lo = static_cast<uint32_t>(lane * 4 * VB);
#pragma unroll
  for (int e = 0; e < P; ++e)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const int off = k_code_bytes(KB) + nb * 64 * 4 * VB;
      if constexpr (VB == 2) {
        d.v[e][nb].w = bload64(rs[e], lo, off);
      } else if constexpr (VB == 4) {
        d.v[e][nb].w = bload128(rs[e], lo, off);
      } else {
        d.v[e][nb].w[0] = bload128(rs[e], lo, off);
        d.v[e][nb].w[1] = bload128(rs[e], lo, off + 16);
      }
    }
}

// The P pages' scale blocks (2 (1 + 2 NG) KB each, verbatim) into this wave's LDS stage, 1 KB per
// global_load_lds_dwordx4 (asynchronous, no registers; waited for with vmcnt before the first read).
template <int KB, int VB, int NG, int P>
__device__ __forceinline__ void copy_scales(float* stage, const uint8_t* const (&rec)[P], int lane) {
  constexpr int SC = 2 * half_scale_floats(NG);
  const uint32_t lo = static_cast<uint32_t>(lane * 16);
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const uint8_t* sbase = rec[e] + scale_offset(KB, VB);
#pragma unroll
    for (int c = 0; c < SC / 256; ++c)
      __builtin_amdgcn_global_load_lds(sbase + (lo + static_cast<uint32_t>(c * 1024)), stage + e * SC + c * 256, 16,
                                       0, 0);
  }
}

__device__ __forceinline__ f16x8 zero8() {
  return f16x8{0, 0, 0, 0, 0, 0, 0, 0};
}

// Per-row constant of a PV product with fp16 weights aw (A operand, rows = query columns):
// -c0 sum_k aw[row][k] + m, with m this lane's share of the row's zero-point sum.  c0n is a B
// operand of -c0 everywhere: against the weights it sums exactly the fp16 weights the PV MFMAs use;
// against one extra k-step holding -m / c0 as fp16 hi + lo (hi exact, lo its remainder) in slots 0
// and 1 it adds m.  Every channel of the row gets the same value.
template <int VB>
__device__ __forceinline__ f32x4 pv_zero_point(const f16x8 (&aw)[4], float m, f16x8 c0n) {
  constexpr float c0 = 0.5f * ((1 << VB) - 1);
  const float x = m * (-1.0f / c0);
  f16x8 afake = zero8();
  const float xh = f16_trunc(x);
  afake[0] = static_cast<_Float16>(xh);
  afake[1] = static_cast<_Float16>(x - xh);
  f32x4 c = mfma16(afake, c0n, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) c = mfma16(aw[kb], c0n, c);
  return c;
}

}  // namespace
}  // namespace kvarn
