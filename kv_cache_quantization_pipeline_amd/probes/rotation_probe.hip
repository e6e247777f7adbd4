// Rotation-only timing: the quantiser's Hadamard rotation on the matrix cores (16x16x32 fp16 MFMA
// against +-1 register patterns) beside a fast Walsh-Hadamard transform on the VALU (7 butterfly
// stages, two of them across lanes), over the bulk-quantise workload's tiles: 1024 tiles of 128
// tokens x 4 kv heads x 128 channels, K and V, one workgroup of 2 waves per (tile, head, K|V) as in
// the quantiser.  The rotation is step 2 of blog.hypho.cn, "KV-cache 量化终于能跑生产了？KVarN 用方差
// 归一化打破 vLLM 的吞吐量魔咒", section "它怎么做到的：四步流水线".
//
// It prints a Parseval cross-check (sum of y^2 over a wave's 64 tokens equals 128 times sum of x^2 for
// both forms, since H H^T = 128 I) and the median time of one launch at 1 and 8 rotation passes per
// wave; the difference between the two isolates the rotation from the tile loads.
//
// Build: hipcc -O3 -std=c++17 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops
//        -o _build/rotation_probe kv_cache_quantization_pipeline_amd/probes/rotation_probe.hip
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#define CK(x)                                                                                  \
  do {                                                                                         \
    hipError_t e_ = (x);                                                                       \
    if (e_ != hipSuccess) {                                                                    \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__);   \
      exit(1);                                                                                 \
    }                                                                                          \
  } while (0)

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTok = 128, kCh = 128;

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float as_f(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t as_u(float x) { return __builtin_bit_cast(uint32_t, x); }

// MFMA A operands of a wave's 64 tokens: token 16 mb + nl, channels 32 k4 + 8 gr + s
__device__ __forceinline__ void load_x(f16x8 (&xa)[4][4], const _Float16* __restrict__ x, int64_t row_stride,
                                       int half, int gr, int nl) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int t = 64 * half + 16 * mb + nl;
    const _Float16* row = x + t * row_stride;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) xa[mb][k4] = *reinterpret_cast<const f16x8*>(row + 32 * k4 + 8 * gr);
  }
}

// (a) the quantiser's rotation: Ytilde = X H_128 on the matrix cores, +-1 B patterns
__device__ __forceinline__ float rotate_mfma(const f16x8 (&xa)[4][4], int gr, int nl) {
  f16x8 P0, N0, P1, N1;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int par = __builtin_popcount(s & (nl & 7)) + (gr & 1) * (nl >> 3);
    P0[s] = (par & 1) ? static_cast<_Float16>(-1.0f) : static_cast<_Float16>(1.0f);
  }
  N0 = -P0;
  P1 = (gr >> 1) ? N0 : P0;
  N1 = -P1;
  float ss = 0.f;
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
#pragma unroll
      for (int i = 0; i < 4; ++i) ss = fmaf(c[i], c[i], ss);
    }
  return ss;
}

// (b) FWHT on the VALU, in the load layout: lane (gr, nl) holds channels 32 k4 + 8 gr + s of token
// 16 mb + nl.  Channel bits 0-2 (s) and 5-6 (k4) are butterflies in registers, bits 3-4 (gr) across
// lanes l ^ 16 and l ^ 32 (permlane swaps).  Unnormalised: y = H x.
__device__ __forceinline__ void swap16(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(as_u(a), as_u(b), false, false);
  a = as_f(r[0]);
  b = as_f(r[1]);
}
__device__ __forceinline__ void swap32(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(as_u(a), as_u(b), false, false);
  a = as_f(r[0]);
  b = as_f(r[1]);
}

__device__ __forceinline__ float rotate_fwht(const f16x8 (&xa)[4][4], int gr) {
  float ss = 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    float v[4][8];  // [k4][s]
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
      for (int s = 0; s < 8; ++s) v[k4][s] = static_cast<float>(xa[mb][k4][s]);
    // bits 0-2 (s)
#pragma unroll
    for (int b = 1; b < 8; b <<= 1)
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
        for (int s = 0; s < 8; ++s)
          if (!(s & b)) {
            const float a = v[k4][s], c = v[k4][s | b];
            v[k4][s] = a + c;
            v[k4][s | b] = a - c;
          }
    // bits 5-6 (k4)
#pragma unroll
    for (int b = 1; b < 4; b <<= 1)
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
        if (!(k4 & b))
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const float a = v[k4][s], c = v[k4 | b][s];
            v[k4][s] = a + c;
            v[k4 | b][s] = a - c;
          }
    // bits 3 (lane bit 4) and 4 (lane bit 5): pairs of registers exchanged so that each lane ends with
    // the (sum, difference) of its value and the partner lane's value.  With permlane16_swap(a, b):
    // a = [a.r0, b.r0, a.r2, b.r2], b = [a.r1, b.r1, a.r3, b.r3] (rows of 16 lanes).  Lanes of odd rows
    // hold the upper element: after the swap of (x, x) a row-pair sees both values.
    const bool up16 = gr & 1, up32 = gr >> 1;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        float a = v[k4][s], b = v[k4][s];
        swap16(a, b);  // even rows: a = own, b = odd partner's;  odd rows: a = even partner's, b = own
        v[k4][s] = up16 ? a - b : a + b;
      }
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        float a = v[k4][s], b = v[k4][s];
        swap32(a, b);
        v[k4][s] = up32 ? a - b : a + b;
      }
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
      for (int s = 0; s < 8; ++s) ss = fmaf(v[k4][s], v[k4][s], ss);
  }
  return ss;
}

// one workgroup of 2 waves per (tile, kv head, half), as the quantiser; each wave rotates its 64
// tokens `reps` times (the input nudged by a runtime zero each time, so the repeats are not merged)
template <bool FWHT>
__global__ __launch_bounds__(128, 2) void rot_kernel(const _Float16* __restrict__ k, const _Float16* __restrict__ v,
                                                     int num_kv_heads, int reps, float zero, float* __restrict__ out) {
  const int th = blockIdx.x >> 1;
  const bool is_v = blockIdx.x & 1;
  const int tile = th / num_kv_heads, h = th - tile * num_kv_heads;
  const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * kCh;
  const _Float16* src = (is_v ? v : k) + (static_cast<int64_t>(tile) * kTok * num_kv_heads + h) * kCh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, gr = lane >> 4;
  f16x8 xa[4][4];
  load_x(xa, src, row_stride, wave, gr, nl);
  float ss = 0.f;
  for (int r = 0; r < reps; ++r) {
    if (r > 0) {
      const _Float16 z = static_cast<_Float16>(zero * r);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) xa[mb][k4][0] += z;
    }
    ss += FWHT ? rotate_fwht(xa, gr) : rotate_mfma(xa, gr, nl);
  }
  // sum over the wave
#pragma unroll
  for (int b = 32; b >= 1; b >>= 1) ss += __shfl_xor(ss, b);
  if (lane == 0) out[2 * blockIdx.x + wave] = ss;
}

int main() {
  const int n_tiles = 1024, hkv = 4;
  const size_t n = static_cast<size_t>(n_tiles) * kTok * hkv * kCh;
  std::vector<_Float16> h(n);
  srand(3);
  for (size_t i = 0; i < n; ++i) h[i] = static_cast<_Float16>((rand() / (float)RAND_MAX - 0.5f) * 4.0f);
  _Float16 *k[2], *v[2];
  for (int c = 0; c < 2; ++c) {
    CK(hipMalloc(&k[c], n * 2));
    CK(hipMalloc(&v[c], n * 2));
    CK(hipMemcpy(k[c], h.data(), n * 2, hipMemcpyHostToDevice));
    CK(hipMemcpy(v[c], h.data(), n * 2, hipMemcpyHostToDevice));
  }
  const int nblk = 2 * n_tiles * hkv;
  float *oa, *ob;
  CK(hipMalloc(&oa, 2 * nblk * 4));
  CK(hipMalloc(&ob, 2 * nblk * 4));
  // Parseval check on reps = 1: both kernels give sum y^2 = 128 sum x^2 per wave
  hipLaunchKernelGGL(rot_kernel<false>, dim3(nblk), dim3(128), 0, 0, k[0], v[0], hkv, 1, 0.f, oa);
  hipLaunchKernelGGL(rot_kernel<true>, dim3(nblk), dim3(128), 0, 0, k[0], v[0], hkv, 1, 0.f, ob);
  CK(hipDeviceSynchronize());
  std::vector<float> ha(2 * nblk), hb(2 * nblk);
  CK(hipMemcpy(ha.data(), oa, 2 * nblk * 4, hipMemcpyDeviceToHost));
  CK(hipMemcpy(hb.data(), ob, 2 * nblk * 4, hipMemcpyDeviceToHost));
  double worst = 0, worst_x = 0;
  for (int w = 0; w < 2 * nblk; ++w) {
    worst = std::max(worst, (double)(std::abs(ha[w] - hb[w]) / std::abs(ha[w])));
    // host sum x^2 of that wave's 64 tokens
    const int blk = w / 2, wave = w % 2, th = blk >> 1, isv = blk & 1, tile = th / hkv, hh = th % hkv;
    (void)isv;
    double sx = 0;
    for (int t = 64 * wave; t < 64 * wave + 64; ++t)
      for (int j = 0; j < kCh; ++j) {
        const double x = static_cast<float>(h[((static_cast<size_t>(tile) * kTok + t) * hkv + hh) * kCh + j]);
        sx += x * x;
      }
    worst_x = std::max(worst_x, std::abs(ha[w] - 128.0 * sx) / (128.0 * sx));
  }
  printf("Parseval: max rel diff MFMA vs FWHT %.3g, MFMA vs 128 sum x^2 %.3g\n", worst, worst_x);

  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  for (int reps : {1, 8}) {
    for (int f = 0; f < 2; ++f) {
      std::vector<float> ts;
      for (int it = 0; it < 23; ++it) {
        CK(hipEventRecord(e0, 0));
        if (f)
          hipLaunchKernelGGL(rot_kernel<true>, dim3(nblk), dim3(128), 0, 0, k[it & 1], v[it & 1], hkv, reps, 0.f, ob);
        else
          hipLaunchKernelGGL(rot_kernel<false>, dim3(nblk), dim3(128), 0, 0, k[it & 1], v[it & 1], hkv, reps, 0.f, oa);
        CK(hipEventRecord(e1, 0));
        CK(hipEventSynchronize(e1));
        float ms;
        CK(hipEventElapsedTime(&ms, e0, e1));
        if (it >= 3) ts.push_back(ms * 1000.f);
      }
      std::sort(ts.begin(), ts.end());
      printf("rotation %-5s reps %d: median %.1f us (%d tile-halves, %.1f us per rotation pass)\n", f ? "FWHT" : "MFMA",
             reps, ts[ts.size() / 2], nblk, ts[ts.size() / 2] / reps);
    }
  }
  return 0;
}
