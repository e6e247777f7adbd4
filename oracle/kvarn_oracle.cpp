// KVarN CPU oracle -- TEST INFRASTRUCTURE ONLY.
//
// This file is the slow, plain reference that the GPU path is checked against.
// Only tests/, the smoke check in __graft_entry__.py and the cpu_baseline leg of
// bench.py may load it.  It shares no code, header, table or constant with the
// HIP library: it is written from the method's description, step by step, in
// fp64 with scalar loops.
//
// Pages cited (titles abbreviated, section headings in the page's language):
//   [HYPHO] blog.hypho.cn, "KV-cache 量化终于能跑生产了？KVarN 用方差归一化打破 vLLM
//           的吞吐量魔咒", section "它怎么做到的：四步流水线" (the four-step pipeline),
//           section "论文的核心发现：推理场景的误差累积" (error accumulation),
//           section "工程实践：一行配置启用" (kvarn_k4v2_g128, block_size 128),
//           section "需要关注的几个问题" item 3 (only block size 128).
//   [LEHUY] lehuy.net, "KVarN: Backend lượng tử hóa KV-cache gốc của Huawei ...",
//           section "Cơ chế hoạt động: Chuẩn hóa phương sai" (4 stages per token tile).
//   [OPENAIHUB] openai-hub.net/news/593, section "Technical Details" (per-token scale).
//
// Where the pages are silent the oracle takes one plain reading, stated at the
// function that applies it.
//
// Parity status of each exported function is stated above it.  All of them are
// pinned by tests/test_oracle_pins.py against closed forms, textbook routines,
// hand-made golden bytes or brute force.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

namespace {

constexpr int kTok = 128;   // tokens per tile = page size [HYPHO 工程实践; 需要关注 item 3]
constexpr int kCh = 128;    // head_dim; a token's channels split into 128/g quantisation groups of g

// ---------------------------------------------------------------- fp16 / fp32

// IEEE binary16 -> double (exact).
double half_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int exp = (h >> 10) & 0x1f;
  const int man = h & 0x3ff;
  double mag;
  if (exp == 0) {
    mag = std::ldexp(static_cast<double>(man), -24);          // subnormal: man * 2^-24
  } else if (exp == 31) {
    mag = man ? NAN : INFINITY;
  } else {
    mag = std::ldexp(static_cast<double>(1024 + man), exp - 25);  // (1024+man) * 2^(exp-15-10)
  }
  return sign ? -mag : mag;
}

// double -> IEEE binary16, round to nearest, ties to even.  Written out from the
// format definition: find the representable neighbours and pick the nearer.
uint16_t double_to_half(double x) {
  if (std::isnan(x)) return 0x7e00;
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  double a = std::fabs(x);
  if (a == 0.0) return sign;
  // Scale to an integer significand grid: value = m * 2^e with m in [1024, 2048)
  // for normals (e >= -24) and m < 1024 on the subnormal grid 2^-24.
  int e2;
  std::frexp(a, &e2);           // a = f * 2^e2, f in [0.5, 1)
  int q = e2 - 11;              // grid exponent so that a / 2^q in [1024, 2048)
  if (q < -24) q = -24;         // subnormal grid
  double m = std::ldexp(a, -q); // significand on the grid (not yet integer)
  double fl = std::floor(m);
  double rem = m - fl;
  double r;
  if (rem > 0.5) r = fl + 1;
  else if (rem < 0.5) r = fl;
  else r = (std::fmod(fl, 2.0) == 0.0) ? fl : fl + 1;   // tie -> even
  if (r >= 2048) { r /= 2; q += 1; }
  // r * 2^q; encode
  if (q > 15 - 10) return sign | 0x7c00;                  // overflow -> inf
  if (r < 1024) {                                        // subnormal (q == -24)
    return sign | static_cast<uint16_t>(r);
  }
  const int exp_field = q + 10 + 15;
  if (exp_field >= 31) return sign | 0x7c00;
  return sign | static_cast<uint16_t>((exp_field << 10) | (static_cast<int>(r) - 1024));
}

// ------------------------------------------------------------------- format

struct Fmt {
  int kb, vb, iters;
  int group;   // channels per quantisation group: 128, 64 or 32
  int ng() const { return kCh / group; }
};

size_t k_code_bytes(const Fmt& f) { return static_cast<size_t>(kTok) * kCh * f.kb / 8; }
size_t v_code_bytes(const Fmt& f) { return static_cast<size_t>(kTok) * kCh * f.vb / 8; }
size_t scale_offset(const Fmt& f) { return k_code_bytes(f) + v_code_bytes(f); }
// floats of one half's scales: c[128], s'[ng][128], m'[ng][128]
size_t half_scale_floats(const Fmt& f) { return static_cast<size_t>(kCh) * (1 + 2 * f.ng()); }
size_t record_bytes(const Fmt& f) { return scale_offset(f) + 2 * half_scale_floats(f) * sizeof(float); }

// Record layout (this library's format; the pages fix none of it).
//  K codes, token-major.  Token t owns 16*kb bytes at t*16*kb.  Unit u (0..15)
//  of kb bytes at offset u*kb holds the codes of channels u + 16*e, e = 0..7,
//  code e at bit kb*e of the little-endian unit.
//  V codes.  Unit size U = 2*vb bytes (16 codes).  Unit (nb, gr, nl, half) at
//  ((nb*4 + gr)*16 + nl)*2U + half*U holds channel j = 16*nb + nl for the tokens
//  t = 64*half + 16*mb + 4*gr + i (mb, i in 0..3), code of (mb, i) at bit
//  vb*(4*mb + i).
//  Scales, float32, K half then V half; each half is c[128] (per channel), then
//  s'[ng][128] and m'[ng][128] (group-major: group gi of token t at gi*128 + t),
//  ng = 128 / g groups per token.  For g = 128 these are six float32[128] arrays
//  c_K, s'_K, m'_K, c_V, s'_V, m'_V.
void k_code_pos(const Fmt& f, int t, int j, size_t* byte, int* bit) {
  const int u = j % 16, e = j / 16;
  const size_t bitpos = static_cast<size_t>(t) * 16 * f.kb * 8 + static_cast<size_t>(u) * f.kb * 8 + f.kb * e;
  *byte = bitpos / 8;
  *bit = static_cast<int>(bitpos % 8);
}
void v_code_pos(const Fmt& f, int t, int j, size_t* byte, int* bit) {
  const int nb = j / 16, nl = j % 16;
  const int half = t / 64, mb = (t % 64) / 16, gr = (t % 16) / 4, i = t % 4;
  const size_t U = 2 * f.vb;
  const size_t unit = (static_cast<size_t>(nb * 4 + gr) * 16 + nl) * 2 * U + half * U;
  const size_t bitpos = unit * 8 + static_cast<size_t>(f.vb) * (4 * mb + i);
  *byte = k_code_bytes(f) + bitpos / 8;
  *bit = static_cast<int>(bitpos % 8);
}

// --------------------------------------------------------------- the method

// Sylvester Hadamard matrix of order 128: H_1 = [1], H_2n = [[H, H], [H, -H]].
// Rotation along channels [HYPHO 四步流水线 第二步; LEHUY Cơ chế step 2].
const std::vector<double>& hadamard128() {
  static const std::vector<double> H = [] {
    std::vector<double> h(kCh * kCh, 0.0);
    h[0] = 1.0;
    for (int n = 1; n < kCh; n *= 2) {
      for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) {
          const double x = h[i * kCh + j];
          h[i * kCh + (j + n)] = x;
          h[(i + n) * kCh + j] = x;
          h[(i + n) * kCh + (j + n)] = -x;
        }
    }
    return h;
  }();
  return H;
}

// Y = X Hn with Hn = H_128 / sqrt(128): every token row is rotated along channels.
void rotate_rows(const double* x, double* y, int rows) {
  const auto& H = hadamard128();
  const double inv = 1.0 / std::sqrt(static_cast<double>(kCh));
  for (int t = 0; t < rows; ++t)
    for (int j = 0; j < kCh; ++j) {
      double acc = 0.0;
      for (int k = 0; k < kCh; ++k) acc += x[t * kCh + k] * H[k * kCh + j];
      y[t * kCh + j] = acc * inv;
    }
}

// Alternating row/column normalisation in log space, Sinkhorn style
// [HYPHO 四步流水线 第三步; LEHUY Cơ chế step 3].  A = Y*Y elementwise; the
// channel log-scales v and token log-scales u start at 0 and each iteration
// does one channel pass then one token pass:
//   v_j = 1/2 ln( mean_t A_tj exp(-2 u_t) )
//   u_t = 1/2 ln( mean_j A_tj exp(-2 v_j) )
// An empty (all-zero) row or column keeps log-scale 0.
// If col_dev is given, col_dev[it] = max_j |ln colRMS_j(Z)| after iteration it.
void sinkhorn(const double* Y, int iters, double* u, double* v, double* col_dev) {
  std::vector<double> A(kTok * kCh);
  for (int i = 0; i < kTok * kCh; ++i) A[i] = Y[i] * Y[i];
  for (int t = 0; t < kTok; ++t) u[t] = 0.0;
  for (int j = 0; j < kCh; ++j) v[j] = 0.0;
  for (int it = 0; it < iters; ++it) {
    for (int j = 0; j < kCh; ++j) {
      double s = 0.0;
      for (int t = 0; t < kTok; ++t) s += A[t * kCh + j] * std::exp(-2.0 * u[t]);
      v[j] = (s > 0.0) ? 0.5 * std::log(s / kTok) : 0.0;
    }
    for (int t = 0; t < kTok; ++t) {
      double s = 0.0;
      for (int j = 0; j < kCh; ++j) s += A[t * kCh + j] * std::exp(-2.0 * v[j]);
      u[t] = (s > 0.0) ? 0.5 * std::log(s / kCh) : 0.0;
    }
    if (col_dev) {
      double worst = 0.0;
      for (int j = 0; j < kCh; ++j) {
        double s = 0.0;
        for (int t = 0; t < kTok; ++t) s += A[t * kCh + j] * std::exp(-2.0 * u[t] - 2.0 * v[j]);
        if (s > 0.0) worst = std::max(worst, std::fabs(0.5 * std::log(s / kTok)));
      }
      col_dev[it] = worst;
    }
  }
}

// Asymmetric round-to-nearest of one group of n values (n contiguous channels of
// one token) at b bits [HYPHO 四步流水线 第四步; LEHUY Cơ chế step 4]:
// mn = min z, mx = max z, s = (mx - mn) / (2^b - 1), q = clamp(rint((z - mn) / s),
// 0, 2^b - 1); a constant group (s = 0) gets codes 0.  rint = nearest, ties to
// even.  t_out (optional) receives the unrounded (z - mn)/s.
void rtn_group(const double* z, int n, int bits, double* mn_out, double* s_out, uint8_t* q, double* t_out) {
  double mn = z[0], mx = z[0];
  for (int j = 1; j < n; ++j) {
    mn = std::min(mn, z[j]);
    mx = std::max(mx, z[j]);
  }
  const int qmax = (1 << bits) - 1;
  const double s = (mx - mn) / qmax;
  for (int j = 0; j < n; ++j) {
    if (s > 0.0) {
      const double tv = (z[j] - mn) / s;
      double r = std::nearbyint(tv);   // default rounding mode: ties to even
      r = std::min(std::max(r, 0.0), static_cast<double>(qmax));
      q[j] = static_cast<uint8_t>(r);
      if (t_out) t_out[j] = tv;
    } else {
      q[j] = 0;
      if (t_out) t_out[j] = 0.0;
    }
  }
  *mn_out = mn;
  *s_out = s;
}

// Everything the tile quantizer produces for one 128x128 tile half (K or V).
struct TileOut {
  std::vector<uint8_t> q;          // [t][j]
  std::vector<float> c, sp, mp;    // c[j] = e^{v_j}; [gi][t]: s' = e^{u_t} s_{t,gi}, m' = e^{u_t} mn_{t,gi}
  std::vector<double> y, u, v, z, tval, col_dev;
};

// Steps 1-5 on one tile half: upcast, rotate, normalise, quantise (groups of
// `group` contiguous channels of each token), scales.
// x16: fp16 bits, token t at x16 + t*row_stride, 128 channels contiguous.
void quantize_tile_half(const uint16_t* x16, int64_t row_stride, int bits, int iters, int group, TileOut* o,
                        bool debug) {
  const int ng = kCh / group;
  std::vector<double> x(kTok * kCh), y(kTok * kCh), z(kTok * kCh), tval(kTok * kCh);
  for (int t = 0; t < kTok; ++t)
    for (int j = 0; j < kCh; ++j) x[t * kCh + j] = half_to_double(x16[t * row_stride + j]);
  rotate_rows(x.data(), y.data(), kTok);
  std::vector<double> u(kTok), v(kCh), dev(std::max(iters, 1));
  sinkhorn(y.data(), iters, u.data(), v.data(), debug ? dev.data() : nullptr);
  for (int t = 0; t < kTok; ++t)
    for (int j = 0; j < kCh; ++j) z[t * kCh + j] = y[t * kCh + j] * std::exp(-u[t] - v[j]);
  o->q.assign(kTok * kCh, 0);
  o->c.assign(kCh, 0.f);
  o->sp.assign(static_cast<size_t>(ng) * kTok, 0.f);
  o->mp.assign(static_cast<size_t>(ng) * kTok, 0.f);
  for (int t = 0; t < kTok; ++t) {
    const double r = std::exp(u[t]);
    for (int gi = 0; gi < ng; ++gi) {
      const int j0 = gi * group;
      double mn, s;
      rtn_group(&z[t * kCh + j0], group, bits, &mn, &s, &o->q[t * kCh + j0], &tval[t * kCh + j0]);
      o->sp[gi * kTok + t] = static_cast<float>(r * s);
      o->mp[gi * kTok + t] = static_cast<float>(r * mn);
    }
  }
  for (int j = 0; j < kCh; ++j) o->c[j] = static_cast<float>(std::exp(v[j]));
  if (debug) {
    o->y = y;
    o->u = u;
    o->v = v;
    o->z = z;
    o->tval = tval;
    o->col_dev = dev;
  }
}

void put_code(uint8_t* rec, size_t byte, int bit, int bits, uint8_t code) {
  // A code never straddles a byte: bit offsets are multiples of the width.
  const uint8_t mask = static_cast<uint8_t>(((1u << bits) - 1u) << bit);
  rec[byte] = static_cast<uint8_t>((rec[byte] & ~mask) | ((code << bit) & mask));
}
uint8_t get_code(const uint8_t* rec, size_t byte, int bit, int bits) {
  return static_cast<uint8_t>((rec[byte] >> bit) & ((1u << bits) - 1u));
}

// Step 6: write one record (both halves) in the format above.
void pack_record(const Fmt& f, const TileOut& K, const TileOut& V, uint8_t* rec) {
  std::memset(rec, 0, scale_offset(f));
  for (int t = 0; t < kTok; ++t)
    for (int j = 0; j < kCh; ++j) {
      size_t byte;
      int bit;
      k_code_pos(f, t, j, &byte, &bit);
      put_code(rec, byte, bit, f.kb, K.q[t * kCh + j]);
      v_code_pos(f, t, j, &byte, &bit);
      put_code(rec, byte, bit, f.vb, V.q[t * kCh + j]);
    }
  float* sc = reinterpret_cast<float*>(rec + scale_offset(f));
  const int ng = f.ng();
  const TileOut* half[2] = {&K, &V};
  for (int hv = 0; hv < 2; ++hv) {
    float* h = sc + hv * half_scale_floats(f);
    for (int i = 0; i < kCh; ++i) h[i] = half[hv]->c[i];
    for (int i = 0; i < ng * kTok; ++i) {
      h[kCh + i] = half[hv]->sp[i];
      h[kCh + ng * kTok + i] = half[hv]->mp[i];
    }
  }
}

// Read a record back: codes [t][j] and the scale block (2 * half_scale_floats).
void unpack_record(const Fmt& f, const uint8_t* rec, uint8_t* qk, uint8_t* qv, float* scales) {
  for (int t = 0; t < kTok; ++t)
    for (int j = 0; j < kCh; ++j) {
      size_t byte;
      int bit;
      k_code_pos(f, t, j, &byte, &bit);
      qk[t * kCh + j] = get_code(rec, byte, bit, f.kb);
      v_code_pos(f, t, j, &byte, &bit);
      qv[t * kCh + j] = get_code(rec, byte, bit, f.vb);
    }
  std::memcpy(scales, rec + scale_offset(f), 2 * half_scale_floats(f) * sizeof(float));
}

// Reconstruction of one half: yhat_tj = c_j (m'_{t,g(j)} + s'_{t,g(j)} q_tj) in
// the rotated domain (g(j) = j / group), then xhat_t = Hn yhat_t (Hn is its own
// inverse)  [HYPHO 四步流水线 第四步: scales are restored on read].
void dequant_half(const uint8_t* q, const float* c, const float* sp, const float* mp, int group, double* xhat) {
  std::vector<double> yhat(kTok * kCh);
  for (int t = 0; t < kTok; ++t)
    for (int j = 0; j < kCh; ++j) {
      const int gi = j / group;
      yhat[t * kCh + j] = static_cast<double>(c[j]) * (static_cast<double>(mp[gi * kTok + t]) +
                                                      static_cast<double>(sp[gi * kTok + t]) * q[t * kCh + j]);
    }
  rotate_rows(yhat.data(), xhat, kTok);
}

void dequant_record(const Fmt& f, const uint8_t* rec, double* khat, double* vhat) {
  std::vector<uint8_t> qk(kTok * kCh), qv(kTok * kCh);
  const size_t hs = half_scale_floats(f);
  const int ng = f.ng();
  std::vector<float> sc(2 * hs);
  unpack_record(f, rec, qk.data(), qv.data(), sc.data());
  dequant_half(qk.data(), &sc[0], &sc[kCh], &sc[kCh + ng * kTok], f.group, khat);
  dequant_half(qv.data(), &sc[hs], &sc[hs + kCh], &sc[hs + kCh + ng * kTok], f.group, vhat);
}

void parallel_for(int64_t n, int nthreads, const std::function<void(int64_t)>& fn) {
  if (nthreads <= 0) nthreads = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  if (nthreads == 1 || n <= 1) {
    for (int64_t i = 0; i < n; ++i) fn(i);
    return;
  }
  std::atomic<int64_t> next{0};
  std::vector<std::thread> pool;
  for (int w = 0; w < nthreads; ++w)
    pool.emplace_back([&] {
      for (int64_t i = next++; i < n; i = next++) fn(i);
    });
  for (auto& th : pool) th.join();
}

bool fmt_ok(int kb, int vb, int iters, int group) {
  auto ok = [](int b) { return b == 2 || b == 4 || b == 8; };
  return ok(kb) && ok(vb) && iters >= 0 && (group == 32 || group == 64 || group == 128);
}

}  // namespace

extern "C" {

int oracle_threads_used(int requested) {
  return requested > 0 ? requested : static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
}

size_t oracle_record_bytes(int kb, int vb, int group) { return record_bytes(Fmt{kb, vb, 0, group}); }

// fp16 helpers (pinned against numpy's float16 conversion).
void oracle_half_to_double(const uint16_t* h, double* d, int64_t n) {
  for (int64_t i = 0; i < n; ++i) d[i] = half_to_double(h[i]);
}
void oracle_double_to_half(const double* d, uint16_t* h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = double_to_half(d[i]);
}

// y = x Hn for `rows` rows of 128 (pinned: scipy.linalg.hadamard, H H^T = 128 I).
void oracle_rotate(const double* x, double* y, int rows) { rotate_rows(x, y, rows); }

// Log-space Sinkhorn on A = Y*Y (pinned: rank-1 closed form, unit row RMS,
// monotone column deviation).
void oracle_sinkhorn(const double* y, int iters, double* u, double* v, double* col_dev) {
  sinkhorn(y, iters, u, v, col_dev);
}

// RTN of `rows` groups of n values (pinned: brute-force nearest level, error <= s/2).
void oracle_rtn(const double* z, int rows, int n, int bits, double* mn, double* s, uint8_t* q, double* tval) {
  for (int r = 0; r < rows; ++r)
    rtn_group(z + static_cast<int64_t>(r) * n, n, bits, &mn[r], &s[r], q + static_cast<int64_t>(r) * n,
              tval ? tval + static_cast<int64_t>(r) * n : nullptr);
}

// Full tile-half pipeline with every intermediate exposed (fp64 where the method
// computes, fp32 where it stores): y, u, v, z, tval [t][j] = (z - mn)/s before
// rounding, codes q, scales c[128], s'/m' [128/group][128], col_dev[iters].
int oracle_quantize_tile_debug(const uint16_t* x16, int bits, int iters, int group, double* y, double* u,
                               double* v, double* z, double* tval, uint8_t* q, float* c, float* sp, float* mp,
                               double* col_dev) {
  if (!fmt_ok(bits, bits, iters, group)) return 1;
  TileOut o;
  quantize_tile_half(x16, kCh, bits, iters, group, &o, true);
  std::memcpy(y, o.y.data(), sizeof(double) * kTok * kCh);
  std::memcpy(u, o.u.data(), sizeof(double) * kTok);
  std::memcpy(v, o.v.data(), sizeof(double) * kCh);
  std::memcpy(z, o.z.data(), sizeof(double) * kTok * kCh);
  std::memcpy(tval, o.tval.data(), sizeof(double) * kTok * kCh);
  std::memcpy(q, o.q.data(), kTok * kCh);
  std::memcpy(c, o.c.data(), sizeof(float) * kCh);
  std::memcpy(sp, o.sp.data(), sizeof(float) * o.sp.size());
  std::memcpy(mp, o.mp.data(), sizeof(float) * o.mp.size());
  if (col_dev && iters > 0) std::memcpy(col_dev, o.col_dev.data(), sizeof(double) * iters);
  return 0;
}

// Pack / unpack one record from / to codes [t][j] and the scale block (K half
// c, s'[ng], m'[ng], then the V half; 2 * 128 * (1 + 2 ng) floats).
int oracle_pack_record(int kb, int vb, int group, const uint8_t* qk, const uint8_t* qv, const float* scales,
                       uint8_t* rec) {
  if (!fmt_ok(kb, vb, 0, group)) return 1;
  const Fmt f{kb, vb, 0, group};
  const size_t hs = half_scale_floats(f);
  const int ng = f.ng();
  TileOut K, V;
  K.q.assign(qk, qk + kTok * kCh);
  V.q.assign(qv, qv + kTok * kCh);
  TileOut* half[2] = {&K, &V};
  for (int hv = 0; hv < 2; ++hv) {
    const float* h = scales + hv * hs;
    half[hv]->c.assign(h, h + kCh);
    half[hv]->sp.assign(h + kCh, h + kCh + ng * kTok);
    half[hv]->mp.assign(h + kCh + ng * kTok, h + kCh + 2 * ng * kTok);
  }
  pack_record(f, K, V, rec);
  return 0;
}
int oracle_unpack_record(int kb, int vb, int group, const uint8_t* rec, uint8_t* qk, uint8_t* qv, float* scales) {
  if (!fmt_ok(kb, vb, 0, group)) return 1;
  unpack_record(Fmt{kb, vb, 0, group}, rec, qk, qv, scales);
  return 0;
}

// Dequantised K and V of one record, raw (unrotated) domain, fp64 [t][j].
int oracle_dequant_record(int kb, int vb, int group, const uint8_t* rec, double* khat, double* vhat) {
  if (!fmt_ok(kb, vb, 0, group)) return 1;
  dequant_record(Fmt{kb, vb, 0, group}, rec, khat, vhat);
  return 0;
}

// Bulk quantise: k, v fp16 [num_tiles][128][num_kv_heads][128]; tile i of head h
// goes to cache + dst_pages[i]*page_stride + h*record_bytes.
int oracle_quantize_tiles(int kb, int vb, int iters, int group, int num_tiles, int num_kv_heads, const uint16_t* k,
                          const uint16_t* v, const int32_t* dst_pages, uint8_t* cache, int64_t page_stride,
                          int nthreads) {
  if (!fmt_ok(kb, vb, iters, group) || num_tiles < 0 || num_kv_heads <= 0) return 1;
  const Fmt f{kb, vb, iters, group};
  const size_t R = record_bytes(f);
  const int64_t row_stride = static_cast<int64_t>(num_kv_heads) * kCh;
  parallel_for(static_cast<int64_t>(num_tiles) * num_kv_heads, nthreads, [&](int64_t w) {
    const int64_t tile = w / num_kv_heads;
    const int h = static_cast<int>(w % num_kv_heads);
    const int64_t base = tile * kTok * row_stride + static_cast<int64_t>(h) * kCh;
    TileOut K, V;
    quantize_tile_half(k + base, row_stride, kb, iters, group, &K, false);
    quantize_tile_half(v + base, row_stride, vb, iters, group, &V, false);
    pack_record(f, K, V, cache + dst_pages[tile] * page_stride + static_cast<int64_t>(h) * R);
  });
  return 0;
}

// Append one token per sequence (step 7 of the reading): the token goes, raw
// fp16, into tail[s][h][len % 128]; len += 1; when len % 128 == 0 the tail tile
// is quantised into page page_table[s][len/128 - 1].
int oracle_append_token(int kb, int vb, int iters, int group, int num_seqs, int num_kv_heads, const uint16_t* k_new,
                        const uint16_t* v_new, int32_t* seq_lens, uint16_t* tail_k, uint16_t* tail_v,
                        const int32_t* page_table, int max_pages_per_seq, uint8_t* cache, int64_t page_stride,
                        int nthreads) {
  if (!fmt_ok(kb, vb, iters, group) || num_seqs < 0 || num_kv_heads <= 0) return 1;
  const Fmt f{kb, vb, iters, group};
  const size_t R = record_bytes(f);
  parallel_for(num_seqs, nthreads, [&](int64_t s) {
    const int len = seq_lens[s];
    const int slot = len % kTok;
    for (int h = 0; h < num_kv_heads; ++h) {
      const int64_t tbase = (s * num_kv_heads + h) * static_cast<int64_t>(kTok) * kCh;
      const int64_t nbase = (s * num_kv_heads + h) * static_cast<int64_t>(kCh);
      for (int j = 0; j < kCh; ++j) {
        tail_k[tbase + slot * kCh + j] = k_new[nbase + j];
        tail_v[tbase + slot * kCh + j] = v_new[nbase + j];
      }
      if ((len + 1) % kTok == 0) {
        const int page = page_table[s * max_pages_per_seq + len / kTok];
        TileOut K, V;
        quantize_tile_half(tail_k + tbase, kCh, kb, iters, group, &K, false);
        quantize_tile_half(tail_v + tbase, kCh, vb, iters, group, &V, false);
        pack_record(f, K, V, cache + page * page_stride + static_cast<int64_t>(h) * R);
      }
    }
    seq_lens[s] = len + 1;
  });
  return 0;
}

// Decode attention by definition (step 8 of the reading): for sequence s with L
// tokens and query head hq (kv head hq / (Hq/Hkv)), keys/values of the full pages
// are dequantised and inverse-rotated, tail tokens are the raw fp16 rows, then
// out = softmax(sm_scale * q.K^T) V in fp64, rounded to fp16.  L = 0 -> zeros.
// Each decode step reads every cached token [HYPHO 论文的核心发现].
int oracle_decode_attention(int kb, int vb, int group, int num_seqs, int num_q_heads, int num_kv_heads,
                            const uint16_t* q, const uint8_t* cache, int64_t page_stride, const int32_t* page_table,
                            int max_pages_per_seq, const int32_t* seq_lens, const uint16_t* tail_k,
                            const uint16_t* tail_v, double sm_scale, uint16_t* out, double* out_f64,
                            int nthreads) {
  if (!fmt_ok(kb, vb, 0, group) || num_seqs < 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 1;
  const Fmt f{kb, vb, 0, group};
  const size_t R = record_bytes(f);
  const int G = num_q_heads / num_kv_heads;
  parallel_for(static_cast<int64_t>(num_seqs) * num_kv_heads, nthreads, [&](int64_t w) {
    const int64_t s = w / num_kv_heads;
    const int h = static_cast<int>(w % num_kv_heads);
    const int L = seq_lens[s];
    const int full = L / kTok;
    std::vector<double> K(static_cast<size_t>(L) * kCh), V(static_cast<size_t>(L) * kCh);
    for (int p = 0; p < full; ++p) {
      const uint8_t* rec = cache + page_table[s * max_pages_per_seq + p] * page_stride + static_cast<int64_t>(h) * R;
      dequant_record(f, rec, &K[static_cast<size_t>(p) * kTok * kCh], &V[static_cast<size_t>(p) * kTok * kCh]);
    }
    const int64_t tbase = (s * num_kv_heads + h) * static_cast<int64_t>(kTok) * kCh;
    for (int t = full * kTok; t < L; ++t)
      for (int j = 0; j < kCh; ++j) {
        K[static_cast<size_t>(t) * kCh + j] = half_to_double(tail_k[tbase + (t % kTok) * kCh + j]);
        V[static_cast<size_t>(t) * kCh + j] = half_to_double(tail_v[tbase + (t % kTok) * kCh + j]);
      }
    for (int g = 0; g < G; ++g) {
      const int hq = h * G + g;
      const int64_t qo = (s * num_q_heads + hq) * static_cast<int64_t>(kCh);
      std::vector<double> qq(kCh), logit(L), o(kCh, 0.0);
      for (int j = 0; j < kCh; ++j) qq[j] = half_to_double(q[qo + j]);
      double mx = -INFINITY;
      for (int t = 0; t < L; ++t) {
        double d = 0.0;
        for (int j = 0; j < kCh; ++j) d += qq[j] * K[static_cast<size_t>(t) * kCh + j];
        logit[t] = sm_scale * d;
        mx = std::max(mx, logit[t]);
      }
      double den = 0.0;
      for (int t = 0; t < L; ++t) den += std::exp(logit[t] - mx);
      for (int t = 0; t < L; ++t) {
        const double p = std::exp(logit[t] - mx) / den;
        for (int j = 0; j < kCh; ++j) o[j] += p * V[static_cast<size_t>(t) * kCh + j];
      }
      for (int j = 0; j < kCh; ++j) {
        if (out) out[qo + j] = double_to_half(o[j]);
        if (out_f64) out_f64[qo + j] = o[j];
      }
    }
  });
  return 0;
}

// Chunked prefill attention by definition: sequence s holds L = seq_lens[s] tokens (full pages
// dequantised, tail raw, as for decode) of which the last n = q_lens[s] are this chunk's queries.
// Query i (i < n) sits at position L - n + i and attends causally to positions 0 .. L - n + i.
// q, out: [num_seqs][max_q][num_q_heads][128]; rows i >= n of out are left untouched.
int oracle_prefill_attention(int kb, int vb, int group, int num_seqs, int max_q, int num_q_heads, int num_kv_heads,
                             const uint16_t* q, const int32_t* q_lens, const uint8_t* cache, int64_t page_stride,
                             const int32_t* page_table, int max_pages_per_seq, const int32_t* seq_lens,
                             const uint16_t* tail_k, const uint16_t* tail_v, double sm_scale, uint16_t* out,
                             double* out_f64, int nthreads) {
  if (!fmt_ok(kb, vb, 0, group) || num_seqs < 0 || max_q < 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0)
    return 1;
  for (int s = 0; s < num_seqs; ++s)
    if (q_lens[s] < 0 || q_lens[s] > max_q || q_lens[s] > seq_lens[s]) return 1;
  const Fmt f{kb, vb, 0, group};
  const size_t R = record_bytes(f);
  const int G = num_q_heads / num_kv_heads;
  parallel_for(static_cast<int64_t>(num_seqs) * num_kv_heads, nthreads, [&](int64_t w) {
    const int64_t s = w / num_kv_heads;
    const int h = static_cast<int>(w % num_kv_heads);
    const int L = seq_lens[s];
    const int n = q_lens[s];
    const int full = L / kTok;
    std::vector<double> K(static_cast<size_t>(L) * kCh), V(static_cast<size_t>(L) * kCh);
    for (int p = 0; p < full; ++p) {
      const uint8_t* rec = cache + page_table[s * max_pages_per_seq + p] * page_stride + static_cast<int64_t>(h) * R;
      dequant_record(f, rec, &K[static_cast<size_t>(p) * kTok * kCh], &V[static_cast<size_t>(p) * kTok * kCh]);
    }
    const int64_t tbase = (s * num_kv_heads + h) * static_cast<int64_t>(kTok) * kCh;
    for (int t = full * kTok; t < L; ++t)
      for (int j = 0; j < kCh; ++j) {
        K[static_cast<size_t>(t) * kCh + j] = half_to_double(tail_k[tbase + (t % kTok) * kCh + j]);
        V[static_cast<size_t>(t) * kCh + j] = half_to_double(tail_v[tbase + (t % kTok) * kCh + j]);
      }
    for (int i = 0; i < n; ++i) {
      const int last = L - n + i;   // causal: keys 0 .. last
      for (int g = 0; g < G; ++g) {
        const int hq = h * G + g;
        const int64_t qo = ((s * max_q + i) * static_cast<int64_t>(num_q_heads) + hq) * kCh;
        std::vector<double> qq(kCh), logit(last + 1), o(kCh, 0.0);
        for (int j = 0; j < kCh; ++j) qq[j] = half_to_double(q[qo + j]);
        double mx = -INFINITY;
        for (int t = 0; t <= last; ++t) {
          double d = 0.0;
          for (int j = 0; j < kCh; ++j) d += qq[j] * K[static_cast<size_t>(t) * kCh + j];
          logit[t] = sm_scale * d;
          mx = std::max(mx, logit[t]);
        }
        double den = 0.0;
        for (int t = 0; t <= last; ++t) den += std::exp(logit[t] - mx);
        for (int t = 0; t <= last; ++t) {
          const double p = std::exp(logit[t] - mx) / den;
          for (int j = 0; j < kCh; ++j) o[j] += p * V[static_cast<size_t>(t) * kCh + j];
        }
        for (int j = 0; j < kCh; ++j) {
          if (out) out[qo + j] = double_to_half(o[j]);
          if (out_f64) out_f64[qo + j] = o[j];
        }
      }
    }
  });
  return 0;
}

}  // extern "C"
