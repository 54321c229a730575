// CPU oracle for KVarN block quantisation and decode attention over the packed cache: plain C++17,
// double precision, threads over independent tiles and (sequence, KV head) pairs.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the CPU-baseline leg of the
// benchmark load this library; the product library never links it, and it shares no code, header,
// table or constant generator with the HIP kernels.  It implements the page byte format on its own.
//
// What it computes (the KVarN blog post, "KVarN: Huawei'den KV-Cache Kuantizasyonu için Yerel vLLM
// Backend'i", section "KVarN Nasıl Çalışır?"): every fixed-size block of 128 tokens of K or V goes
// through a Hadamard rotation along channels, a log-space row/column variance normalisation, low-bit
// asymmetric round-to-nearest and packing; section "Pratik Çıkarımlar" names kvarn_k4v2_g128.  Decode
// attention reads the packed pages through a block table with grouped query heads (the "KV Cache"
// glossary page, sections "Boyutu ve Yönetimi" and "Türleri").
//
// The readings it takes where the pages are silent are the same, one by one, as the Python oracle's:
//   * block 128 tokens; head_dim D in {64, 128, 256}; T = 4 iterations; eps = 1e-6 added to the
//     variance; log base 2; both normalisers start at 0; each iteration is a row pass (per token, over
//     the D channels) then a column pass (per channel, over the 128 tokens); variance = centred
//     population variance;
//   * rotation: the natural-order Sylvester Hadamard matrix H[j][k] = (-1)^popcount(j & k) / sqrt(D),
//     no random signs, on K and V alike;
//   * the values that get quantised are N = R * 2^-(rho + gamma) with the stored fp32 rho and gamma,
//     rounded to fp32; the rounding decision is taken in fp32: scale = fp16(fp32(fp32(max - min) /
//     L)), zero = fp16(min), code = clamp(round-half-even(fp32(fp32(N - zero) / scale)), 0, L), and a
//     group whose fp16 scale is 0 stores zero codes;
//   * key groups: one channel over `group` consecutive tokens (entry D*h + j for channel j, token
//     half h); value groups: one token over min(group, D) consecutive channels (entry 128*h + t);
//   * page = codes | scale fp16[n] | zero fp16[n] | rho fp32[128] | gamma fp32[D], little endian.
//     Key codes token-major (4 bits: byte (D/2)*t + k holds channels 2k | 2k+1 << 4; 8 bits: byte
//     D*t + c); value codes channel-major (2 bits: byte 32*c + k holds token 4k+i at bits 2i; 4 bits:
//     byte 64*c + k holds tokens 2k | 2k+1 << 4);
//   * decode: query head h reads KV head h / (Hq / Hkv); logits scaled by 1/sqrt(D) unless a positive
//     scale is given; softmax with the maximum subtracted; output in the original basis; an optional
//     fp16 tail of seq_len % 128 rows follows the packed blocks.
//
// Two rotation modes: the dense matrix product (the definition) and the fast Walsh-Hadamard
// transform, whose butterflies add fp16 inputs exactly in double and round once when scaled; the two
// agree to about 1e-15 relative.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

constexpr int kBlock = 128;
constexpr int kIters = 4;
constexpr double kEps = 1e-6;

// ---------------------------------------------------------------------------------------------
// IEEE 754 binary16, from its definition: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits;
// exponent 0 holds the subnormals m * 2^-24, exponent 31 infinities and NaNs.
// ---------------------------------------------------------------------------------------------
double half_to_double(uint16_t h) {
  const int e = (h >> 10) & 31;
  const int m = h & 1023;
  double v;
  if (e == 0)
    v = std::ldexp(static_cast<double>(m), -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = std::ldexp(static_cast<double>(m + 1024), e - 25);
  return (h & 0x8000) ? -v : v;
}

// Nearest binary16 to x, ties to even (x is exact in double; used on fp32 values).
uint16_t double_to_half(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  const double a = std::fabs(x);
  if (std::isnan(a)) return sign | 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;  // half-way past the largest finite value, 65504, rounds up
  int e = 0;
  std::frexp(a, &e);  // a in [2^(e-1), 2^e)
  // spacing of binary16 numbers around a: 2^-24 below 2^-14 (subnormals), else 2^(e-11)
  const double quantum = a < std::ldexp(1.0, -14) ? std::ldexp(1.0, -24) : std::ldexp(1.0, e - 11);
  const double r = std::nearbyint(a / quantum) * quantum;  // a / quantum is exact: quantum is 2^k
  if (r == 0.0) return sign;
  if (r < std::ldexp(1.0, -14)) return sign | static_cast<uint16_t>(r / std::ldexp(1.0, -24));
  const int ex = std::ilogb(r);  // r in [2^ex, 2^(ex+1))
  const int frac = static_cast<int>(r / std::ldexp(1.0, ex - 10)) - 1024;
  return sign | static_cast<uint16_t>(((ex + 15) << 10) | frac);
}

// ---------------------------------------------------------------------------------------------
// Format of one page
// ---------------------------------------------------------------------------------------------
struct Fmt {
  int D, bits, group, is_v;
  int levels() const { return (1 << bits) - 1; }
  int code_bytes() const { return kBlock * D * bits / 8; }
  int vgroup() const { return std::min(group, D); }  // channels per value group
  int ngroups() const { return is_v ? (D / vgroup()) * kBlock : (kBlock / group) * D; }
  int scale_off() const { return code_bytes(); }
  int zero_off() const { return code_bytes() + 2 * ngroups(); }
  int rho_off() const { return code_bytes() + 4 * ngroups(); }
  int gam_off() const { return rho_off() + 4 * kBlock; }
  int page_bytes() const { return gam_off() + 4 * D; }
};

bool fmt_ok(int D, int bits, int group, int is_v) {
  if (D != 64 && D != 128 && D != 256) return false;
  if (group != 64 && group != 128) return false;
  return is_v ? (bits == 2 || bits == 4) : (bits == 4 || bits == 8);
}

void put_u16(uint8_t* p, uint16_t v) {
  p[0] = static_cast<uint8_t>(v & 0xFF);
  p[1] = static_cast<uint8_t>(v >> 8);
}
uint16_t get_u16(const uint8_t* p) { return static_cast<uint16_t>(p[0] | (p[1] << 8)); }
void put_f32(uint8_t* p, float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  for (int i = 0; i < 4; ++i) p[i] = static_cast<uint8_t>(u >> (8 * i));
}
float get_f32(const uint8_t* p) {
  uint32_t u = 0;
  for (int i = 0; i < 4; ++i) u |= static_cast<uint32_t>(p[i]) << (8 * i);
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// ---------------------------------------------------------------------------------------------
// Stage 2, rotation: out[t][j] = sum_k H[j][k] x[t][k] for every row t
// ---------------------------------------------------------------------------------------------
int popcount(unsigned v) {
  int c = 0;
  for (; v; v &= v - 1) ++c;
  return c;
}

void rotate_rows(const double* x, double* out, int rows, int D, bool fwht) {
  const double inv = 1.0 / std::sqrt(static_cast<double>(D));
  std::vector<double> a(D);
  for (int t = 0; t < rows; ++t) {
    const double* xr = x + static_cast<size_t>(t) * D;
    double* o = out + static_cast<size_t>(t) * D;
    if (fwht) {
      // butterflies over index bit b: pairs (i, i + 2^b) become (sum, difference)
      for (int k = 0; k < D; ++k) a[k] = xr[k];
      for (int len = 1; len < D; len <<= 1)
        for (int i = 0; i < D; i += 2 * len)
          for (int k = i; k < i + len; ++k) {
            const double u = a[k], w = a[k + len];
            a[k] = u + w;
            a[k + len] = u - w;
          }
      for (int j = 0; j < D; ++j) o[j] = a[j] * inv;
    } else {
      for (int j = 0; j < D; ++j) {
        double s = 0.0;
        for (int k = 0; k < D; ++k) s += ((popcount(static_cast<unsigned>(j & k)) & 1) ? -inv : inv) * xr[k];
        o[j] = s;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Stage 3, normalisation: rho per row, gamma per column, log2 units
// ---------------------------------------------------------------------------------------------
void normalize(const double* r, int rows, int cols, int iters, double eps, double* rho, double* gam) {
  for (int t = 0; t < rows; ++t) rho[t] = 0.0;
  for (int j = 0; j < cols; ++j) gam[j] = 0.0;
  std::vector<double> y(std::max(rows, cols));
  for (int it = 0; it < iters; ++it) {
    for (int t = 0; t < rows; ++t) {  // row pass: the variance of each row of the normalised block
      double mean = 0.0;
      for (int j = 0; j < cols; ++j) {
        y[j] = r[static_cast<size_t>(t) * cols + j] * std::exp2(-(rho[t] + gam[j]));
        mean += y[j];
      }
      mean /= cols;
      double var = 0.0;
      for (int j = 0; j < cols; ++j) var += (y[j] - mean) * (y[j] - mean);
      var /= cols;
      rho[t] += 0.5 * std::log2(var + eps);
    }
    for (int j = 0; j < cols; ++j) {  // column pass, with the rows' new normalisers
      double mean = 0.0;
      for (int t = 0; t < rows; ++t) {
        y[t] = r[static_cast<size_t>(t) * cols + j] * std::exp2(-(rho[t] + gam[j]));
        mean += y[t];
      }
      mean /= rows;
      double var = 0.0;
      for (int t = 0; t < rows; ++t) var += (y[t] - mean) * (y[t] - mean);
      var /= rows;
      gam[j] += 0.5 * std::log2(var + eps);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Stage 4, round to nearest: one group of fp32 values -> codes, fp16 scale and zero
// ---------------------------------------------------------------------------------------------
void rtn_group(const float* const* v, int n, int levels, uint8_t* const* codes, uint16_t* sbits, uint16_t* zbits) {
  float mn = *v[0], mx = *v[0];
  for (int i = 1; i < n; ++i) {
    mn = std::min(mn, *v[i]);
    mx = std::max(mx, *v[i]);
  }
  const float range = mx - mn;
  const float s32 = range / static_cast<float>(levels);
  *sbits = double_to_half(s32);
  *zbits = double_to_half(mn);
  const float s = static_cast<float>(half_to_double(*sbits));
  const float z = static_cast<float>(half_to_double(*zbits));
  for (int i = 0; i < n; ++i) {
    if (s == 0.0f) {
      *codes[i] = 0;
      continue;
    }
    const float d = *v[i] - z;
    const float u = d / s;
    const float c = std::nearbyint(u);  // round half to even (default rounding mode)
    *codes[i] = static_cast<uint8_t>(std::min(std::max(c, 0.0f), static_cast<float>(levels)));
  }
}

// One 128-token tile: x16 rows are token t at x16 + t * row_stride (D fp16 values each).
void quantize_tile(const uint16_t* x16, size_t row_stride, const Fmt& f, bool fwht, uint8_t* page) {
  const int D = f.D;
  std::vector<double> x(static_cast<size_t>(kBlock) * D), r(static_cast<size_t>(kBlock) * D);
  for (int t = 0; t < kBlock; ++t)
    for (int k = 0; k < D; ++k) x[static_cast<size_t>(t) * D + k] = half_to_double(x16[t * row_stride + k]);
  rotate_rows(x.data(), r.data(), kBlock, D, fwht);
  std::vector<double> rho(kBlock), gam(D);
  normalize(r.data(), kBlock, D, kIters, kEps, rho.data(), gam.data());
  std::vector<float> rho32(kBlock), gam32(D);
  for (int t = 0; t < kBlock; ++t) rho32[t] = static_cast<float>(rho[t]);
  for (int j = 0; j < D; ++j) gam32[j] = static_cast<float>(gam[j]);
  // the values to quantise, from the stored fp32 normalisers
  std::vector<float> n32(static_cast<size_t>(kBlock) * D);
  for (int t = 0; t < kBlock; ++t)
    for (int j = 0; j < D; ++j)
      n32[static_cast<size_t>(t) * D + j] = static_cast<float>(
          r[static_cast<size_t>(t) * D + j] * std::exp2(-(static_cast<double>(rho32[t]) + static_cast<double>(gam32[j]))));
  std::vector<uint8_t> codes(static_cast<size_t>(kBlock) * D);
  std::vector<uint16_t> sb(f.ngroups()), zb(f.ngroups());
  std::vector<const float*> gv(kBlock);
  std::vector<uint8_t*> gc(kBlock);
  if (!f.is_v) {
    for (int h = 0; h < kBlock / f.group; ++h)
      for (int j = 0; j < D; ++j) {
        for (int i = 0; i < f.group; ++i) {
          const size_t e = static_cast<size_t>(f.group * h + i) * D + j;
          gv[i] = &n32[e];
          gc[i] = &codes[e];
        }
        rtn_group(gv.data(), f.group, f.levels(), gc.data(), &sb[D * h + j], &zb[D * h + j]);
      }
  } else {
    const int g = f.vgroup();
    for (int h = 0; h < D / g; ++h)
      for (int t = 0; t < kBlock; ++t) {
        for (int i = 0; i < g; ++i) {
          const size_t e = static_cast<size_t>(t) * D + g * h + i;
          gv[i] = &n32[e];
          gc[i] = &codes[e];
        }
        rtn_group(gv.data(), g, f.levels(), gc.data(), &sb[kBlock * h + t], &zb[kBlock * h + t]);
      }
  }
  // pack
  std::memset(page, 0, f.code_bytes());
  for (int t = 0; t < kBlock; ++t)
    for (int c = 0; c < D; ++c) {
      const uint8_t q = codes[static_cast<size_t>(t) * D + c];
      if (!f.is_v) {
        if (f.bits == 8)
          page[D * t + c] = q;
        else
          page[(D / 2) * t + c / 2] |= static_cast<uint8_t>(q << (4 * (c & 1)));
      } else {
        if (f.bits == 2)
          page[32 * c + t / 4] |= static_cast<uint8_t>(q << (2 * (t & 3)));
        else
          page[64 * c + t / 2] |= static_cast<uint8_t>(q << (4 * (t & 1)));
      }
    }
  for (int i = 0; i < f.ngroups(); ++i) {
    put_u16(page + f.scale_off() + 2 * i, sb[i]);
    put_u16(page + f.zero_off() + 2 * i, zb[i]);
  }
  for (int t = 0; t < kBlock; ++t) put_f32(page + f.rho_off() + 4 * t, rho32[t]);
  for (int j = 0; j < D; ++j) put_f32(page + f.gam_off() + 4 * j, gam32[j]);
}

uint8_t unpack_code(const uint8_t* page, const Fmt& f, int t, int c) {
  if (!f.is_v) {
    if (f.bits == 8) return page[f.D * t + c];
    return (page[(f.D / 2) * t + c / 2] >> (4 * (c & 1))) & 15;
  }
  if (f.bits == 2) return (page[32 * c + t / 4] >> (2 * (t & 3))) & 3;
  return (page[64 * c + t / 2] >> (4 * (t & 1))) & 15;
}

// Dequantise one page to the original basis: N^ = s q + z, R^ = N^ 2^(rho + gamma), X^ = H R^.
void dequantize_page(const uint8_t* page, const Fmt& f, bool fwht, double* out) {
  const int D = f.D;
  std::vector<double> rh(static_cast<size_t>(kBlock) * D);
  for (int t = 0; t < kBlock; ++t) {
    const double rho = get_f32(page + f.rho_off() + 4 * t);
    for (int j = 0; j < D; ++j) {
      const int gi = f.is_v ? kBlock * (j / f.vgroup()) + t : D * (t / f.group) + j;
      const double s = half_to_double(get_u16(page + f.scale_off() + 2 * gi));
      const double z = half_to_double(get_u16(page + f.zero_off() + 2 * gi));
      const double gam = get_f32(page + f.gam_off() + 4 * j);
      rh[static_cast<size_t>(t) * D + j] = (unpack_code(page, f, t, j) * s + z) * std::exp2(rho + gam);
    }
  }
  // H is symmetric and its own inverse
  rotate_rows(rh.data(), out, kBlock, D, fwht);
}

// ---------------------------------------------------------------------------------------------
// Threads: fn(i) for i in [0, n) on up to `threads` workers (0 = every hardware thread)
// ---------------------------------------------------------------------------------------------
template <class Fn>
void parallel_for(long n, int threads, Fn fn) {
  int nt = threads > 0 ? threads : static_cast<int>(std::thread::hardware_concurrency());
  if (nt < 1) nt = 1;
  if (nt > n) nt = static_cast<int>(std::max(1L, n));
  if (nt == 1) {
    for (long i = 0; i < n; ++i) fn(i);
    return;
  }
  std::atomic<long> next(0);
  std::vector<std::thread> pool;
  for (int w = 0; w < nt; ++w)
    pool.emplace_back([&]() {
      for (long i = next.fetch_add(1); i < n; i = next.fetch_add(1)) fn(i);
    });
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

// Bytes of one page of this format; 0 if the format is not one the oracle knows.
long kvo_page_bytes(int head_dim, int bits, int group, int is_v) {
  if (!fmt_ok(head_dim, bits, group, is_v)) return 0;
  return Fmt{head_dim, bits, group, is_v}.page_bytes();
}

// fp16 conversions (exposed for their pins).
double kvo_half_to_double(uint16_t h) { return half_to_double(h); }
uint16_t kvo_double_to_half(double x) { return double_to_half(x); }

// out[rows][D] = rows of x rotated by the orthonormal Hadamard matrix (fwht: 1 butterflies, 0 dense).
int kvo_rotate(const double* x, int rows, int D, int fwht, double* out) {
  if (D < 1 || (D & (D - 1))) return -1;
  rotate_rows(x, out, rows, D, fwht != 0);
  return 0;
}

// Log2 normalisers of an r[rows][cols] block (any shape), as the quantiser computes them.
int kvo_normalize(const double* r, int rows, int cols, int iters, double eps, double* rho, double* gam) {
  if (rows < 1 || cols < 1 || iters < 0) return -1;
  normalize(r, rows, cols, iters, eps, rho, gam);
  return 0;
}

// Quantise n_blocks 128-token blocks of K and V, fp16 [n_blocks*128][hkv][D], into the pools
// ([num_pages][hkv][page bytes]): block b of head h goes to page dst_pages[b].  Entries outside
// [0, num_pages) are skipped and counted in the return value; -1 for an unknown format.
long kvo_quantize_blocks(const uint16_t* k, const uint16_t* v, int n_blocks, int hkv, int head_dim,
                         const int32_t* dst_pages, uint8_t* k_pool, uint8_t* v_pool, int num_pages, int kbits,
                         int vbits, int group, int fwht, int threads) {
  if (!fmt_ok(head_dim, kbits, group, 0) || !fmt_ok(head_dim, vbits, group, 1)) return -1;
  const Fmt fk{head_dim, kbits, group, 0}, fv{head_dim, vbits, group, 1};
  std::atomic<long> bad(0);
  parallel_for(2L * n_blocks * hkv, threads, [&](long i) {
    const bool is_v = i & 1;
    const long bh = i >> 1;
    const int b = static_cast<int>(bh / hkv), h = static_cast<int>(bh % hkv);
    const int p = dst_pages[b];
    if (p < 0 || p >= num_pages) {
      if (!is_v && h == 0) bad.fetch_add(1);  // counted once per block
      return;
    }
    const Fmt& f = is_v ? fv : fk;
    const uint16_t* src = (is_v ? v : k) + (static_cast<size_t>(b) * kBlock * hkv + h) * head_dim;
    uint8_t* dst = (is_v ? v_pool : k_pool) + (static_cast<size_t>(p) * hkv + h) * f.page_bytes();
    quantize_tile(src, static_cast<size_t>(hkv) * head_dim, f, fwht != 0, dst);
  });
  return bad.load();
}

// One page back to the original basis: out[128][D] in double.
int kvo_dequantize_page(const uint8_t* page, int is_v, int head_dim, int bits, int group, int fwht, double* out) {
  if (!fmt_ok(head_dim, bits, group, is_v)) return -1;
  dequantize_page(page, Fmt{head_dim, bits, group, is_v}, fwht != 0, out);
  return 0;
}

// Decode attention: out[b][h][D] (double) for every sequence b and query head h, or only for the
// (b, h) pairs listed in `pairs` ([n_pairs][2]; NULL = all; other rows are left untouched; a pair out
// of range returns -1 before anything is computed).
// Sequence b attends to pages block_table[b][0 .. seq_lens[b]/128) (an id outside [0, num_pages) is
// left out) and, when k_tail / v_tail are given (fp16 [batch][128][hkv][D]), to the seq_lens[b] % 128
// tail rows after them; without tails the remainder is ignored.  A length below 0 or with more full
// blocks than max_blocks gives zeros.  Returns -1 for an unknown format.
int kvo_decode(const uint16_t* q, const uint8_t* k_pool, const uint8_t* v_pool, int num_pages,
               const int32_t* block_table, int max_blocks, const int32_t* seq_lens, const uint16_t* k_tail,
               const uint16_t* v_tail, int batch, int hq, int hkv, int head_dim, int kbits, int vbits, int group,
               double softmax_scale, const int32_t* pairs, int n_pairs, int fwht, int threads, double* out) {
  if (!fmt_ok(head_dim, kbits, group, 0) || !fmt_ok(head_dim, vbits, group, 1) || hkv < 1 || hq % hkv) return -1;
  const int D = head_dim;
  const Fmt fk{D, kbits, group, 0}, fv{D, vbits, group, 1};
  const int G = hq / hkv;
  const double scale = softmax_scale > 0 ? softmax_scale : 1.0 / std::sqrt(static_cast<double>(D));
  // work list: (sequence, KV head) units, each with the query heads it serves
  std::vector<std::vector<int>> heads(static_cast<size_t>(batch) * hkv);
  if (pairs) {
    for (int i = 0; i < n_pairs; ++i) {
      const int pb = pairs[2 * i], ph = pairs[2 * i + 1];
      if (pb < 0 || pb >= batch || ph < 0 || ph >= hq) return -1;
      heads[static_cast<size_t>(pb) * hkv + ph / G].push_back(ph);
    }
  } else {
    for (int b = 0; b < batch; ++b)
      for (int h = 0; h < hq; ++h) heads[static_cast<size_t>(b) * hkv + h / G].push_back(h);
  }
  std::vector<long> units;
  for (size_t u = 0; u < heads.size(); ++u)
    if (!heads[u].empty()) units.push_back(static_cast<long>(u));
  parallel_for(static_cast<long>(units.size()), threads, [&](long ui) {
    const long u = units[ui];
    const int b = static_cast<int>(u / hkv), g = static_cast<int>(u % hkv);
    // a length below 0 or past the block table gives a sequence with no rows (output 0)
    const int raw = seq_lens[b];
    const int len = raw < 0 || raw / kBlock > max_blocks ? 0 : raw;
    const int ntail = (k_tail && v_tail) ? len % kBlock : 0;
    // a page id outside [0, num_pages) names no block: that block is left out
    std::vector<int> pages;
    for (int i = 0; i < len / kBlock; ++i) {
      const int p = block_table[static_cast<size_t>(b) * max_blocks + i];
      if (p >= 0 && p < num_pages) pages.push_back(p);
    }
    const int nblk = static_cast<int>(pages.size());
    const int rows = nblk * kBlock + ntail;
    std::vector<double> kh(static_cast<size_t>(rows) * D), vh(static_cast<size_t>(rows) * D);
    for (int i = 0; i < nblk; ++i) {
      const size_t off = static_cast<size_t>(i) * kBlock * D;
      dequantize_page(k_pool + (static_cast<size_t>(pages[i]) * hkv + g) * fk.page_bytes(), fk, fwht != 0, &kh[off]);
      dequantize_page(v_pool + (static_cast<size_t>(pages[i]) * hkv + g) * fv.page_bytes(), fv, fwht != 0, &vh[off]);
    }
    for (int r = 0; r < ntail; ++r)
      for (int j = 0; j < D; ++j) {
        const size_t src = ((static_cast<size_t>(b) * kBlock + r) * hkv + g) * D + j;
        kh[static_cast<size_t>(nblk * kBlock + r) * D + j] = half_to_double(k_tail[src]);
        vh[static_cast<size_t>(nblk * kBlock + r) * D + j] = half_to_double(v_tail[src]);
      }
    std::vector<double> logit(rows);
    for (int h : heads[u]) {
      double* o = out + (static_cast<size_t>(b) * hq + h) * D;
      if (rows == 0) {
        for (int j = 0; j < D; ++j) o[j] = 0.0;
        continue;
      }
      const uint16_t* qh = q + (static_cast<size_t>(b) * hq + h) * D;
      double mx = -INFINITY;
      for (int i = 0; i < rows; ++i) {
        double s = 0.0;
        for (int j = 0; j < D; ++j) s += kh[static_cast<size_t>(i) * D + j] * half_to_double(qh[j]);
        logit[i] = scale * s;
        mx = std::max(mx, logit[i]);
      }
      double sum = 0.0;
      for (int i = 0; i < rows; ++i) {
        logit[i] = std::exp(logit[i] - mx);
        sum += logit[i];
      }
      for (int j = 0; j < D; ++j) o[j] = 0.0;
      for (int i = 0; i < rows; ++i) {
        const double p = logit[i] / sum;
        for (int j = 0; j < D; ++j) o[j] += p * vh[static_cast<size_t>(i) * D + j];
      }
    }
  });
  return 0;
}

}  // extern "C"
