// Self-test of the C++ oracle (kvarn_oracle.cpp), TEST INFRASTRUCTURE ONLY.
//
// Built with g++ under AddressSanitizer + UndefinedBehaviorSanitizer (and, separately, under
// ThreadSanitizer for the threaded driver) and run by the CPU tests: every exported function over every
// format and head size, with the edge cases the oracle promises to handle (pages out of range,
// lengths below 0 or past the block table, empty sequences, pairs out of range), and a few checks that
// need nothing but the mathematics: fp16 round trips of every code, the Hadamard matrix being its own
// inverse, FWHT agreeing with the dense product, reconstruction within the grid's reach, decode equal
// to plain softmax attention over the rebuilt pages, and the same bytes from 1 and 4 threads.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
long kvo_page_bytes(int head_dim, int bits, int group, int is_v);
double kvo_half_to_double(uint16_t h);
uint16_t kvo_double_to_half(double x);
int kvo_rotate(const double* x, int rows, int D, int fwht, double* out);
int kvo_normalize(const double* r, int rows, int cols, int iters, double eps, double* rho, double* gam);
long kvo_quantize_blocks(const uint16_t* k, const uint16_t* v, int n_blocks, int hkv, int head_dim,
                         const int32_t* dst_pages, uint8_t* k_pool, uint8_t* v_pool, int num_pages, int kbits,
                         int vbits, int group, int fwht, int threads);
int kvo_dequantize_page(const uint8_t* page, int is_v, int head_dim, int bits, int group, int fwht, double* out);
int kvo_decode(const uint16_t* q, const uint8_t* k_pool, const uint8_t* v_pool, int num_pages,
               const int32_t* block_table, int max_blocks, const int32_t* seq_lens, const uint16_t* k_tail,
               const uint16_t* v_tail, int batch, int hq, int hkv, int head_dim, int kbits, int vbits, int group,
               double softmax_scale, const int32_t* pairs, int n_pairs, int fwht, int threads, double* out);
}

namespace {

long g_checks = 0, g_failures = 0;

void check(bool ok, const char* what, double a = 0, double b = 0) {
  ++g_checks;
  if (!ok && ++g_failures <= 20) std::printf("FAILED: %s (%g, %g)\n", what, a, b);
}

bool is_nan_half(uint16_t h) { return (h & 0x7C00) == 0x7C00 && (h & 0x03FF) != 0; }

void test_half() {
  for (uint32_t h = 0; h < 65536; ++h) {
    const uint16_t x = static_cast<uint16_t>(h);
    if (is_nan_half(x)) {
      check(std::isnan(kvo_half_to_double(x)), "NaN code decodes to NaN", h);
      continue;
    }
    const uint16_t back = kvo_double_to_half(kvo_half_to_double(x));
    check(back == x, "fp16 round trip", h, back);
  }
  // round to nearest, ties to even, overflow to infinity, gradual underflow
  check(kvo_double_to_half(1.0 + std::ldexp(1.0, -11)) == 0x3C00, "tie rounds to even (down)");
  check(kvo_double_to_half(1.0 + 3 * std::ldexp(1.0, -11)) == 0x3C02, "tie rounds to even (up)");
  check(kvo_double_to_half(65504.0) == 0x7BFF, "largest finite");
  check(kvo_double_to_half(65520.0) == 0x7C00, "overflow to infinity");
  check(kvo_double_to_half(-65520.0) == 0xFC00, "overflow to -infinity");
  check(kvo_double_to_half(std::ldexp(1.0, -24)) == 0x0001, "smallest subnormal");
  check(kvo_double_to_half(std::ldexp(1.0, -25)) == 0x0000, "half the smallest subnormal rounds to 0");
  check(kvo_double_to_half(1.5 * std::ldexp(1.0, -25)) == 0x0001, "above half rounds up");
  check(is_nan_half(kvo_double_to_half(std::nan(""))), "NaN encodes to NaN");
}

std::vector<double> gaussian(size_t n, unsigned seed, double scale = 1.0) {
  std::mt19937_64 g(seed);
  std::normal_distribution<double> d(0.0, scale);
  std::vector<double> x(n);
  for (double& v : x) v = d(g);
  return x;
}

void test_rotate_normalize() {
  for (int D : {64, 128, 256}) {
    const int rows = 5;
    std::vector<double> x = gaussian(static_cast<size_t>(rows) * D, D);
    std::vector<double> dense(x.size()), fast(x.size()), twice(x.size());
    check(kvo_rotate(x.data(), rows, D, 0, dense.data()) == 0, "rotate dense");
    check(kvo_rotate(x.data(), rows, D, 1, fast.data()) == 0, "rotate fwht");
    check(kvo_rotate(dense.data(), rows, D, 1, twice.data()) == 0, "rotate back");
    double dmax = 0, imax = 0, n0 = 0, n1 = 0;
    for (size_t i = 0; i < x.size(); ++i) {
      dmax = std::fmax(dmax, std::fabs(dense[i] - fast[i]));
      imax = std::fmax(imax, std::fabs(twice[i] - x[i]));
      n0 += x[i] * x[i];
      n1 += dense[i] * dense[i];
    }
    check(dmax <= 1e-12, "FWHT equals the dense product", D, dmax);
    check(imax <= 1e-12, "the rotation is its own inverse", D, imax);
    check(std::fabs(n0 - n1) <= 1e-9 * n0, "the rotation keeps norms", D, n1 - n0);
    // normalisation of a block with outliers, of a constant block and of a zero block
    std::vector<double> r = gaussian(static_cast<size_t>(128) * D, 7 * D);
    for (int t = 0; t < 128; ++t) r[static_cast<size_t>(t) * D + 3] *= 40.0;
    std::vector<double> rho(128), gam(D);
    for (int kind = 0; kind < 3; ++kind) {
      if (kind == 1) std::fill(r.begin(), r.end(), 2.5);
      if (kind == 2) std::fill(r.begin(), r.end(), 0.0);
      check(kvo_normalize(r.data(), 128, D, 4, 1e-6, rho.data(), gam.data()) == 0, "normalize");
      bool finite = true;
      for (double v : rho) finite = finite && std::isfinite(v);
      for (double v : gam) finite = finite && std::isfinite(v);
      check(finite, "normalisers finite", D, kind);
    }
  }
  double x[4] = {1, 2, 3, 4}, y[4];
  check(kvo_rotate(x, 1, 3, 1, y) == -1 && kvo_rotate(x, 1, 0, 0, y) == -1, "rotate rejects a non power of two");
  check(kvo_normalize(x, 0, 4, 4, 1e-6, y, y) == -1 && kvo_normalize(x, 1, 4, -1, 1e-6, y, y) == -1,
        "normalize rejects bad shapes");
}

std::vector<uint16_t> halves(const std::vector<double>& x) {
  std::vector<uint16_t> h(x.size());
  for (size_t i = 0; i < x.size(); ++i) h[i] = kvo_double_to_half(x[i]);
  return h;
}

// relative Frobenius error of page `p`, head `h` against the fp16 input block b
double rebuild_error(const uint8_t* pool, long pb, int is_v, int D, int bits, int group, const std::vector<uint16_t>& x,
                     int b, int h, int hkv, int p) {
  std::vector<double> out(static_cast<size_t>(128) * D);
  check(kvo_dequantize_page(pool + (static_cast<size_t>(p) * hkv + h) * pb, is_v, D, bits, group, 1, out.data()) == 0,
        "dequantize");
  double e = 0, n = 0;
  for (int t = 0; t < 128; ++t)
    for (int j = 0; j < D; ++j) {
      const double ref = kvo_half_to_double(x[((static_cast<size_t>(b) * 128 + t) * hkv + h) * D + j]);
      e += (out[static_cast<size_t>(t) * D + j] - ref) * (out[static_cast<size_t>(t) * D + j] - ref);
      n += ref * ref;
    }
  return std::sqrt(e / n);
}

void test_formats() {
  const int n_blocks = 3, hkv = 2, num_pages = 5;
  const int32_t dst[n_blocks] = {3, -1, 0};  // block 1 names no page
  for (int D : {64, 128, 256})
    for (int kb : {4, 8})
      for (int vb : {2, 4})
        for (int g : {64, 128}) {
          const long kpb = kvo_page_bytes(D, kb, g, 0), vpb = kvo_page_bytes(D, vb, g, 1);
          check(kpb > 0 && vpb > 0, "page bytes");
          const size_t n = static_cast<size_t>(n_blocks) * 128 * hkv * D;
          std::vector<double> kd = gaussian(n, 11 + D + kb), vd = gaussian(n, 13 + D + vb);
          for (size_t i = 5; i < n; i += D) kd[i] *= 20.0;  // an outlier channel
          const std::vector<uint16_t> k = halves(kd), v = halves(vd);
          std::vector<uint8_t> kp1(static_cast<size_t>(num_pages) * hkv * kpb, 0xA5), vp1(static_cast<size_t>(num_pages) * hkv * vpb, 0xA5);
          std::vector<uint8_t> kp4 = kp1, vp4 = vp1;
          const long bad1 = kvo_quantize_blocks(k.data(), v.data(), n_blocks, hkv, D, dst, kp1.data(), vp1.data(),
                                                num_pages, kb, vb, g, 1, 1);
          const long bad4 = kvo_quantize_blocks(k.data(), v.data(), n_blocks, hkv, D, dst, kp4.data(), vp4.data(),
                                                num_pages, kb, vb, g, 0, 4);
          check(bad1 == 1 && bad4 == 1, "one block without a page", bad1, bad4);
          check(kp1 == kp4 && vp1 == vp4, "1 and 4 threads, FWHT and dense: the same bytes", D, kb);
          bool untouched = true;
          for (int p : {1, 2, 4})
            for (long i = 0; i < hkv * kpb; ++i) untouched = untouched && kp1[static_cast<size_t>(p) * hkv * kpb + i] == 0xA5;
          check(untouched, "pages no block names stay untouched", D);
          // reach of the grids: error of round to nearest on normalised data, loosely bounded
          const double kmax = kb == 4 ? 0.12 : 0.01, vmax = vb == 2 ? 0.6 : 0.12;
          for (int h = 0; h < hkv; ++h) {
            const double ek = rebuild_error(kp1.data(), kpb, 0, D, kb, g, k, 0, h, hkv, 3);
            const double ev = rebuild_error(vp1.data(), vpb, 1, D, vb, g, v, 2, h, hkv, 0);
            check(ek < kmax, "K rebuilt within the grid's reach", D * 100 + kb, ek);
            check(ev < vmax, "V rebuilt within the grid's reach", D * 100 + vb, ev);
          }
          check(kvo_quantize_blocks(k.data(), v.data(), 0, hkv, D, dst, kp1.data(), vp1.data(), num_pages, kb, vb, g, 1,
                                    4) == 0, "no blocks");
        }
  check(kvo_page_bytes(96, 4, 128, 0) == 0 && kvo_page_bytes(128, 3, 128, 0) == 0 && kvo_page_bytes(128, 4, 32, 1) == 0,
        "unknown formats have no page size");
}

void test_decode() {
  const int D = 128, kb = 4, vb = 2, g = 128, hkv = 2, hq = 4, batch = 5, max_blocks = 2, num_pages = 4;
  const long kpb = kvo_page_bytes(D, kb, g, 0), vpb = kvo_page_bytes(D, vb, g, 1);
  const size_t n = static_cast<size_t>(num_pages) * 128 * hkv * D;
  const std::vector<uint16_t> k = halves(gaussian(n, 21)), v = halves(gaussian(n, 22));
  const int32_t dst[num_pages] = {0, 1, 2, 3};
  std::vector<uint8_t> kp(static_cast<size_t>(num_pages) * hkv * kpb), vp(static_cast<size_t>(num_pages) * hkv * vpb);
  check(kvo_quantize_blocks(k.data(), v.data(), num_pages, hkv, D, dst, kp.data(), vp.data(), num_pages, kb, vb, g, 1,
                            2) == 0, "pages for decode");
  const std::vector<uint16_t> q = halves(gaussian(static_cast<size_t>(batch) * hq * D, 23));
  const std::vector<uint16_t> kt = halves(gaussian(static_cast<size_t>(batch) * 128 * hkv * D, 24));
  const std::vector<uint16_t> vt = halves(gaussian(static_cast<size_t>(batch) * 128 * hkv * D, 25));
  // table: sequence 1 names a page out of range; lengths: two pages, empty, below 0, past the table, a tail
  const int32_t table[batch * max_blocks] = {2, 0, 1, 7, 3, 3, 0, 1, 1, 2};
  const int32_t lens[batch] = {256, 0, -5, 128 * max_blocks + 128, 128 + 77};
  std::vector<double> out(static_cast<size_t>(batch) * hq * D, -7.0), out4(out.size(), -7.0);
  check(kvo_decode(q.data(), kp.data(), vp.data(), num_pages, table, max_blocks, lens, nullptr, nullptr, batch, hq, hkv,
                   D, kb, vb, g, 0.0, nullptr, 0, 1, 1, out.data()) == 0, "decode");
  check(kvo_decode(q.data(), kp.data(), vp.data(), num_pages, table, max_blocks, lens, nullptr, nullptr, batch, hq, hkv,
                   D, kb, vb, g, 0.0, nullptr, 0, 0, 4, out4.data()) == 0, "decode, 4 threads, dense");
  double dmax = 0;
  for (size_t i = 0; i < out.size(); ++i) dmax = std::fmax(dmax, std::fabs(out[i] - out4[i]));
  check(dmax <= 1e-12, "decode: threads and rotation modes agree", dmax);
  for (int b : {1, 2, 3}) {
    bool zero = true;
    for (int i = 0; i < hq * D; ++i) zero = zero && out[static_cast<size_t>(b) * hq * D + i] == 0.0;
    check(zero, "sequence with no rows gives zeros", b);
  }
  // sequence 0, query head 3 (KV head 1): plain softmax attention over the rebuilt pages
  {
    std::vector<double> kh(256 * D), vh(256 * D);
    for (int i = 0; i < 2; ++i) {
      kvo_dequantize_page(kp.data() + (static_cast<size_t>(table[i]) * hkv + 1) * kpb, 0, D, kb, g, 1, &kh[i * 128 * D]);
      kvo_dequantize_page(vp.data() + (static_cast<size_t>(table[i]) * hkv + 1) * vpb, 1, D, vb, g, 1, &vh[i * 128 * D]);
    }
    std::vector<double> w(256);
    double mx = -INFINITY, sum = 0;
    for (int t = 0; t < 256; ++t) {
      double s = 0;
      for (int j = 0; j < D; ++j) s += kh[t * D + j] * kvo_half_to_double(q[3 * D + j]);
      w[t] = s / std::sqrt(static_cast<double>(D));
      mx = std::fmax(mx, w[t]);
    }
    for (int t = 0; t < 256; ++t) sum += (w[t] = std::exp(w[t] - mx));
    double err = 0;
    for (int j = 0; j < D; ++j) {
      double o = 0;
      for (int t = 0; t < 256; ++t) o += w[t] / sum * vh[t * D + j];
      err = std::fmax(err, std::fabs(o - out[3 * D + j]));
    }
    check(err <= 1e-12, "decode equals attention over the rebuilt pages", err);
  }
  // tails: sequence 4 has one page and 77 fp16 rows; sequence 3 (past the table) still gives zeros
  std::vector<double> outt(out.size(), -7.0);
  check(kvo_decode(q.data(), kp.data(), vp.data(), num_pages, table, max_blocks, lens, kt.data(), vt.data(), batch, hq,
                   hkv, D, kb, vb, g, 0.0, nullptr, 0, 1, 3, outt.data()) == 0, "decode with tails");
  bool finite = true, zero3 = true;
  for (int i = 0; i < hq * D; ++i) {
    finite = finite && std::isfinite(outt[4 * hq * D + i]);
    zero3 = zero3 && outt[3 * hq * D + i] == 0.0;
  }
  check(finite && zero3, "tails: finite rows, out-of-table sequence zero");
  // pairs: only the listed rows are written; a pair out of range is refused before any work
  std::vector<double> outp(out.size(), -7.0);
  const int32_t pairs[4] = {0, 3, 4, 1};
  check(kvo_decode(q.data(), kp.data(), vp.data(), num_pages, table, max_blocks, lens, nullptr, nullptr, batch, hq, hkv,
                   D, kb, vb, g, 0.0, pairs, 2, 1, 2, outp.data()) == 0, "decode of pairs");
  check(outp[3 * D] == out[3 * D] && outp[0] == -7.0 && outp[(4 * hq + 1) * D] == out[(4 * hq + 1) * D],
        "pairs: listed rows written, others untouched");
  const int32_t bad_pairs[4] = {0, 3, 5, 0};
  std::vector<double> outb(out.size(), -7.0);
  check(kvo_decode(q.data(), kp.data(), vp.data(), num_pages, table, max_blocks, lens, nullptr, nullptr, batch, hq, hkv,
                   D, kb, vb, g, 0.0, bad_pairs, 2, 1, 2, outb.data()) == -1 && outb[3 * D] == -7.0,
        "a pair out of range is refused");
  check(kvo_decode(q.data(), kp.data(), vp.data(), num_pages, table, max_blocks, lens, nullptr, nullptr, batch, 3, hkv,
                   D, kb, vb, g, 0.0, nullptr, 0, 1, 2, outb.data()) == -1, "query heads not a multiple");
}

}  // namespace

int main() {
  test_half();
  test_rotate_normalize();
  test_formats();
  test_decode();
  std::printf("oracle self-test: %ld checks, %ld failed\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
