// oracle_check.cpp -- drives every entry point of the CPU oracle on small inputs,
// including the edge cases (NaN, infinite and huge offsets, samples outside the image,
// RoIs outside the batch, empty batches, offset groups, invalid descriptors), so that
// a build with AddressSanitizer and UndefinedBehaviorSanitizer sees every code path.
// Test infrastructure: built and run by tests/test_sanitizers.py on the CPU.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <vector>

#include "dcn_oracle.h"

namespace {

unsigned rng_state = 12345u;
float urand(float lo, float hi) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return lo + (hi - lo) * static_cast<float>(rng_state >> 8) / 16777216.0f;
}

// one element more than asked, so an empty array still has an address
std::vector<float> rnd(size_t n, float lo, float hi) {
  std::vector<float> v(n + 1);
  for (auto& e : v) e = urand(lo, hi);
  return v;
}

int fails = 0;
void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAIL %s\n", what);
    ++fails;
  }
}

void run_conv(int64_t B, int64_t Cin, int64_t H, int64_t W, int64_t Cout, int64_t K, int64_t s, int64_t p,
              int64_t d, int64_t G, bool with_mask, bool specials) {
  oracle_desc desc{B, Cin, H, W, Cout, K, s, p, d, G};
  int64_t Ho = 0, Wo = 0;
  if (oracle_output_hw(&desc, &Ho, &Wo) != 0) {
    expect(false, "output_hw");
    return;
  }
  const int64_t Gx = G > 1 ? G : 1, KK = K * K;
  auto x = rnd(B * Cin * H * W, -1.f, 1.f);
  auto off = rnd(B * 2 * KK * Gx * Ho * Wo, -3.f, 3.f);
  if (specials) {
    const float sp[] = {std::numeric_limits<float>::quiet_NaN(), std::numeric_limits<float>::infinity(),
                        -std::numeric_limits<float>::infinity(), 1e30f, -1e30f, 0.5f};
    for (size_t i = 0; i + 1 < off.size(); i += 3) off[i] = sp[i % 6];
  }
  auto m = rnd(B * KK * Gx * Ho * Wo, 0.f, 1.f);
  auto w = rnd(Cout * Cin * KK, -1.f, 1.f);
  auto bias = rnd(Cout, -1.f, 1.f);
  const float* mp = with_mask ? m.data() : nullptr;
  std::vector<double> y(B * Cout * Ho * Wo + 1), a(y.size());
  expect(oracle_forward(&desc, x.data(), off.data(), mp, w.data(), bias.data(), 0, Cout, y.data(), a.data(), 2) == 0,
         "forward");
  for (size_t i = 0; i + 1 < y.size(); ++i) expect(std::isfinite(y[i]) && a[i] >= 0.0, "forward finite");
  if (B > 0 && Cout > 0) {
    std::vector<int64_t> pts = {0, 0, 0, 0, B - 1, Cout - 1, Ho - 1, Wo - 1};
    double py[2], pa[2];
    expect(oracle_points(&desc, x.data(), off.data(), mp, w.data(), nullptr, pts.data(), 2, py, pa, 1) == 0,
           "points");
  }
  auto gy = rnd(B * Cout * Ho * Wo + 1, -1.f, 1.f);
  std::vector<double> gx(B * Cin * H * W + 1), go(off.size() + 1), gm(m.size() + 1), gw(w.size()), gb(Cout + 1);
  expect(oracle_backward(&desc, x.data(), off.data(), mp, w.data(), gy.data(), gx.data(), go.data(),
                         with_mask ? gm.data() : nullptr, gw.data(), gb.data(), 2) == 0,
         "backward");
}

void run_roi() {
  const int64_t B = 2, C = 3, H = 9, W = 11, k = 3, S = 2;
  const float rois[] = {0, 1, 1, 6, 7,   1, -5, -5, 30, 40,   2, 1, 1, 5, 5,   -1, 0, 0, 3, 3,
                        0, 100, 100, 120, 130,   1, 2.5f, 3.5f, 2.5f, 3.5f};
  const int64_t R = 6;
  oracle_roi_desc d{B, C, H, W, R, k, S, 0.5, 0.3};
  auto x = rnd(B * C * H * W, -1.f, 1.f);
  auto off = rnd(R * 2 * k * k, -1.f, 1.f);
  auto m = rnd(R * k * k, 0.f, 1.f);
  std::vector<double> y(R * C * k * k), a(y.size());
  expect(oracle_roi_pool(&d, x.data(), rois, off.data(), m.data(), y.data(), a.data(), 2) == 0, "roi");
  expect(oracle_roi_pool(&d, x.data(), rois, nullptr, nullptr, y.data(), nullptr, 1) == 0, "roi plain");
}

}  // namespace

int main() {
  run_conv(2, 5, 9, 11, 7, 3, 1, 1, 1, 1, true, false);
  run_conv(1, 6, 8, 7, 4, 3, 2, 2, 2, 2, true, true);
  run_conv(2, 4, 5, 6, 3, 1, 1, 0, 1, 1, false, true);
  run_conv(1, 3, 12, 10, 2, 5, 3, 2, 2, 3, true, false);
  run_conv(0, 3, 6, 6, 2, 3, 1, 1, 1, 1, true, false);   // empty batch
  run_conv(1, 3, 6, 6, 0, 3, 1, 1, 1, 1, true, false);   // no output channels
  run_conv(1, 2, 1, 1, 3, 3, 1, 1, 1, 1, true, true);    // 1 x 1 image
  run_roi();
  // invalid descriptors are rejected without touching the outputs
  oracle_desc bad{1, 3, 4, 4, 2, 3, 0, 1, 1, 1};
  int64_t ho = 0, wo = 0;
  expect(oracle_output_hw(&bad, &ho, &wo) != 0, "stride 0 rejected");
  oracle_desc bad2{1, 3, 2, 2, 2, 5, 1, 0, 1, 1};
  expect(oracle_output_hw(&bad2, &ho, &wo) != 0, "empty output rejected");
  std::printf("%s\n", fails == 0 ? "ORACLE SANITIZE OK" : "ORACLE SANITIZE FAILED");
  return fails == 0 ? 0 : 1;
}
