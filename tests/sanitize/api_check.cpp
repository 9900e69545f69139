// api_check.cpp -- drives the host side of the C ABI (descriptor checks, output size,
// planner, workspace sizing, plan descriptions, argument errors) with no GPU, so a
// host build with AddressSanitizer and UndefinedBehaviorSanitizer sees those paths.
// No call here reaches a kernel launch: each one returns from the host checks.
// Test infrastructure: built and run by tests/test_sanitizers.py on the CPU.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "dcn.h"

namespace {

int fails = 0;
void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAIL %s\n", what);
    ++fails;
  }
}

dcn_desc make(int64_t B, int64_t C, int64_t H, int64_t W, int64_t O, int64_t K, int64_t s, int64_t p, int64_t d,
              int32_t dt, int32_t G = 1) {
  dcn_desc x;
  std::memset(&x, 0, sizeof(x));
  x.batch = B;
  x.in_channels = C;
  x.height = H;
  x.width = W;
  x.out_channels = O;
  x.kernel_size = K;
  x.stride = s;
  x.pad = p;
  x.dilation = d;
  x.dtype = dt;
  x.offset_groups = G;
  return x;
}

void plan_all(const dcn_desc& d) {
  int64_t ho = 0, wo = 0;
  const int rc = dcn_output_hw(&d, &ho, &wo);
  size_t nb = 0;
  const int rw = dcn_workspace_bytes(&d, &nb);
  (void)dcn_variant_name(&d);
  char buf[512], tiny[8];
  (void)dcn_plan_describe(&d, buf, sizeof(buf));
  (void)dcn_plan_describe(&d, tiny, sizeof(tiny));
  size_t nom = 0, nbw = 0;
  (void)dcn_offset_mask_workspace_bytes(&d, &nom);
  (void)dcn_backward_workspace_bytes(&d, &nbw);
  if (rc == DCN_OK && rw == DCN_OK) {
    // every required pointer null: rejected before any launch
    expect(dcn_forward(&d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) != DCN_OK ||
               d.batch == 0 || d.out_channels == 0,
           "forward with null pointers");
    // a workspace that is too small, with non-null (never dereferenced) tensors
    if (nb > 0) {
      char dummy[16];
      expect(dcn_forward(&d, dummy, dummy, nullptr, dummy, nullptr, dummy, dummy, nb - 1, nullptr) ==
                 DCN_E_WORKSPACE,
             "forward with a small workspace");
      expect(dcn_stage(&d, dummy, dummy, nullptr, nb, nullptr) == DCN_E_WORKSPACE, "stage without workspace");
    }
    expect(dcn_backward(&d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr, 0, nullptr) != DCN_OK ||
               d.batch == 0 || d.out_channels == 0,
           "backward with null pointers");
  }
}

}  // namespace

int main() {
  const int32_t F = DCN_F32, BF = DCN_BF16;
  // the named layers and edge shapes, both element types
  const dcn_desc shapes[] = {
      make(1, 3, 32, 32, 8, 3, 1, 1, 1, F),       make(1, 3, 224, 224, 64, 3, 1, 1, 1, F),
      make(2, 128, 100, 168, 128, 3, 1, 1, 1, BF), make(2, 256, 100, 168, 256, 3, 2, 1, 1, BF),
      make(8, 512, 25, 42, 512, 3, 1, 2, 2, BF),   make(2, 256, 100, 168, 256, 3, 2, 1, 1, BF, 4),
      make(3, 37, 11, 13, 70, 3, 1, 1, 1, BF),     make(2, 16, 9, 7, 24, 1, 1, 0, 1, F),
      make(1, 12, 23, 19, 40, 5, 3, 2, 2, BF),     make(2, 8, 1, 1, 5, 3, 1, 1, 1, BF),
      make(1, 64, 12, 14, 300, 3, 1, 1, 1, BF),    make(0, 8, 9, 9, 4, 3, 1, 1, 1, BF),
      make(2, 8, 9, 9, 0, 3, 1, 1, 1, F),          make(1, 48, 30, 26, 96, 5, 2, 2, 1, BF),
      make(2, 64, 17, 19, 130, 1, 1, 0, 1, BF),    make(1, 64, 12, 14, 130, 5, 1, 2, 1, BF, 8),
  };
  for (const dcn_desc& d : shapes) {
    plan_all(d);
    dcn_desc f = d;
    f.dtype = (d.dtype == F) ? BF : F;
    plan_all(f);
  }
  // invalid descriptors: every entry point rejects them
  const dcn_desc bad[] = {
      make(1, 0, 9, 9, 4, 3, 1, 1, 1, F),  make(1, 8, 9, 9, 4, 0, 1, 1, 1, F),  make(1, 8, 9, 9, 4, 3, 0, 1, 1, F),
      make(1, 8, 9, 9, 4, 3, 1, -1, 1, F), make(1, 8, 2, 2, 4, 5, 1, 0, 1, F),  make(-1, 8, 9, 9, 4, 3, 1, 1, 1, F),
      make(1, 9, 9, 9, 4, 3, 1, 1, 1, F, 2), make(1, 8, 9, 9, 4, 3, 1, 1, 1, 7),
      make(1, 8, int64_t(1) << 40, 9, 4, 3, 1, 1, 1, BF),
  };
  for (const dcn_desc& d : bad) {
    int64_t ho, wo;
    size_t nb;
    expect(dcn_output_hw(&d, &ho, &wo) != DCN_OK || dcn_workspace_bytes(&d, &nb) != DCN_OK, "bad descriptor");
    plan_all(d);
  }
  expect(dcn_output_hw(nullptr, nullptr, nullptr) == DCN_E_ARG, "null descriptor");
  expect(std::strcmp(dcn_variant_name(nullptr), "invalid") == 0, "variant of null");
  // the tuning variables, well-formed and not
  const char* tiles[] = {"4,5,10", "garbage", "99,1,1", ""};
  for (const char* t : tiles) {
    setenv("DCN_BOX_TILE", t, 1);
    setenv("DCN_BOX_PW", "8", 1);
    setenv("DCN_BOX_ROLES", "1", 1);
    plan_all(shapes[3]);
  }
  setenv("DCN_VARIANT", "no_such_variant", 1);
  plan_all(shapes[3]);
  unsetenv("DCN_VARIANT");
  unsetenv("DCN_BOX_TILE");
  unsetenv("DCN_BOX_PW");
  unsetenv("DCN_BOX_ROLES");
  // RoI pooling descriptors
  dcn_roi_desc r;
  std::memset(&r, 0, sizeof(r));
  r.batch = 2;
  r.channels = 256;
  r.height = 50;
  r.width = 84;
  r.num_rois = 512;
  r.pooled_size = 7;
  r.samples = 2;
  r.spatial_scale = 1.0f / 16;
  r.gamma = 0.1f;
  r.dtype = BF;
  size_t nb = 0;
  expect(dcn_roi_pool_workspace_bytes(&r, &nb) == DCN_OK, "roi workspace");
  expect(dcn_roi_pool(&r, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) != DCN_OK,
         "roi with null pointers");
  r.pooled_size = 0;
  expect(dcn_roi_pool_workspace_bytes(&r, &nb) != DCN_OK, "roi k = 0");
  for (int s = -3; s < 8; ++s) expect(dcn_status_str(s) != nullptr, "status string");
  std::printf("%s\n", fails == 0 ? "API SANITIZE OK" : "API SANITIZE FAILED");
  return fails == 0 ? 0 : 1;
}
