// dcn_api.hip -- host side of the C ABI declared in include/dcn.h: argument
// validation, output geometry, workspace layout, variant choice and launches.
// Every check happens before the first HIP call; nothing here allocates or
// synchronises.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <mutex>

#include "dcn.h"
#include "dcn_internal.h"

namespace {

using dcn::FusedArgs;
using dcn::StageArgs;

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;   // int32 element indexing
constexpr size_t kAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Output size of the strided, padded, dilated window, as for a regular
// convolution (torchvision deform_conv2d parameter table: stride, padding,
// dilation).  Returns 0 when the window does not fit.
int64_t out_extent(int64_t in, int64_t K, int64_t stride, int64_t pad, int64_t dil) {
  const int64_t span = in + 2 * pad - dil * (K - 1) - 1;
  return span < 0 ? 0 : span / stride + 1;
}

struct BoxPlan {
  int fm = 0, fn = 0;           // MT = 64*fm output channels, 16*fn pixel slots
  int TH = 0, TW = 0, tiles_x = 0, tiles_per_img = 0;
  int box_px = 0, lds = 0;
  int split = 0;                // BoxArgs::split_roles
  int pw = 4;                   // BoxArgs::pw
  double cost = 1e300;
};

struct Plan {
  int64_t Ho = 0, Wo = 0;
  int variant = -1;
  int64_t Cp = 0, Mp = 0;       // channel and output-channel padding of the staged buffers
  size_t ws_x = 0, ws_w = 0;    // workspace byte offsets
  size_t ws_bytes = 0;
  bool empty = false;           // B == 0 or Cout == 0: nothing to launch
  BoxPlan box;
};

bool geometry_ok(const dcn_desc* d) {
  if (d == nullptr || d->offset_groups < 0) return false;
  if (d->batch < 0 || d->out_channels < 0) return false;
  if (d->in_channels < 1 || d->height < 1 || d->width < 1 || d->kernel_size < 1) return false;
  if (d->stride < 1 || d->dilation < 1 || d->pad < 0) return false;
  // keep intermediate products far from int64 overflow
  const int64_t big = int64_t(1) << 30;
  if (d->height > big || d->width > big || d->kernel_size > 4096 || d->stride > big ||
      d->pad > big || d->dilation > big || d->batch > big || d->in_channels > big ||
      d->out_channels > big)
    return false;
  if (d->offset_groups > 1 && d->in_channels % d->offset_groups != 0) return false;
  return true;
}

int64_t offset_groups(const dcn_desc* d) { return d->offset_groups > 1 ? d->offset_groups : 1; }

// Variants that take offset groups: the tile kernels, when every 16-byte channel
// vector of the staged copy lies in one group; the box kernel for 3x3 when every
// 32-channel chunk does.
bool groups_fit(const dcn_desc* d, int variant) {
  if (offset_groups(d) == 1) return true;
  const dcn::VariantInfo& vi = dcn::variant_info(variant);
  const int64_t Cg = d->in_channels / offset_groups(d);
  if (variant == dcn::V_BOX_BF16_M128 || variant == dcn::V_BOX_BF16_M256)
    return d->kernel_size == 3 && Cg % 32 == 0;
  if (!vi.staged) return false;
  return Cg % (vi.is_bf16 ? 8 : 4) == 0;
}

// Tile plan of the box kernel: the output tile (TH x TW pixels of one image by
// 64*fm output channels) minimising an estimate of the time of the busiest CU,
// assuming one workgroup per CU on 256 CUs.  Per reduction step (32 channels of one
// kernel point) a SIMD runs one consumer wave (fm*fn MFMA 16x16x32, 16 cycles each)
// next to one producer wave (about 50 VALU instructions of 4 cycles per 64 column
// units); per workgroup the vector-memory pipe moves the weight rows and the input
// box at about 50 bytes per cycle.  The workgroup time is the larger of the two,
// times the number of rounds of workgroups.
bool plan_box(const dcn_desc* d, int64_t Ho, int64_t Wo, int fm_only, BoxPlan* out) {
  if (d->dtype != DCN_BF16) return false;
  if (d->height > 32000 || d->width > 32000) return false;
  const int64_t K = d->kernel_size, KK = K * K;
  if (KK > dcn::kBoxMaxKK) return false;
  const int64_t M = d->out_channels, Cp = round_up(d->in_channels, 32), Kr = Cp * KK;
  const int64_t s = d->stride, dil = d->dilation;
  const int64_t steps = (Cp / 32) * KK;
  // 32-bit byte offsets inside the kernel: staged x and repacked weight under 4 GiB
  if (static_cast<double>(d->batch) * d->height * d->width * Cp * 2 >= 4294967296.0) return false;
  if (static_cast<double>(round_up(M, 256)) * Kr * 2 >= 4294967296.0) return false;
  // DCN_BOX_TILE="fn,TH,TW" restricts the search to one tile shape (tile sweeps)
  int want_fn = 0, want_th = 0, want_tw = 0;
  if (const char* t = std::getenv("DCN_BOX_TILE")) {
    if (std::sscanf(t, "%d,%d,%d", &want_fn, &want_th, &want_tw) != 3) want_fn = want_th = want_tw = 0;
  }
  BoxPlan best;
  for (int fm = 2; fm <= 4; fm += 2) {
    if (fm_only && fm != fm_only) continue;
    const int64_t MT = 64 * fm, m_tiles = (M + MT - 1) / MT;
    for (int fn : {4, 6, 8, 10}) {
      if (fm == 4 && fn > 6) continue;
      const int NT = 16 * fn;
      const bool grouped = offset_groups(d) > 1;
      if (grouped && !dcn::box_groups_supported(fm, fn)) continue;
      const int box_px = dcn::box_capacity_px(fn, grouped);
      if (box_px < 64) continue;
      for (int TH = 1; TH <= 16; ++TH) {
        for (int dw = 0; dw < (want_fn ? NT : 3); ++dw) {
          const int TW = NT / TH - dw;
          if (TW < 1 || (TH * TW + 15) / 16 != fn) continue;
          if (want_fn && (fn != want_fn || TH != want_th || TW != want_tw)) continue;
          const int64_t bh0 = (TH - 1) * s + (K - 1) * dil + 2, bw0 = (TW - 1) * s + (K - 1) * dil + 2;
          // the kernel clips the box to one pixel around the image
          if (std::min<int64_t>(bh0, d->height + 2) * std::min<int64_t>(bw0, d->width + 2) > box_px) continue;
          const int64_t ty = (Ho + TH - 1) / TH, tx = (Wo + TW - 1) / TW;
          const int64_t tiles = d->batch * ty * tx * m_tiles;
          if (tiles > (int64_t(1) << 30)) continue;
          const double est_box = std::min<double>(std::min<double>((bh0 + 6) * (bw0 + 6), box_px),
                                                  (d->height + 2.0) * (d->width + 2.0));
          const double mfma_step = double(fm) * fn * 16;
          const double valu_step = std::ceil(NT * 4 / 256.0) * 50 * 4 + 40;
          const double compute = steps * std::max(mfma_step, valu_step);
          const double mem = (double(MT) * Kr * 2 + est_box * Cp * 2) / 50;
          const double wg = std::max(compute, mem) + 4000;
          const double rounds = std::ceil(double(tiles) / 256);
          // margin of the capped box around the offset-free window: samples pushed
          // past it take the slower global path, so thin margins are penalised
          int64_t mg = 0;
          while ((bh0 + 2 * (mg + 1)) * (bw0 + 2 * (mg + 1)) <= box_px) ++mg;
          // tiles about twice as wide as tall measured fastest (rows of the box and of
          // the NCHW output are longer; the margin still grows in both directions)
          const double aspect = std::fabs(std::log2(double(TW) / (2.0 * TH)));
          // an odd tile width (narrower than the output) leaves half the tiles' output
          // column pairs misaligned, stored as single elements (c3: 9x17 -> 10x16 tiles
          // 40.5 -> 39.7 us; c5: 7x13 -> 6x14 98.9 -> 97.1 us); fewer tiles break ties
          const double odd_w = (TW & 1) && TW < Wo ? 1.15 : 1.0;
          const double cost = rounds * wg * (1.0 + 4.0 / (1.0 + static_cast<double>(mg))) * (1.0 + 0.3 * aspect) *
                              odd_w * (1.0 + 1e-6 * static_cast<double>(tiles));
          if (cost < best.cost) {
            best.fm = fm;
            best.fn = fn;
            best.TH = TH;
            best.TW = TW;
            best.tiles_x = static_cast<int>(tx);
            best.tiles_per_img = static_cast<int>(ty * tx);
            best.box_px = box_px;
            best.lds = dcn::kLdsBudget;
            best.cost = cost;
          }
        }
      }
    }
  }
  if (best.fm == 0) return false;
  // Eight producer waves (two per SIMD, 4 channels per thread and sample) where that
  // kernel is built (256 x 64 and 256 x 96, 128 x 128 and 128 x 160 tiles; 3x3, one
  // offset group), on paired roles (c4 layer: 33.1 -> 31.6 us; the c5 layer's 6x14 tiles:
  // 93.1 us, against 96.4 us with four producer waves on split roles).
  // Otherwise four producer waves, and for 256 output channels and 96 pixel slots (12
  // matrix instructions per consumer wave and step, two samples per producer thread)
  // split roles: the consumers and producers do not share SIMDs (c5, 6x14 tiles: 104.9
  // -> 96.4 us); with 64 slots, halving the SIMDs that run matrix instructions costs more
  // than it saves (c4: 36 -> 38 us).
  // DCN_BOX_PW=4|8 pins the producer waves where built.
  const bool pw8_built = dcn::box_pw8_supported(best.fm, best.fn) && d->kernel_size == 3 && offset_groups(d) == 1;
  best.split = best.fm == 4 && best.fn == 6 && !pw8_built;
  best.pw = pw8_built ? 8 : 4;
  if (const char* w = std::getenv("DCN_BOX_PW")) {
    if (w[0] == '4') {   // four producer waves, on the roles that suit them
      best.pw = 4;
      best.split = best.fm == 4 && best.fn == 6;
    }
    if (w[0] == '8' && pw8_built) {
      best.pw = 8;
      best.split = 0;
    }
  }
  // DCN_BOX_ROLES=0|1 pins the role placement (split roles: four producer waves)
  if (const char* r = std::getenv("DCN_BOX_ROLES")) {
    if (r[0] == '0' || r[0] == '1') best.split = r[0] - '0';
    if (best.split) best.pw = 4;
  }
  *out = best;
  return true;
}

// The direct kernel: at most 4 input channels, K*K in {1, 4, 9}, and every tensor it
// reads or writes under 2 GiB (it addresses them with 32-bit byte offsets).
bool direct_fits(const dcn_desc* d, int64_t HoWo) {
  const int64_t KK = d->kernel_size * d->kernel_size;
  if (!dcn::direct_supported(static_cast<int>(d->in_channels), static_cast<int>(KK))) return false;
  const double es = d->dtype == DCN_BF16 ? 2.0 : 4.0, lim = 2147483647.0;
  return static_cast<double>(d->batch) * d->in_channels * d->height * d->width * es < lim &&
         static_cast<double>(d->batch) * 2 * KK * HoWo * es < lim &&
         static_cast<double>(d->out_channels) * d->in_channels * KK * es < lim &&
         static_cast<double>(d->batch) * d->out_channels * HoWo * es < lim;
}

// Pick the kernel variant for a valid descriptor.
int choose_variant(const dcn_desc* d, int64_t N, int64_t Ho, int64_t Wo, BoxPlan* bp) {
  const int64_t M = d->out_channels;
  const bool grouped = offset_groups(d) > 1;
  // tiny reductions (an RGB first layer): the column fits in registers
  if (!grouped && direct_fits(d, Ho * Wo))
    return d->dtype == DCN_F32 ? dcn::V_DIRECT_F32 : dcn::V_DIRECT_BF16;
  if (d->dtype == DCN_F32) return M <= 64 ? dcn::V_TILE_F32_M64_N64 : dcn::V_TILE_F32_M128_N64;
  // the box kernel for channel counts where a 32-channel chunk is mostly real data
  // (offset groups: 3x3 with whole 32-channel chunks per group)
  const bool box_groups_ok = !grouped || (d->kernel_size == 3 && (d->in_channels / offset_groups(d)) % 32 == 0);
  if (box_groups_ok && d->in_channels >= 24 && M >= 64 && plan_box(d, Ho, Wo, 0, bp))
    return bp->fm == 2 ? dcn::V_BOX_BF16_M128 : dcn::V_BOX_BF16_M256;
  if (M <= 64) return dcn::V_TILE_BF16_M64_N64;
  // enough workgroups to cover 256 CUs with the wider tile?
  if (M >= 256 && (N + 63) / 64 * ((M + 255) / 256) >= 512) return dcn::V_TILE_BF16_M256_N64;
  if ((N + 63) / 64 * ((M + 127) / 128) >= 512) return dcn::V_TILE_BF16_M128_N64;
  return dcn::V_TILE_BF16_M128_N32;
}

int compute_plan(const dcn_desc* d, Plan* p, int force_variant = -1) {
  if (!geometry_ok(d)) return DCN_E_ARG;
  if (d->dtype != DCN_F32 && d->dtype != DCN_BF16) return DCN_E_UNSUPPORTED;
  p->Ho = out_extent(d->height, d->kernel_size, d->stride, d->pad, d->dilation);
  p->Wo = out_extent(d->width, d->kernel_size, d->stride, d->pad, d->dilation);
  if (p->Ho < 1 || p->Wo < 1) return DCN_E_ARG;
  const int64_t B = d->batch, Cin = d->in_channels, H = d->height, W = d->width;
  const int64_t Cout = d->out_channels, K = d->kernel_size, KK = K * K;
  const int64_t HoWo = p->Ho * p->Wo;
  const int64_t N = B * HoWo;
  const int64_t G = offset_groups(d);
  p->variant = force_variant >= 0 ? force_variant : choose_variant(d, N, p->Ho, p->Wo, &p->box);
  // DCN_VARIANT=<name> pins the kernel variant (tile sweeps and tests); an
  // unknown name or one built for the other dtype is rejected.
  const char* force = force_variant >= 0 ? nullptr : std::getenv("DCN_VARIANT");
  if (force) {
    if (force[0] != '\0') {
      int found = -1;
      for (int v = 0; v < dcn::V_COUNT; ++v)
        if (std::strcmp(force, dcn::variant_info(v).name) == 0) found = v;
      if (found < 0 || found == dcn::V_OM_BF16 || dcn::variant_info(found).is_bf16 != (d->dtype == DCN_BF16))
        return DCN_E_UNSUPPORTED;
      if ((found == dcn::V_DIRECT_F32 || found == dcn::V_DIRECT_BF16) && !direct_fits(d, HoWo))
        return DCN_E_UNSUPPORTED;
      if (found == dcn::V_BOX_BF16_M128 || found == dcn::V_BOX_BF16_M256) {
        if (!plan_box(d, p->Ho, p->Wo, found == dcn::V_BOX_BF16_M128 ? 2 : 4, &p->box)) return DCN_E_UNSUPPORTED;
      }
      p->variant = found;
    }
  }
  if (!groups_fit(d, p->variant)) return DCN_E_UNSUPPORTED;
  const dcn::VariantInfo& vi = dcn::variant_info(p->variant);
  p->Cp = round_up(Cin, vi.ck);
  p->Mp = round_up(Cout > 0 ? Cout : 1, vi.mt);
  // element-count limits (int32 indexing inside the kernels)
  const double lim = static_cast<double>(kMaxElems);
  if (static_cast<double>(B) * Cin * H * W > lim || static_cast<double>(B) * 2 * KK * G * HoWo > lim ||
      static_cast<double>(Cout) * Cin * KK > lim || static_cast<double>(B) * Cout * HoWo > lim ||
      static_cast<double>(B) * H * W * p->Cp > lim || static_cast<double>(p->Mp) * KK * p->Cp > lim ||
      static_cast<double>(N) + vi.nt > lim)
    return DCN_E_UNSUPPORTED;
  // the offset/mask convolution addresses the staged copy with 32-bit byte offsets
  if (p->variant == dcn::V_OM_BF16 && static_cast<double>(B) * H * W * p->Cp * 2 >= 4294967296.0 - 64)
    return DCN_E_UNSUPPORTED;
  const size_t es = d->dtype == DCN_BF16 ? 2 : 4;
  p->empty = (B == 0 || Cout == 0);
  if (vi.staged && !p->empty) {
    p->ws_x = 0;
    p->ws_w = align_up(static_cast<size_t>(B * H * W * p->Cp) * es, kAlign);
    p->ws_bytes = p->ws_w + align_up(static_cast<size_t>(p->Mp * KK * p->Cp) * es, kAlign);
  }
  return DCN_OK;
}

// Plans are cached per descriptor (and the two tuning variables), so repeated calls
// with one shape skip the tile search.  Thread-safe; a small round-robin table.
struct PlanKey {
  dcn_desc d;
  char variant[48], tile[48], roles[8], pw[8];
};
struct PlanSlot {
  bool used = false;
  PlanKey key;
  Plan plan;
};

void fill_key(const dcn_desc* d, PlanKey* k) {
  std::memset(k, 0, sizeof(*k));
  std::memcpy(&k->d, d, sizeof(dcn_desc));
  if (const char* v = std::getenv("DCN_VARIANT")) std::strncpy(k->variant, v, sizeof(k->variant) - 1);
  if (const char* t = std::getenv("DCN_BOX_TILE")) std::strncpy(k->tile, t, sizeof(k->tile) - 1);
  if (const char* r = std::getenv("DCN_BOX_ROLES")) std::strncpy(k->roles, r, sizeof(k->roles) - 1);
  if (const char* w = std::getenv("DCN_BOX_PW")) std::strncpy(k->pw, w, sizeof(k->pw) - 1);
}

int make_plan(const dcn_desc* d, Plan* p) {
  if (d == nullptr) return DCN_E_ARG;
  static std::mutex mu;
  static PlanSlot slots[32];
  static int next = 0;
  PlanKey key;
  fill_key(d, &key);
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const PlanSlot& sl : slots)
      if (sl.used && std::memcmp(&sl.key, &key, sizeof(key)) == 0) {
        *p = sl.plan;
        return DCN_OK;
      }
  }
  Plan fresh;
  const int rc = compute_plan(d, &fresh);
  if (rc != DCN_OK) return rc;
  {
    std::lock_guard<std::mutex> lock(mu);
    PlanSlot& sl = slots[next];
    next = (next + 1) % 32;
    sl.used = true;
    sl.key = key;
    sl.plan = fresh;
  }
  *p = fresh;
  return DCN_OK;
}

int check_workspace(const Plan& p, const void* ws, size_t ws_bytes) {
  if (p.ws_bytes == 0) return DCN_OK;
  if (ws == nullptr || ws_bytes < p.ws_bytes) return DCN_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return DCN_E_WORKSPACE;
  return DCN_OK;
}

bool is_box(int variant) { return variant == dcn::V_BOX_BF16_M128 || variant == dcn::V_BOX_BF16_M256; }
bool is_direct(int variant) { return variant == dcn::V_DIRECT_F32 || variant == dcn::V_DIRECT_BF16; }

StageArgs stage_args(const dcn_desc* d, const Plan& p, const void* x, const void* w, void* ws) {
  StageArgs a{};
  a.x = x;
  a.w = w;
  a.xs = static_cast<unsigned char*>(ws) + p.ws_x;
  a.wp = static_cast<unsigned char*>(ws) + p.ws_w;
  a.B = static_cast<int>(d->batch);
  a.Cin = static_cast<int>(d->in_channels);
  a.HW = static_cast<int>(d->height * d->width);
  a.Cp = static_cast<int>(p.Cp);
  a.Cout = static_cast<int>(d->out_channels);
  a.Mp = static_cast<int>(p.Mp);
  a.KK = static_cast<int>(d->kernel_size * d->kernel_size);
  a.wlayout = p.variant == dcn::V_OM_BF16 ? 2 : is_box(p.variant) ? 1 : 0;
  return a;
}

FusedArgs fused_args(const dcn_desc* d, const Plan& p, const void* x, const void* offset, const void* mask,
                     const void* w, const void* bias, void* out, const void* ws) {
  const dcn::VariantInfo& vi = dcn::variant_info(p.variant);
  const int nt = vi.nt > 0 ? vi.nt : 16 * p.box.fn;
  FusedArgs a{};
  a.xs = ws ? static_cast<const unsigned char*>(ws) + p.ws_x : nullptr;
  a.wp = ws ? static_cast<const unsigned char*>(ws) + p.ws_w : nullptr;
  a.x = x;
  a.w = w;
  a.offset = offset;
  a.mask = mask;
  a.bias = bias;
  a.out = out;
  a.B = static_cast<int>(d->batch);
  a.Cin = static_cast<int>(d->in_channels);
  a.H = static_cast<int>(d->height);
  a.W = static_cast<int>(d->width);
  a.Cp = static_cast<int>(p.Cp);
  a.Cout = static_cast<int>(d->out_channels);
  a.K = static_cast<int>(d->kernel_size);
  a.KK = a.K * a.K;
  a.stride = static_cast<int>(d->stride);
  a.pad = static_cast<int>(d->pad);
  a.dil = static_cast<int>(d->dilation);
  a.G = static_cast<int>(offset_groups(d));
  a.Cg = static_cast<int>(d->in_channels / a.G);
  a.Ho = static_cast<int>(p.Ho);
  a.Wo = static_cast<int>(p.Wo);
  a.HoWo = a.Ho * a.Wo;
  a.N = a.B * a.HoWo;
  a.m_tiles = static_cast<int>(p.Mp / vi.mt);
  a.n_tiles = (a.N + nt - 1) / nt;
  return a;
}

hipError_t launch_fused_plan(const Plan& p, const FusedArgs& a, hipStream_t stream) {
  if (is_direct(p.variant)) return dcn::launch_direct(p.variant == dcn::V_DIRECT_BF16, a, stream);
  if (!is_box(p.variant)) return dcn::launch_fused(p.variant, a, stream);
  dcn::BoxArgs ba{};
  ba.f = a;
  ba.TH = p.box.TH;
  ba.TW = p.box.TW;
  ba.tiles_x = p.box.tiles_x;
  ba.tiles_per_img = p.box.tiles_per_img;
  ba.box_px = p.box.box_px;
  ba.KK_NT = a.KK * 16 * p.box.fn;
  ba.lds_bytes = 0;
  ba.split_roles = p.box.split;
  ba.pw = p.box.pw;
  return dcn::launch_box(p.box.fm, p.box.fn, ba, stream);
}

int check_positions(const dcn_desc* d, int64_t K, int64_t stride, int64_t pad, int64_t dil, int64_t Ho,
                    int64_t Wo) {
  // Base sampling positions oy*stride - pad + i*dilation must be exact in fp32
  // (the fractional offset is added separately): keep them below 2^24.
  const double ymax = static_cast<double>(Ho) * stride + pad + static_cast<double>(K) * dil;
  const double xmax = static_cast<double>(Wo) * stride + pad + static_cast<double>(K) * dil;
  const double hmax = static_cast<double>(d->height) + 2, wmax = static_cast<double>(d->width) + 2;
  const double lim = 16777216.0;
  return (ymax < lim && xmax < lim && hmax < lim && wmax < lim) ? DCN_OK : DCN_E_UNSUPPORTED;
}

}  // namespace

namespace dcn {

int check_desc(const dcn_desc* d, int64_t* Ho, int64_t* Wo) {
  if (!geometry_ok(d)) return DCN_E_ARG;
  if (d->dtype != DCN_F32 && d->dtype != DCN_BF16) return DCN_E_UNSUPPORTED;
  *Ho = out_extent(d->height, d->kernel_size, d->stride, d->pad, d->dilation);
  *Wo = out_extent(d->width, d->kernel_size, d->stride, d->pad, d->dilation);
  if (*Ho < 1 || *Wo < 1) return DCN_E_ARG;
  return check_positions(d, d->kernel_size, d->stride, d->pad, d->dilation, *Ho, *Wo);
}

}  // namespace dcn

extern "C" int dcn_output_hw(const dcn_desc* desc, int64_t* out_h, int64_t* out_w) {
  if (out_h == nullptr || out_w == nullptr || !geometry_ok(desc)) return DCN_E_ARG;
  const int64_t ho = out_extent(desc->height, desc->kernel_size, desc->stride, desc->pad, desc->dilation);
  const int64_t wo = out_extent(desc->width, desc->kernel_size, desc->stride, desc->pad, desc->dilation);
  if (ho < 1 || wo < 1) return DCN_E_ARG;
  *out_h = ho;
  *out_w = wo;
  return DCN_OK;
}

extern "C" int dcn_workspace_bytes(const dcn_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return DCN_E_ARG;
  Plan p;
  const int rc = make_plan(desc, &p);
  if (rc != DCN_OK) return rc;
  *bytes = p.ws_bytes;
  return DCN_OK;
}

extern "C" const char* dcn_variant_name(const dcn_desc* desc) {
  Plan p;
  if (make_plan(desc, &p) != DCN_OK) return "invalid";
  return dcn::variant_info(p.variant).name;
}

extern "C" int dcn_plan_describe(const dcn_desc* desc, char* buf, size_t len) {
  if (buf == nullptr || len == 0) return DCN_E_ARG;
  Plan p;
  const int rc = make_plan(desc, &p);
  if (rc != DCN_OK) {
    buf[0] = '\0';
    return rc;
  }
  const dcn::VariantInfo& vi = dcn::variant_info(p.variant);
  if (is_box(p.variant)) {
    std::snprintf(buf, len,
                  "%s tile=%dx%d px (%d slots) x %d ch, tiles=%lld, box_px=%d, roles=%s, producer waves=%d, "
                  "offset groups=%lld, ws=%zu B",
                  vi.name, p.box.TH, p.box.TW, 16 * p.box.fn, 64 * p.box.fm,
                  static_cast<long long>(desc->batch) * p.box.tiles_per_img * (p.Mp / (64 * p.box.fm)),
                  p.box.box_px, p.box.split ? "split" : "paired", p.box.pw,
                  static_cast<long long>(offset_groups(desc)), p.ws_bytes);
  } else {
    std::snprintf(buf, len, "%s tile=%d px x %d ch, offset groups=%lld, ws=%zu B", vi.name, vi.nt, vi.mt,
                  static_cast<long long>(offset_groups(desc)), p.ws_bytes);
  }
  return DCN_OK;
}

// ---- the offset/mask branch: a regular convolution with 3*G*K*K outputs (bf16: the
// kernel of dcn_om.hip; fp32: the tile kernels at zero offsets with no mask), its
// epilogue splitting offsets and mask
namespace {

// arguments of the offset/mask convolution reading the staged copy at ws + p.ws_x and the
// repacked branch weight at wp_om
dcn::OmArgs om_args(const dcn_desc* od, const Plan& p, const void* ws, const void* bias_om, void* offset,
                    void* mask, int split, const void* wp_om = nullptr) {
  dcn::OmArgs a{};
  a.xs = static_cast<const unsigned char*>(ws) + p.ws_x;
  a.wp = wp_om != nullptr ? wp_om : static_cast<const unsigned char*>(ws) + p.ws_w;
  a.bias = bias_om;
  a.offset = offset;
  a.mask = mask;
  a.B = static_cast<int>(od->batch);
  a.H = static_cast<int>(od->height);
  a.W = static_cast<int>(od->width);
  a.Cp = static_cast<int>(p.Cp);
  a.M = static_cast<int>(od->out_channels);
  a.Mp = static_cast<int>(p.Mp);
  a.K = static_cast<int>(od->kernel_size);
  a.KK = a.K * a.K;
  a.stride = static_cast<int>(od->stride);
  a.pad = static_cast<int>(od->pad);
  a.dil = static_cast<int>(od->dilation);
  a.Ho = static_cast<int>(p.Ho);
  a.Wo = static_cast<int>(p.Wo);
  a.HoWo = a.Ho * a.Wo;
  a.N = a.B * a.HoWo;
  a.split = split;
  return a;
}

int om_plan(const dcn_desc* d, dcn_desc* od, Plan* p) {
  if (!geometry_ok(d)) return DCN_E_ARG;
  if (d->dtype != DCN_F32 && d->dtype != DCN_BF16) return DCN_E_UNSUPPORTED;
  *od = *d;
  od->out_channels = 3 * offset_groups(d) * d->kernel_size * d->kernel_size;
  od->offset_groups = 1;
  const int64_t Ho = out_extent(od->height, od->kernel_size, od->stride, od->pad, od->dilation);
  const int64_t Wo = out_extent(od->width, od->kernel_size, od->stride, od->pad, od->dilation);
  // bf16: the convolution kernel of dcn_om.hip (rows in 32-row tiles, the column
  // matrix read straight from the staged copy); fp32: the tile kernels
  (void)Ho;
  (void)Wo;
  if (d->dtype == DCN_BF16) return compute_plan(od, p, dcn::V_OM_BF16);
  const bool small = od->out_channels <= 64;
  const int variant = d->dtype == DCN_F32 ? (small ? dcn::V_TILE_F32_M64_N64 : dcn::V_TILE_F32_M128_N64)
                                          : (small ? dcn::V_TILE_BF16_M64_N64 : dcn::V_TILE_BF16_M128_N64);
  return compute_plan(od, p, variant);
}

}  // namespace

extern "C" int dcn_offset_mask_workspace_bytes(const dcn_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return DCN_E_ARG;
  dcn_desc od;
  Plan p;
  const int rc = om_plan(desc, &od, &p);
  if (rc != DCN_OK) return rc;
  *bytes = p.ws_bytes;
  return DCN_OK;
}

extern "C" int dcn_offset_mask(const dcn_desc* desc, const void* x, const void* weight_om, const void* bias_om,
                               void* offset, void* mask, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  dcn_desc od;
  Plan p;
  int rc = om_plan(desc, &od, &p);
  if (rc != DCN_OK) return rc;
  if (p.empty) return DCN_OK;
  if (x == nullptr || weight_om == nullptr || offset == nullptr || mask == nullptr) return DCN_E_ARG;
  rc = check_positions(&od, od.kernel_size, od.stride, od.pad, od.dilation, p.Ho, p.Wo);
  if (rc != DCN_OK) return rc;
  rc = check_workspace(p, workspace, workspace_bytes);
  if (rc != DCN_OK) return rc;
  const StageArgs s = stage_args(&od, p, x, weight_om, workspace);
  if (dcn::launch_stage(p.variant, s, stream) != hipSuccess) return DCN_E_HIP;
  const int split = static_cast<int>(2 * offset_groups(desc) * desc->kernel_size * desc->kernel_size);
  if (p.variant == dcn::V_OM_BF16) {
    const dcn::OmArgs oa = om_args(&od, p, workspace, bias_om, offset, mask, split);
    return dcn::launch_om(oa, stream) == hipSuccess ? DCN_OK : DCN_E_HIP;
  }
  FusedArgs a = fused_args(&od, p, x, nullptr, nullptr, weight_om, bias_om, offset, workspace);
  a.out2 = mask;
  a.om_split = split;
  return launch_fused_plan(p, a, stream) == hipSuccess ? DCN_OK : DCN_E_HIP;
}

extern "C" const char* dcn_status_str(int status) {
  switch (status) {
    case DCN_OK: return "ok";
    case DCN_E_ARG: return "invalid argument";
    case DCN_E_UNSUPPORTED: return "unsupported (dtype or size limit)";
    case DCN_E_WORKSPACE: return "workspace missing, too small or misaligned";
    case DCN_E_HIP: return "HIP kernel launch failed";
    case DCN_E_SCRATCH: return "the problem needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

namespace {

int validate_call(const dcn_desc* desc, Plan* p, const void* offset, const void* weight, const void* out,
                  const void* x) {
  const int rc = make_plan(desc, p);
  if (rc != DCN_OK) return rc;
  if (p->empty) return DCN_OK;
  if (x == nullptr || offset == nullptr || weight == nullptr || out == nullptr) return DCN_E_ARG;
  return check_positions(desc, desc->kernel_size, desc->stride, desc->pad, desc->dilation, p->Ho, p->Wo);
}

}  // namespace

extern "C" int dcn_stage(const dcn_desc* desc, const void* x, const void* weight, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  int rc = make_plan(desc, &p);
  if (rc != DCN_OK) return rc;
  if (p.empty || !dcn::variant_info(p.variant).staged) return DCN_OK;
  if (x == nullptr || weight == nullptr) return DCN_E_ARG;
  rc = check_workspace(p, workspace, workspace_bytes);
  if (rc != DCN_OK) return rc;
  const StageArgs a = stage_args(desc, p, x, weight, workspace);
  return dcn::launch_stage(p.variant, a, stream) == hipSuccess ? DCN_OK : DCN_E_HIP;
}

extern "C" int dcn_forward_staged(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                                  const void* weight, const void* bias, void* out, const void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  int rc = validate_call(desc, &p, offset, weight, out, x);
  if (rc != DCN_OK) return rc;
  if (p.empty) return DCN_OK;
  rc = check_workspace(p, workspace, workspace_bytes);
  if (rc != DCN_OK) return rc;
  const FusedArgs a = fused_args(desc, p, x, offset, mask, weight, bias, out, workspace);
  return launch_fused_plan(p, a, stream) == hipSuccess ? DCN_OK : DCN_E_HIP;
}

extern "C" int dcn_forward(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                           const void* weight, const void* bias, void* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  int rc = validate_call(desc, &p, offset, weight, out, x);
  if (rc != DCN_OK) return rc;
  if (p.empty) return DCN_OK;
  rc = check_workspace(p, workspace, workspace_bytes);
  if (rc != DCN_OK) return rc;
  if (dcn::variant_info(p.variant).staged) {
    const StageArgs s = stage_args(desc, p, x, weight, workspace);
    if (dcn::launch_stage(p.variant, s, stream) != hipSuccess) return DCN_E_HIP;
  }
  const FusedArgs a = fused_args(desc, p, x, offset, mask, weight, bias, out, workspace);
  return launch_fused_plan(p, a, stream) == hipSuccess ? DCN_OK : DCN_E_HIP;
}

// ---- dcn_forward without a caller workspace: a file-scope device array serves as the
// workspace.  In host code `scratch` names a host-side stand-in, never the device
// array: its device address is looked up once per device with hipGetSymbolAddress
// (that device current) and only that address is passed to kernels.
namespace {

__device__ __align__(256) unsigned char scratch[DCN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// the current device's address of `scratch`, looked up on the first call on that device
int current_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return DCN_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DCN_E_HIP;
    if (reinterpret_cast<uintptr_t>(p) % kAlign != 0) return DCN_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return DCN_OK;
}

}  // namespace

extern "C" int dcn_forward_noalloc(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                                   const void* weight, const void* bias, void* out, hipStream_t stream) {
  Plan p;
  int rc = validate_call(desc, &p, offset, weight, out, x);
  if (rc != DCN_OK) return rc;
  if (p.empty) return DCN_OK;
  if (p.ws_bytes > DCN_NOALLOC_SCRATCH_BYTES) return DCN_E_SCRATCH;
  void* ws = nullptr;
  if (p.ws_bytes > 0) {
    rc = current_scratch(&ws);
    if (rc != DCN_OK) return rc;
  }
  if (dcn::variant_info(p.variant).staged) {
    const StageArgs s = stage_args(desc, p, x, weight, ws);
    if (dcn::launch_stage(p.variant, s, stream) != hipSuccess) return DCN_E_HIP;
  }
  const FusedArgs a = fused_args(desc, p, x, offset, mask, weight, bias, out, ws);
  return launch_fused_plan(p, a, stream) == hipSuccess ? DCN_OK : DCN_E_HIP;
}

// ---- the DCNv2 layer in one call: the offset/mask branch and the deformable convolution
// off one staged copy of x (csdn.net tags page "可变形卷积：Deformable ConvNets", DCNv2
// section 3.2: the branch is a convolution of the same input feature map)
namespace {

struct LayerPlan {
  Plan fwd, om;
  dcn_desc od;          // the branch's convolution
  bool shared = false;  // one staging launch writes x once and both repacked weights
  size_t wp_om = 0;     // shared: byte offset of the branch's weight; else of its workspace part
  size_t fwd_base = 0;  // byte offset of the deformable layer's workspace part (not shared)
  size_t ws_bytes = 0;
  int split = 0;
};

int layer_plan(const dcn_desc* d, LayerPlan* lp) {
  int rc = make_plan(d, &lp->fwd);
  if (rc != DCN_OK) return rc;
  rc = om_plan(d, &lp->od, &lp->om);
  if (rc != DCN_OK) return rc;
  lp->split = static_cast<int>(2 * offset_groups(d) * d->kernel_size * d->kernel_size);
  const bool fs = dcn::variant_info(lp->fwd.variant).staged && !lp->fwd.empty;
  const bool os = dcn::variant_info(lp->om.variant).staged && !lp->om.empty;
  // the staged copies coincide when both paths stage x with the same channel padding
  lp->shared = fs && os && lp->fwd.Cp == lp->om.Cp && lp->fwd.ws_x == 0 && lp->om.ws_x == 0 &&
               lp->fwd.ws_w == lp->om.ws_w;
  if (lp->shared) {
    lp->wp_om = lp->fwd.ws_bytes;
    lp->ws_bytes = lp->fwd.ws_bytes + (lp->om.ws_bytes - lp->om.ws_w);
  } else {
    lp->wp_om = 0;
    lp->fwd_base = align_up(lp->om.ws_bytes, kAlign);
    lp->ws_bytes = lp->fwd_base + lp->fwd.ws_bytes;
  }
  return DCN_OK;
}

}  // namespace

extern "C" int dcn_layer_workspace_bytes(const dcn_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return DCN_E_ARG;
  LayerPlan lp;
  const int rc = layer_plan(desc, &lp);
  if (rc != DCN_OK) return rc;
  *bytes = lp.ws_bytes;
  return DCN_OK;
}

extern "C" int dcn_layer_forward(const dcn_desc* desc, const void* x, const void* weight_om, const void* bias_om,
                                 const void* weight, const void* bias, void* offset, void* mask, void* out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  LayerPlan lp;
  int rc = layer_plan(desc, &lp);
  if (rc != DCN_OK) return rc;
  if (lp.om.empty) return DCN_OK;   // B == 0
  if (x == nullptr || weight_om == nullptr || offset == nullptr || mask == nullptr) return DCN_E_ARG;
  if (!lp.fwd.empty && (weight == nullptr || out == nullptr)) return DCN_E_ARG;
  rc = check_positions(&lp.od, lp.od.kernel_size, lp.od.stride, lp.od.pad, lp.od.dilation, lp.om.Ho, lp.om.Wo);
  if (rc != DCN_OK) return rc;
  if (lp.ws_bytes > 0 &&
      (workspace == nullptr || workspace_bytes < lp.ws_bytes || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0))
    return DCN_E_WORKSPACE;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if (lp.shared) {
    // one launch: x staged once, the layer's weight and the branch's weight repacked
    StageArgs s = stage_args(desc, lp.fwd, x, weight, ws);
    s.w2 = weight_om;
    s.wp2 = ws + lp.wp_om;
    s.Cout2 = static_cast<int>(lp.od.out_channels);
    s.Mp2 = static_cast<int>(lp.om.Mp);
    s.wlayout2 = stage_args(&lp.od, lp.om, x, weight_om, ws).wlayout;
    if (dcn::launch_stage(lp.fwd.variant, s, stream) != hipSuccess) return DCN_E_HIP;
    if (lp.om.variant == dcn::V_OM_BF16) {
      const dcn::OmArgs oa = om_args(&lp.od, lp.om, ws, bias_om, offset, mask, lp.split, ws + lp.wp_om);
      if (dcn::launch_om(oa, stream) != hipSuccess) return DCN_E_HIP;
    } else {
      FusedArgs a = fused_args(&lp.od, lp.om, x, nullptr, nullptr, weight_om, bias_om, offset, ws);
      a.wp = ws + lp.wp_om;
      a.out2 = mask;
      a.om_split = lp.split;
      if (launch_fused_plan(lp.om, a, stream) != hipSuccess) return DCN_E_HIP;
    }
    const FusedArgs f = fused_args(desc, lp.fwd, x, offset, mask, weight, bias, out, ws);
    return launch_fused_plan(lp.fwd, f, stream) == hipSuccess ? DCN_OK : DCN_E_HIP;
  }
  // the two calls one after the other, each on its own part of the workspace
  rc = dcn_offset_mask(desc, x, weight_om, bias_om, offset, mask, lp.om.ws_bytes ? ws : nullptr, lp.om.ws_bytes,
                       stream);
  if (rc != DCN_OK || lp.fwd.empty) return rc;
  return dcn_forward(desc, x, offset, mask, weight, bias, out, lp.fwd.ws_bytes ? ws + lp.fwd_base : nullptr,
                     lp.fwd.ws_bytes, stream);
}
