// dcn_direct.hip -- gfx950 kernel for deformable convolutions with a tiny reduction
// (at most 4 input channels, K*K in {1, 4, 9}), such as a first layer on RGB input.
//
// With Cin*K*K <= 36 the column of one output pixel fits in registers and the
// contraction is a handful of fused multiply-adds per output channel, so there is no
// staging copy, no LDS tile and no matrix-core work: the output write dominates the
// traffic.  One thread owns one output pixel and a group of output channels:
//   * for each kernel point it reads the offsets and the mask of its pixel
//     (consecutive lanes read consecutive pixels), forms the sampling position, the
//     four bilinear weights times the mask (zero for a neighbour outside the image),
//     and interpolates the Cin input channels from x in its given [B][Cin][H][W]
//     layout (x is small; its reads are cache hits);
//   * for each output channel of its group it contracts the register column with
//     the weight row (the same for the whole wave: scalar loads), adds the bias and
//     stores; consecutive lanes store consecutive pixels.
//
// The computation is the deformable-convolution equation (csdn.net tags page
// "可变形卷积：Deformable ConvNets", part "Deformable Convolutional Networks",
// section on deformable convolution) with the DCNv2 modulation scalar (same page,
// section 3.2) and bilinear interpolation from the four integer neighbours (same
// page, bilinear-interpolation equation); neighbours outside the image contribute 0.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcn_internal.h"

namespace dcn {
namespace {

constexpr int kCinMax = 4;

template <bool BF16>
__device__ __forceinline__ float ld(const void* p, int64_t idx) {
  if constexpr (BF16) {
    const uint16_t v = reinterpret_cast<const uint16_t*>(p)[idx];
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  } else {
    return reinterpret_cast<const float*>(p)[idx];
  }
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

}  // namespace

template <bool BF16, int KKT>
__global__ __launch_bounds__(64) void dcn_direct_kernel(FusedArgs a, int og) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  const bool live = n < a.N;
  const int nn = live ? n : 0;
  const int b = nn / a.HoWo, rem = nn - (nn / a.HoWo) * a.HoWo;
  const int oy = rem / a.Wo, ox = rem - (rem / a.Wo) * a.Wo;
  const int64_t plane = static_cast<int64_t>(a.H) * a.W;

  float col[kCinMax][KKT];
#pragma unroll
  for (int k = 0; k < KKT; ++k) {
    const int i = k / a.K, j = k - (k / a.K) * a.K;
    const int64_t ob = (static_cast<int64_t>(b) * 2 * KKT + 2 * k) * a.HoWo + rem;
    const float dy = ld<BF16>(a.offset, ob);
    const float dx = ld<BF16>(a.offset, ob + a.HoWo);
    const float m = a.mask ? ld<BF16>(a.mask, (static_cast<int64_t>(b) * KKT + k) * a.HoWo + rem) : 1.f;
    // integer and fractional parts of the offset are exact in fp32
    const float fy = floorf(dy), fx = floorf(dx);
    const float ly = dy - fy, lx = dx - fx;
    const float y0 = static_cast<float>(oy * a.stride - a.pad + i * a.dil) + fy;
    const float x0 = static_cast<float>(ox * a.stride - a.pad + j * a.dil) + fx;
    // inside tests on floats first: NaN and huge values fail every test
    const bool vy0 = (y0 >= 0.f) && (y0 <= static_cast<float>(a.H - 1));
    const bool vy1 = (y0 >= -1.f) && (y0 <= static_cast<float>(a.H - 2));
    const bool vx0 = (x0 >= 0.f) && (x0 <= static_cast<float>(a.W - 1));
    const bool vx1 = (x0 >= -1.f) && (x0 <= static_cast<float>(a.W - 2));
    const bool any = (vy0 || vy1) && (vx0 || vx1);
    const int iy = any ? static_cast<int>(y0) : 0, ix = any ? static_cast<int>(x0) : 0;
    const float hy = 1.f - ly, hx = 1.f - lx;
    const float w00 = (vy0 && vx0) ? hy * hx * m : 0.f, w01 = (vy0 && vx1) ? hy * lx * m : 0.f;
    const float w10 = (vy1 && vx0) ? ly * hx * m : 0.f, w11 = (vy1 && vx1) ? ly * lx * m : 0.f;
    const int64_t p00 = static_cast<int64_t>(iy) * a.W + ix;
#pragma unroll
    for (int c = 0; c < kCinMax; ++c) {
      float v = 0.f;
      if (c < a.Cin) {
        const int64_t base = (static_cast<int64_t>(b) * a.Cin + c) * plane + p00;
        if (vy0 && vx0) v += w00 * ld<BF16>(a.x, base);
        if (vy0 && vx1) v += w01 * ld<BF16>(a.x, base + 1);
        if (vy1 && vx0) v += w10 * ld<BF16>(a.x, base + a.W);
        if (vy1 && vx1) v += w11 * ld<BF16>(a.x, base + a.W + 1);
      }
      col[c][k] = v;
    }
  }

  const int o0 = blockIdx.y * og, o1 = min(o0 + og, a.Cout);
  const int RK = a.Cin * KKT;
  for (int o = o0; o < o1; ++o) {
    float acc = a.bias ? ld<BF16>(a.bias, o) : 0.f;
#pragma unroll
    for (int c = 0; c < kCinMax; ++c) {
      if (c < a.Cin) {
#pragma unroll
        for (int k = 0; k < KKT; ++k) acc = __builtin_fmaf(ld<BF16>(a.w, static_cast<int64_t>(o) * RK + c * KKT + k), col[c][k], acc);
      }
    }
    if (live) {
      const int64_t e = (static_cast<int64_t>(b) * a.Cout + o) * a.HoWo + rem;
      if constexpr (BF16) reinterpret_cast<uint16_t*>(a.out)[e] = to_bf16(acc);
      else reinterpret_cast<float*>(a.out)[e] = acc;
    }
  }
}

bool direct_supported(int cin, int kk) { return cin >= 1 && cin <= kCinMax && (kk == 1 || kk == 4 || kk == 9); }

hipError_t launch_direct(bool bf16, const FusedArgs& a, hipStream_t stream) {
  // output channels per thread: enough threads to fill the chip, at most 32 per thread
  const int pixel_blocks = (a.N + 63) / 64;
  int og = a.Cout;
  while (og > 8 && static_cast<int64_t>(pixel_blocks) * ((a.Cout + og - 1) / og) < 2048) og = (og + 1) / 2;
  og = og < 32 ? og : 32;
  og = og > 0 ? og : 1;
  const dim3 grid(pixel_blocks, (a.Cout + og - 1) / og);
  FusedArgs fa = a;
  void* args[] = {&fa, &og};
  const void* fn = nullptr;
#define DCN_DIRECT(B, KKv) \
  if (bf16 == B && a.KK == KKv) fn = reinterpret_cast<const void*>(&dcn_direct_kernel<B, KKv>);
  DCN_DIRECT(false, 1) DCN_DIRECT(false, 4) DCN_DIRECT(false, 9)
  DCN_DIRECT(true, 1) DCN_DIRECT(true, 4) DCN_DIRECT(true, 9)
#undef DCN_DIRECT
  if (fn == nullptr) return hipErrorInvalidValue;
  return hipLaunchKernel(fn, grid, dim3(64), args, 0, stream);
}

}  // namespace dcn
