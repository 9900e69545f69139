// dcn_direct.hip -- gfx950 kernel for deformable convolutions with a tiny reduction
// (at most 4 input channels, K*K in {1, 4, 9}), such as a first layer on RGB input.
//
// With Cin*K*K <= 36 the column of one output pixel fits in registers and the
// contraction is a handful of fused multiply-adds per output channel, so there is no
// staging copy, no LDS tile and no matrix-core work: the output write dominates the
// traffic.  A workgroup owns 64 output pixels (one per lane) and up to 64 output
// channels:
//   * each of its four waves samples a share of the kernel points: it reads the
//     offsets and the mask of its pixels (consecutive lanes, consecutive pixels),
//     forms the sampling position and the four bilinear weights times the mask (zero
//     for a neighbour outside the image), interpolates the Cin input channels from x
//     in its given [B][Cin][H][W] layout (x is small; its reads are cache hits; two
//     horizontal neighbours are one 8-byte load in fp32) and puts the column entries
//     in LDS;
//   * after a barrier every lane holds its pixel's whole column in registers and
//     each wave contracts it with a quarter of the output channels' weight rows (the
//     rows are staged in LDS at the start; every lane of a wave reads the same
//     address), adds the bias and stores; consecutive lanes store consecutive pixels.
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

// Raw buffer loads with 32-bit byte offsets (the host keeps every tensor the kernel
// reads under 2 GiB).  An offset past the end reads 0 without touching memory, which
// is how neighbours outside the image are read: no branch around the load.
constexpr uint32_t kOutside = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

template <bool BF16>
__device__ __forceinline__ float ldb(__amdgpu_buffer_rsrc_t r, uint32_t elem) {
  if constexpr (BF16) {
    const uint32_t v = __builtin_amdgcn_raw_buffer_load_b16(r, elem * 2u, 0, 0);
    return __uint_as_float(v << 16);
  } else {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, elem * 4u, 0, 0));
  }
}
// element index, or one that reads as zero
template <bool BF16>
__device__ __forceinline__ float ldb_if(__amdgpu_buffer_rsrc_t r, bool ok, uint32_t elem) {
  return ldb<BF16>(r, ok ? elem : kOutside / (BF16 ? 2u : 4u));
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

}  // namespace

// CINT: the number of input channels when known at compile time (then the column has
// exactly Cin*K*K entries), or 0 for any Cin <= 4 (column padded with zeros to 4*K*K).
template <bool BF16, int KKT, int CINT>
__global__ __launch_bounds__(256) void dcn_direct_kernel(FusedArgs a) {
  constexpr uint32_t ES = BF16 ? 2u : 4u;
  constexpr int CMAX = CINT > 0 ? CINT : kCinMax;
  constexpr int RMAX = CMAX * KKT;
  __shared__ float colbuf[RMAX][64];
  __shared__ __attribute__((aligned(16))) float wsm[64][RMAX];   // weight rows o0 .. o0+63 (zero past Cin*K*K)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int RK = a.Cin * KKT;
  const int o0 = blockIdx.y * 64, o1 = min(o0 + 64, a.Cout);
  const uint32_t HW = static_cast<uint32_t>(a.H) * static_cast<uint32_t>(a.W);
  const auto rx = rsrc(a.x, static_cast<uint32_t>(a.B) * a.Cin * HW * ES);
  const auto ro = rsrc(a.offset, static_cast<uint32_t>(a.B) * 2 * KKT * a.HoWo * ES);
  const auto rm = rsrc(a.mask ? a.mask : a.offset, static_cast<uint32_t>(a.B) * KKT * a.HoWo * ES);
  {
    // weight rows into LDS: all loads first, then the stores
    const auto rw = rsrc(a.w, static_cast<uint32_t>(a.Cout) * RK * ES);
    constexpr int NW = (64 * RMAX + 255) / 256;
    float wv[NW];
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int e = tid + t * 256;
      const int ol = e / RMAX, r = e - (e / RMAX) * RMAX;
      wv[t] = ldb_if<BF16>(rw, e < 64 * RMAX && o0 + ol < a.Cout && r < RK, static_cast<uint32_t>(o0 + ol) * RK + r);
    }
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int e = tid + t * 256;
      if (e < 64 * RMAX) wsm[e / RMAX][e - (e / RMAX) * RMAX] = wv[t];
    }
  }
  const int n = blockIdx.x * 64 + lane;
  const bool live = n < a.N;
  const int nn = live ? n : 0;
  const int b = nn / a.HoWo, rem = nn - (nn / a.HoWo) * a.HoWo;
  const int oy = rem / a.Wo, ox = rem - (rem / a.Wo) * a.Wo;

  // ---- column of the workgroup's 64 pixels: wave w samples kernel points k = w, w+4, ...
  // Offsets and mask first, then the positions, then every input load (no branches:
  // neighbours outside the image read as zero), then the interpolation.
  constexpr int KPW = (KKT + 3) / 4;   // kernel points per wave (at most)
  float dy[KPW], dx[KPW], mk[KPW];
#pragma unroll
  for (int t = 0; t < KPW; ++t) {
    const int k = min(wave + 4 * t, KKT - 1);
    const uint32_t ob = (static_cast<uint32_t>(b) * 2 * KKT + 2 * k) * a.HoWo + rem;
    dy[t] = ldb<BF16>(ro, ob);
    dx[t] = ldb<BF16>(ro, ob + a.HoWo);
    mk[t] = a.mask ? ldb<BF16>(rm, (static_cast<uint32_t>(b) * KKT + k) * a.HoWo + rem) : 1.f;
  }
  float xv[KPW][CMAX][4], wq[KPW][4];
#pragma unroll
  for (int t = 0; t < KPW; ++t) {
    const int k = min(wave + 4 * t, KKT - 1);
    const int i = k / a.K, j = k - (k / a.K) * a.K;
    // integer and fractional parts of the offset are exact in fp32
    const float fy = floorf(dy[t]), fx = floorf(dx[t]);
    const float ly = dy[t] - fy, lx = dx[t] - fx;
    const float y0 = static_cast<float>(oy * a.stride - a.pad + i * a.dil) + fy;
    const float x0 = static_cast<float>(ox * a.stride - a.pad + j * a.dil) + fx;
    // inside tests on floats first: NaN and huge values fail every test
    const bool vy0 = (y0 >= 0.f) && (y0 <= static_cast<float>(a.H - 1));
    const bool vy1 = (y0 >= -1.f) && (y0 <= static_cast<float>(a.H - 2));
    const bool vx0 = (x0 >= 0.f) && (x0 <= static_cast<float>(a.W - 1));
    const bool vx1 = (x0 >= -1.f) && (x0 <= static_cast<float>(a.W - 2));
    const bool any = (vy0 || vy1) && (vx0 || vx1);
    const int iy = any ? static_cast<int>(y0) : 0, ix = any ? static_cast<int>(x0) : 0;
    const float hy = 1.f - ly, hx = 1.f - lx, m = mk[t];
    const bool v00 = vy0 && vx0, v01 = vy0 && vx1, v10 = vy1 && vx0, v11 = vy1 && vx1;
    wq[t][0] = v00 ? hy * hx * m : 0.f;
    wq[t][1] = v01 ? hy * lx * m : 0.f;
    wq[t][2] = v10 ? ly * hx * m : 0.f;
    wq[t][3] = v11 ? ly * lx * m : 0.f;
    // (iy, ix) may be -1 for a lower neighbour outside; those corners are not read
    const uint32_t p00 = static_cast<uint32_t>(iy * a.W + ix);
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
      const bool on = c < a.Cin;
      const uint32_t base = (static_cast<uint32_t>(b) * a.Cin + c) * HW + p00;
      xv[t][c][0] = ldb_if<BF16>(rx, on && v00, base);
      xv[t][c][1] = ldb_if<BF16>(rx, on && v01, base + 1);
      xv[t][c][2] = ldb_if<BF16>(rx, on && v10, base + a.W);
      xv[t][c][3] = ldb_if<BF16>(rx, on && v11, base + a.W + 1);
    }
  }
#pragma unroll
  for (int t = 0; t < KPW; ++t) {
    const int k = wave + 4 * t;
    if (k >= KKT) continue;
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
      if (c >= a.Cin) continue;
      colbuf[c * KKT + k][lane] =
          wq[t][0] * xv[t][c][0] + wq[t][1] * xv[t][c][1] + wq[t][2] * xv[t][c][2] + wq[t][3] * xv[t][c][3];
    }
  }
  __syncthreads();

  // ---- contraction: every lane holds its pixel's column; wave w does output channels
  // o0 + 16w .. o0 + 16w + 15, four at a time (independent accumulators); the weight
  // rows come from LDS (every lane of the wave reads the same address)
  float col[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) col[r] = (r < RK) ? colbuf[r][lane] : 0.f;
  const int ob0 = o0 + 16 * wave, ob1 = min(ob0 + 16, o1);
  for (int o = ob0; o < ob1; o += 4) {
    float acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = (a.bias && o + u < ob1) ? ldb<BF16>(rsrc(a.bias, a.Cout * ES), o + u) : 0.f;
#pragma unroll
    for (int r = 0; r < RMAX; ++r)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = __builtin_fmaf(wsm[min(o + u - o0, 63)][r], col[r], acc[u]);
    if (live) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (o + u >= ob1) break;
        const int64_t e = (static_cast<int64_t>(b) * a.Cout + o + u) * a.HoWo + rem;
        if constexpr (BF16) reinterpret_cast<uint16_t*>(a.out)[e] = to_bf16(acc[u]);
        else reinterpret_cast<float*>(a.out)[e] = acc[u];
      }
    }
  }
}

bool direct_supported(int cin, int kk) { return cin >= 1 && cin <= kCinMax && (kk == 1 || kk == 4 || kk == 9); }

hipError_t launch_direct(bool bf16, const FusedArgs& a, hipStream_t stream) {
  // 64 pixels x 64 output channels per workgroup
  const dim3 grid((a.N + 63) / 64, (a.Cout + 63) / 64);
  FusedArgs fa = a;
  void* args[] = {&fa};
  const void* fn = nullptr;
#define DCN_DIRECT(B, KKv) \
  if (bf16 == B && a.KK == KKv) fn = reinterpret_cast<const void*>(&dcn_direct_kernel<B, KKv, 0>);
  DCN_DIRECT(false, 1) DCN_DIRECT(false, 4) DCN_DIRECT(false, 9)
  DCN_DIRECT(true, 1) DCN_DIRECT(true, 4) DCN_DIRECT(true, 9)
#undef DCN_DIRECT
  // three channels (RGB) with a 3x3 kernel: exact column length
  if (a.Cin == 3 && a.KK == 9)
    fn = bf16 ? reinterpret_cast<const void*>(&dcn_direct_kernel<true, 9, 3>)
              : reinterpret_cast<const void*>(&dcn_direct_kernel<false, 9, 3>);
  if (fn == nullptr) return hipErrorInvalidValue;
  return hipLaunchKernel(fn, grid, dim3(256), args, 0, stream);
}

}  // namespace dcn
