// dcn_om.hip -- gfx950 kernel of the DCNv2 offset/mask branch: the regular convolution
// of the layer's input with 3*G*K*K outputs, whose first 2*G*K*K channels are the
// offsets and the rest, through a sigmoid, the modulation scalars (csdn.net tags page
// "可变形卷积：Deformable ConvNets", DCNv2 section 3.2).
//
// The input is the staged channels-last copy [B][H][W][Cp] that the deformable layer
// reads as well.  At zero offsets a column entry is one input value at an integer
// position, so the column matrix is read straight from that copy: the 16-channel k-step
// of one tap is one 16-byte vector per lane (channels 0-7 in lanes 0-31, 8-15 in lanes
// 32-63), exactly the B operand of MFMA 32x32x16 bf16, and taps in the padding read
// past the end of a raw buffer resource, which returns zeros.  The weight, repacked
// to [tap * Cp/16 + channel step][Mp][16], is the A operand the same way.
//
// A workgroup computes 32 output rows (the 27 of a 3x3 branch, padded) for 32 output
// pixels.  Its sixteen waves split the K*K*Cp reduction into contiguous ranges (nine
// k-steps each for the c4 layer: every load of a wave in flight at once), each
// accumulates one 32x32 fp32 block, and the partial blocks are summed through LDS in
// a fixed order (deterministic); the epilogue adds the bias, applies the sigmoid to the
// mask rows, rounds to bf16 (nearest even) and stores both outputs in NCHW.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "dcn_internal.h"

namespace dcn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kOmWaves = 16;
constexpr int kOmThreads = 64 * kOmWaves;
constexpr int kOmPx = 32;                  // output pixels per workgroup
constexpr int kOmUnroll = 9;               // k-steps whose loads are issued together
constexpr uint32_t kOmOOB = 0xfffffff0u;   // a byte offset past every buffer here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t om_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

// Workgroup g runs on XCD g mod 8: give each XCD a contiguous run of the T tiles, so
// neighbouring pixel tiles (which read overlapping input rows) share that XCD's L2.
__device__ __forceinline__ int om_xcd_tile(int g, int T) {
  const int xcd = g & 7, idx = g >> 3;
  const int q = T >> 3, r = T & 7;
  return xcd * q + min(xcd, r) + idx;
}

__global__ __launch_bounds__(kOmThreads) void om_conv_kernel(OmArgs a) {
  __shared__ float red[kOmWaves][32][33];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const int m_tiles = a.Mp >> 5;
  const int t = om_xcd_tile(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int mt = t % m_tiles, nt = t / m_tiles;
  const int m0 = mt * 32;
  // the lane's output pixel (B-operand column l32)
  const int n = nt * kOmPx + l32;
  const bool nvalid = n < a.N;
  const int nn = nvalid ? n : 0;
  const int b = nn / a.HoWo, p = nn - b * a.HoWo;
  const int oy = p / a.Wo, ox = p - (p / a.Wo) * a.Wo;
  const int csteps = a.Cp >> 4;        // 16-channel k-steps per tap
  const int S = a.KK * csteps;          // k-steps in all
  const int s0 = (S * wave) / kOmWaves, s1 = (S * (wave + 1)) / kOmWaves;
  const uint32_t xs_bytes = static_cast<uint32_t>(a.B * a.H) * static_cast<uint32_t>(a.W * a.Cp) * 2u;
  const __amdgpu_buffer_rsrc_t rsrc = om_rsrc(a.xs, xs_bytes);
  const uint32_t img = static_cast<uint32_t>(b * a.H) * static_cast<uint32_t>(a.W * a.Cp) * 2u +
                       static_cast<uint32_t>(lh * 16);
  const unsigned char* wp = static_cast<const unsigned char*>(a.wp) +
                            (static_cast<size_t>(m0 + l32) * 16 + 8 * lh) * 2;
  const size_t wstep = static_cast<size_t>(a.Mp) * 32;   // bytes per k-step of the weight

  // The k-step walks (tap, 16-channel step) in order: the pixel's byte offset for the
  // current tap (past the end of the buffer when the tap falls outside the image) is
  // recomputed only when the tap changes.
  int tap = s0 / csteps, c16 = s0 - (s0 / csteps) * csteps;
  auto tap_off = [&](int t) __attribute__((always_inline)) -> uint32_t {
    const int i = t / a.K, j = t - (t / a.K) * a.K;
    const int iy = oy * a.stride - a.pad + i * a.dil, ix = ox * a.stride - a.pad + j * a.dil;
    const bool in = nvalid && t < a.KK && iy >= 0 && iy < a.H && ix >= 0 && ix < a.W;
    return in ? img + static_cast<uint32_t>(iy * a.W + ix) * static_cast<uint32_t>(a.Cp) * 2u : kOmOOB;
  };
  uint32_t poff = tap_off(tap);

  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int s = s0; s < s1; s += kOmUnroll) {
    uint4 av[kOmUnroll];
    u32x4 bv[kOmUnroll];
    // every load of the group first (steps past the range load a valid step and are
    // not multiplied)
#pragma unroll
    for (int u = 0; u < kOmUnroll; ++u) {
      const int su = min(s + u, s1 - 1);
      const uint32_t voff = poff == kOmOOB ? kOmOOB : poff + static_cast<uint32_t>(c16 * 32);
      bv[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, 0, 0);
      av[u] = *reinterpret_cast<const uint4*>(wp + static_cast<size_t>(su) * wstep);
      if (s + u + 1 < s1 && ++c16 == csteps) {
        c16 = 0;
        poff = tap_off(++tap);
      }
    }
#pragma unroll
    for (int u = 0; u < kOmUnroll; ++u) {
      if (s + u < s1)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                      __builtin_bit_cast(bf16x8, bv[u]), acc, 0, 0, 0);
    }
  }
  // partial blocks to LDS: accumulator element r is row 8*(r/4) + 4*lh + r%4, column l32
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wave][8 * (r >> 2) + 4 * lh + (r & 3)][l32] = acc[r];
  __syncthreads();
  uint16_t* off_out = static_cast<uint16_t*>(a.offset);
  uint16_t* msk_out = static_cast<uint16_t*>(a.mask);
  for (int e = tid; e < 32 * kOmPx; e += kOmThreads) {
    const int row = e / kOmPx, col = e - (e / kOmPx) * kOmPx;
    const int o = m0 + row, nc = nt * kOmPx + col;
    if (o >= a.M || nc >= a.N) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kOmWaves; ++w) v += red[w][row][col];
    if (a.bias != nullptr)
      v += __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.bias)[o]) << 16);
    const int bc = nc / a.HoWo, pc = nc - (nc / a.HoWo) * a.HoWo;
    if (o < a.split) {
      off_out[(static_cast<size_t>(bc) * a.split + o) * a.HoWo + pc] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    } else {
      const float sg = 1.f / (1.f + expf(-v));
      msk_out[(static_cast<size_t>(bc) * (a.M - a.split) + (o - a.split)) * a.HoWo + pc] =
          __builtin_bit_cast(uint16_t, static_cast<__bf16>(sg));
    }
  }
}

}  // namespace

hipError_t launch_om(const OmArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<OmArgs*>(&a)};
  const unsigned grid = static_cast<unsigned>((a.Mp / 32) * ((a.N + kOmPx - 1) / kOmPx));
  return hipLaunchKernel(reinterpret_cast<const void*>(&om_conv_kernel), dim3(grid), dim3(kOmThreads), args, 0,
                         stream);
}

}  // namespace dcn
