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
// Two kernels compute 32 output rows (the 27 of a 3x3 branch, padded) for 32 output
// pixels per workgroup:
//  * om_box_kernel (used whenever its box fits): the 32 pixels are a TH x TW block of
//    one image, and the rectangle of input pixels their taps read (the "box") is
//    copied, a chunk of channels at a time, from the staged copy into LDS with whole
//    16-byte vectors per pixel, so each input vector crosses the memory pipe once per
//    workgroup; the B operands are then LDS reads.  Box pixels are padded by 16 bytes
//    so the 32 lanes of a read spread over the banks.  Its eight waves take every
//    eighth k-step of a chunk;
//  * om_conv_kernel (any shape): the B operand is read straight from the staged copy
//    (one 16-byte vector per lane and k-step); sixteen waves split the reduction into
//    contiguous ranges.
// Each wave accumulates one 32x32 fp32 block, and the partial blocks are summed
// through LDS in a fixed order (deterministic); the epilogue adds the bias, applies
// the sigmoid to the mask rows, rounds to bf16 (nearest even) and stores both outputs
// in NCHW.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
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


// ---------------------------------------------------------------------------------
// om_box_kernel: one workgroup per (32-row block, TH x TW pixel block); see the top.
struct OmBoxArgs {
  OmArgs a;
  int TH, TW;            // output pixel block (TH * TW = 32) of one image
  int tiles_x;           // blocks per row of blocks
  int tiles_per_img;
  int BH, BW;            // box: the input rows and columns the block's taps read
  int CC;                // channels per box chunk (a power of two >= 16 that divides Cp)
  int cc_sh;             // log2(CC)
};
constexpr int kObMaxTaps = 64;   // K*K of the box kernel at most (its tap table)

constexpr int kObWaves = 8;
constexpr int kObThreads = 64 * kObWaves;
constexpr int kObUnits = 8;     // 16-byte box vectors per thread and chunk (at most)
constexpr int kObUnroll = 9;    // k-steps whose loads are issued together

__global__ __launch_bounds__(kObThreads) void om_box_kernel(OmBoxArgs ob) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  __shared__ int tapoff[kObMaxTaps];   // box-pixel offset of each tap from tap (0, 0)
  const OmArgs& a = ob.a;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const int m_tiles = a.Mp >> 5;
  const int t = om_xcd_tile(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int mt = t % m_tiles, pt = t / m_tiles;
  const int b = pt / ob.tiles_per_img, rt = pt - (pt / ob.tiles_per_img) * ob.tiles_per_img;
  const int ty = rt / ob.tiles_x, tx = rt - (rt / ob.tiles_x) * ob.tiles_x;
  const int oy0 = ty * ob.TH, ox0 = tx * ob.TW;
  const int m0 = mt * 32;
  const int iy0 = oy0 * a.stride - a.pad, ix0 = ox0 * a.stride - a.pad;
  const int CC = ob.CC, PXS = 2 * CC + 16, BW = ob.BW, BP = ob.BH * ob.BW;
  const int cu_sh = ob.cc_sh - 3;          // log2 of the 16-byte vectors per box pixel
  if (tid < a.KK) tapoff[tid] = (tid / a.K) * a.dil * BW + (tid - (tid / a.K) * a.K) * a.dil;
  // The thread's box vectors: vector cu of pixels p0, p0 + ps, p0 + 2 ps, ...  (the
  // vectors per pixel divide the thread count), their rows and columns kept
  // incrementally so the copy has no divisions.
  const int cu = tid & ((1 << cu_sh) - 1), p0 = tid >> cu_sh, ps = kObThreads >> cu_sh;
  const int ps_r = ps / BW, ps_c = ps - (ps / BW) * BW;
  const int by0 = p0 / BW, bx0 = p0 - (p0 / BW) * BW;
  // the lane's output pixel (B-operand column l32) and its box position at tap (0, 0)
  const int py = l32 / ob.TW, px = l32 - (l32 / ob.TW) * ob.TW;
  const int bp0 = py * a.stride * BW + px * a.stride;
  const int cs_sh = ob.cc_sh - 4;          // log2 of the 16-channel k-steps per tap and chunk
  const int nsteps = a.KK << cs_sh;        // k-steps per chunk
  const int nchunks = a.Cp / CC;
  const int cps = a.Cp >> 4;               // k-steps per tap in the weight layout
  const unsigned char* xs = static_cast<const unsigned char*>(a.xs) +
                            static_cast<size_t>(b) * a.H * a.W * a.Cp * 2;
  const unsigned char* wp = static_cast<const unsigned char*>(a.wp) +
                            (static_cast<size_t>(m0 + l32) * 16 + 8 * lh) * 2;
  const size_t wstep = static_cast<size_t>(a.Mp) * 32;   // bytes per k-step of the weight

  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int ch = 0; ch < nchunks; ++ch) {
    const int c0 = ch * CC;
    // the chunk's box: every load first (pixels outside the image are zero), then,
    // once the previous chunk's reads are done, the LDS stores
    uint4 v[kObUnits];
    {
      int by = by0, bx = bx0;
#pragma unroll
      for (int j = 0; j < kObUnits; ++j) {
        const int p = p0 + j * ps;
        v[j] = make_uint4(0u, 0u, 0u, 0u);
        const int iy = iy0 + by, ix = ix0 + bx;
        if (p < BP && iy >= 0 && iy < a.H && ix >= 0 && ix < a.W)
          v[j] = *reinterpret_cast<const uint4*>(xs + (static_cast<size_t>(iy * a.W + ix) * a.Cp + c0 + cu * 8) * 2);
        by += ps_r;
        bx += ps_c;
        if (bx >= BW) {
          bx -= BW;
          ++by;
        }
      }
    }
    if (ch > 0) __syncthreads();
#pragma unroll
    for (int j = 0; j < kObUnits; ++j) {
      const int p = p0 + j * ps;
      if (p < BP) *reinterpret_cast<uint4*>(lds + p * PXS + cu * 16) = v[j];
    }
    __syncthreads();
    // this wave's k-steps s = wave, wave + 8, ...: kObUnroll at a time, every load of
    // the group first (past the chunk's last step a valid step is re-read and not
    // multiplied)
    for (int s = wave; s < nsteps; s += kObWaves * kObUnroll) {
      uint4 av[kObUnroll], bv[kObUnroll];
#pragma unroll
      for (int u = 0; u < kObUnroll; ++u) {
        const int su = min(s + u * kObWaves, nsteps - 1);
        const int tap = su >> cs_sh, c16 = su & ((1 << cs_sh) - 1);
        bv[u] = *reinterpret_cast<const uint4*>(lds + (bp0 + tapoff[tap]) * PXS + c16 * 32 + lh * 16);
        av[u] = *reinterpret_cast<const uint4*>(wp + static_cast<size_t>(tap * cps + (c0 >> 4) + c16) * wstep);
      }
#pragma unroll
      for (int u = 0; u < kObUnroll; ++u) {
        if (s + u * kObWaves < nsteps)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                        __builtin_bit_cast(bf16x8, bv[u]), acc, 0, 0, 0);
      }
    }
  }
  // partial blocks to LDS (over the box, once every wave is done reading it):
  // accumulator element r is row 8*(r/4) + 4*lh + r%4, column l32
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);   // [wave][32][33]
#pragma unroll
  for (int r = 0; r < 16; ++r) red[(wave * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)) * 33 + l32] = acc[r];
  __syncthreads();
  uint16_t* off_out = static_cast<uint16_t*>(a.offset);
  uint16_t* msk_out = static_cast<uint16_t*>(a.mask);
  for (int e = tid; e < 32 * 32; e += kObThreads) {
    const int row = e >> 5, col = e & 31;
    const int o = m0 + row;
    const int qy = col / ob.TW, qx = col - (col / ob.TW) * ob.TW;
    const int oy = oy0 + qy, ox = ox0 + qx;
    if (o >= a.M || oy >= a.Ho || ox >= a.Wo) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kObWaves; ++w) v += red[(w * 32 + row) * 33 + col];
    if (a.bias != nullptr)
      v += __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.bias)[o]) << 16);
    const int pc = oy * a.Wo + ox;
    if (o < a.split) {
      off_out[(static_cast<size_t>(b) * a.split + o) * a.HoWo + pc] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
    } else {
      const float sg = 1.f / (1.f + expf(-v));
      msk_out[(static_cast<size_t>(b) * (a.M - a.split) + (o - a.split)) * a.HoWo + pc] =
          __builtin_bit_cast(uint16_t, static_cast<__bf16>(sg));
    }
  }
}

// The box kernel's tile and channel chunk for a problem: the TH x TW block of 32
// pixels (1 x 32 to 32 x 1) and the largest chunk of channels (a power of two from 16
// to 256 that divides Cp) whose box fits in kObBoxBudget bytes of LDS, choosing the tile
// with the fewest box pixels loaded in all.  False when no chunk fits.
constexpr int kObBoxBudget = 64 * 1024;
bool om_box_plan(const OmArgs& a, OmBoxArgs& ob) {
  if (a.KK > kObMaxTaps) return false;
  long long best = -1;
  for (int th = 1; th <= 32; th *= 2) {
    const int tw = 32 / th;
    const int bh = (th - 1) * a.stride + (a.K - 1) * a.dil + 1, bw = (tw - 1) * a.stride + (a.K - 1) * a.dil + 1;
    int cc = 0;
    for (int c = 256; c >= 16; c /= 2)
      if (a.Cp % c == 0 && static_cast<long long>(bh) * bw * (2 * c + 16) <= kObBoxBudget &&
          static_cast<long long>(bh) * bw * (c / 8) <= static_cast<long long>(kObUnits) * kObThreads) {
        cc = c;
        break;
      }
    if (cc == 0) continue;
    const long long tiles = static_cast<long long>((a.Ho + th - 1) / th) * ((a.Wo + tw - 1) / tw);
    const long long cost = tiles * bh * bw;
    if (best < 0 || cost < best) {
      best = cost;
      ob.TH = th;
      ob.TW = tw;
      ob.BH = bh;
      ob.BW = bw;
      ob.CC = cc;
      ob.cc_sh = __builtin_ctz(static_cast<unsigned>(cc));
      ob.tiles_x = (a.Wo + tw - 1) / tw;
      ob.tiles_per_img = static_cast<int>(tiles);
    }
  }
  return best >= 0;
}

}  // namespace

hipError_t launch_om(const OmArgs& a, hipStream_t stream) {
  OmBoxArgs ob;
  ob.a = a;
  if (om_box_plan(a, ob)) {
    void* args[] = {&ob};
    const size_t lds = std::max<size_t>(static_cast<size_t>(ob.BH) * ob.BW * (2 * ob.CC + 16),
                                        static_cast<size_t>(kObWaves) * 32 * 33 * 4);
    const unsigned grid = static_cast<unsigned>((a.Mp / 32) * ob.tiles_per_img * a.B);
    return hipLaunchKernel(reinterpret_cast<const void*>(&om_box_kernel), dim3(grid), dim3(kObThreads), args, lds,
                           stream);
  }
  void* args[] = {const_cast<OmArgs*>(&a)};
  const unsigned grid = static_cast<unsigned>((a.Mp / 32) * ((a.N + kOmPx - 1) / kOmPx));
  return hipLaunchKernel(reinterpret_cast<const void*>(&om_conv_kernel), dim3(grid), dim3(kOmThreads), args, 0,
                         stream);
}

}  // namespace dcn
