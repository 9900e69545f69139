// dcn_roi.hip -- gfx950 deformable RoI pooling.
//
// The RoI is split into k x k bins; bin (i, j) is shifted by its own offset, which is
// normalised by the RoI's size (scaled by gamma times the RoI's height for rows and
// width for columns), and pooled by averaging S x S bilinear samples taken at the
// centres of equal sub-cells; the DCNv2 form multiplies the average by the bin's
// modulation scalar (the csdn.net tags page "可变形卷积：Deformable ConvNets", part (i)
// section 4 and the DCNv2 section 3.2, and part "Deformable Convolutional Networks",
// section Deformable RoI Pooling; 51itzy.com/kjqy/64159.html, section 二).  A
// neighbour outside the image contributes zero, as in the convolution.
//
// One thread per output element (RoI, channel, bin row, bin column), bin columns
// fastest: a wave covers whole bins of a few channels of one RoI, and neighbouring
// lanes sample neighbouring positions of one channel plane.  The RoI's geometry and
// the bin's offset and mask are read once per thread; the S x S samples are gathered
// from the NCHW input (the pooling reads each sample's four corners once, so a staged
// copy would cost more bytes than it saves).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "dcn.h"
#include "dcn_internal.h"

namespace dcn {
namespace {

constexpr int kRT = 256;

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, size_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
template <typename T>
__device__ __forceinline__ T st(float v);
template <>
__device__ __forceinline__ float st<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t st<uint16_t>(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }

// One bilinear sample of bin (i, j), sub-cell (u, v): its position in P, its top-left
// neighbour and the four neighbour weights in fp32.  The position follows the
// definition: y1 + (i + (u + 1/2) / S) * h / k + dy, likewise for columns (with 1/S and
// h/k formed once per RoI).  The fp32 kernel takes P = double, so the RoI arithmetic rounds nothing that
// a 1e-4 relative bound would see near the image border; for bf16 results fp32
// positions (relative error about 1e-6 of the coordinates) are far inside the bound.
template <typename P>
struct RoiGeom {
  P y1, x1, h, w, dy, dx;
  P bh, bw, inv_s;   // h / k, w / k, 1 / S
};
struct RoiSample {
  bool any;        // at least one neighbour inside the image
  int y0, x0;
  float w00, w01, w10, w11;
};
template <typename P>
__device__ __forceinline__ RoiSample roi_sample(const RoiGeom<P>& g, int i, int j, int u, int v, int H, int W) {
  const P half = static_cast<P>(0.5);
  const P py = g.y1 + (static_cast<P>(i) + (static_cast<P>(u) + half) * g.inv_s) * g.bh + g.dy;
  const P px = g.x1 + (static_cast<P>(j) + (static_cast<P>(v) + half) * g.inv_s) * g.bw + g.dx;
  RoiSample r;
  // no neighbour inside (or NaN): nothing to add
  r.any = py > static_cast<P>(-1) && py < static_cast<P>(H) && px > static_cast<P>(-1) && px < static_cast<P>(W);
  if (!r.any) return r;
  const P y0f = floor(py), x0f = floor(px);
  const float ly = static_cast<float>(py - y0f), lx = static_cast<float>(px - x0f);
  r.y0 = static_cast<int>(y0f);
  r.x0 = static_cast<int>(x0f);
  r.w00 = (1.f - ly) * (1.f - lx);
  r.w01 = (1.f - ly) * lx;
  r.w10 = ly * (1.f - lx);
  r.w11 = ly * lx;
  return r;
}

struct RoiArgs {
  const void* x;        // [B][C][H][W]; position-sensitive: [B][C*k*k][H][W]
  const float* rois;    // [R][5]: batch index, x1, y1, x2, y2
  const void* offset;   // [R][2G][k][k] or null
  const void* mask;     // [R][k][k] or null
  void* out;            // [R][C][k][k]
  int B, C, H, W, R, k, S;
  float scale, gamma;
  int ps;               // 1: bin (i, j) of output channel c pools score map (c*k + i)*k + j
  int G;                // offset groups of output channels (1 for plain pooling)
};

template <typename T>
__global__ __launch_bounds__(kRT) void roi_pool_kernel(RoiArgs a) {
  const long long e = static_cast<long long>(blockIdx.x) * kRT + threadIdx.x;
  const long long n = static_cast<long long>(a.R) * a.C * a.k * a.k;
  if (e >= n) return;
  const int kk = a.k * a.k;
  const int j = static_cast<int>(e % a.k), i = static_cast<int>((e / a.k) % a.k);
  const long long rc = e / kk;
  const int c = static_cast<int>(rc % a.C), r = static_cast<int>(rc / a.C);
  // the plane this output pools: channel c, or (position-sensitive) the bin's own score map
  const int cin = a.ps ? (c * a.k + i) * a.k + j : c;
  const int nin = a.ps ? a.C * a.k * a.k : a.C;
  const int g = c / (a.C / a.G);   // offset group
  const float* roi = a.rois + static_cast<size_t>(r) * 5;
  const float bi = roi[0];
  T* out = static_cast<T*>(a.out);
  if (!(bi >= 0.f && bi < static_cast<float>(a.B))) {   // no such image (or NaN): zeros
    out[e] = st<T>(0.f);
    return;
  }
  const int b = static_cast<int>(bi);
  using P = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
  RoiGeom<P> geo;
  geo.x1 = static_cast<P>(roi[1]) * a.scale;
  geo.y1 = static_cast<P>(roi[2]) * a.scale;
  geo.w = (static_cast<P>(roi[3]) - roi[1]) * a.scale;
  geo.h = (static_cast<P>(roi[4]) - roi[2]) * a.scale;
  geo.bh = geo.h / static_cast<P>(a.k);
  geo.bw = geo.w / static_cast<P>(a.k);
  geo.inv_s = static_cast<P>(1) / static_cast<P>(a.S);
  geo.dy = geo.dx = 0;
  float m = 1.f;
  if (a.offset != nullptr) {
    const T* off = static_cast<const T*>(a.offset);
    geo.dy = a.gamma * geo.h * ld(off, ((static_cast<size_t>(r) * 2 * a.G + 2 * g) * a.k + i) * a.k + j);
    geo.dx = a.gamma * geo.w * ld(off, ((static_cast<size_t>(r) * 2 * a.G + 2 * g + 1) * a.k + i) * a.k + j);
  }
  if (a.mask != nullptr) m = ld(static_cast<const T*>(a.mask), (static_cast<size_t>(r) * a.k + i) * a.k + j);
  const T* plane = static_cast<const T*>(a.x) + (static_cast<size_t>(b) * nin + cin) * a.H * a.W;
  const float inv = 1.f / static_cast<float>(a.S);
  float acc = 0.f;
  for (int u = 0; u < a.S; ++u) {
    for (int v = 0; v < a.S; ++v) {
      const RoiSample sp = roi_sample(geo, i, j, u, v, a.H, a.W);
      if (!sp.any) continue;
      const int y0 = sp.y0, x0 = sp.x0;
      const bool iy0 = y0 >= 0, iy1 = y0 + 1 < a.H, ix0 = x0 >= 0, ix1 = x0 + 1 < a.W;
      const int q = y0 * a.W + x0;
      const float v00 = (iy0 && ix0) ? ld(plane, q) : 0.f;
      const float v01 = (iy0 && ix1) ? ld(plane, q + 1) : 0.f;
      const float v10 = (iy1 && ix0) ? ld(plane, q + a.W) : 0.f;
      const float v11 = (iy1 && ix1) ? ld(plane, q + a.W + 1) : 0.f;
      acc += sp.w00 * v00 + sp.w01 * v01 + sp.w10 * v10 + sp.w11 * v11;
    }
  }
  out[e] = st<T>(m * acc * inv * inv);
}

// bf16 with a channels-last copy of the input: one workgroup per (RoI, block of 64
// channels).  A unit of work is (bin, 8 channels): eight neighbouring lanes take the
// eight 8-channel groups of one bin, so each corner is one 128-byte read of 64 channels
// of one pixel.  The k*k x 64 results go through LDS, channel-major, and are stored as
// one contiguous run of out[r][c0 .. c0+63][k][k].
// Plain pooling: xs [B][H][W][Cp] (px_stride = Cp, bin_stride = 0).  Position-sensitive
// pooling: xs [B][H][W][k*k][Cp] (px_stride = k*k*Cp, bin_stride = Cp), bin (i, j)'s
// score maps of every output channel contiguous, with one offset group or (C/G) % 8 == 0
// so that each 8-channel group lies in one offset group.
__global__ __launch_bounds__(kRT) void roi_pool_cl_kernel(RoiArgs a, const uint16_t* xs, int px_stride,
                                                          int bin_stride) {
  extern __shared__ uint16_t tile[];   // [64 channels][bin], stride k*k + 1
  const int ncb = (a.C + 63) / 64;
  const int r = blockIdx.x / ncb, c0 = (blockIdx.x - r * ncb) * 64;
  const int kk = a.k * a.k, ts = kk + 1;
  const float* roi = a.rois + static_cast<size_t>(r) * 5;
  const float bi = roi[0];
  const bool batch_ok = bi >= 0.f && bi < static_cast<float>(a.B);
  const int b = batch_ok ? static_cast<int>(bi) : 0;
  RoiGeom<float> geo;
  geo.x1 = roi[1] * a.scale;
  geo.y1 = roi[2] * a.scale;
  geo.w = (roi[3] - roi[1]) * a.scale;
  geo.h = (roi[4] - roi[2]) * a.scale;
  geo.bh = geo.h / static_cast<float>(a.k);
  geo.bw = geo.w / static_cast<float>(a.k);
  geo.inv_s = 1.f / static_cast<float>(a.S);
  const float inv = 1.f / static_cast<float>(a.S);
  const uint16_t* img = xs + static_cast<size_t>(b) * a.H * a.W * px_stride;
  for (int u = threadIdx.x; u < kk * 8; u += blockDim.x) {
    const int bin = u >> 3, gq = u & 7, c = c0 + 8 * gq;
    const int i = bin / a.k, j = bin - (bin / a.k) * a.k;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    float m = 0.f;
    if (batch_ok && c < a.C) {
      RoiGeom<float> g = geo;
      g.dy = g.dx = 0.f;
      m = 1.f;
      if (a.offset != nullptr) {
        const uint16_t* off = static_cast<const uint16_t*>(a.offset);
        const int og = c / (a.C / a.G);   // offset group of the 8 channels
        g.dy = a.gamma * g.h * ld(off, ((static_cast<size_t>(r) * 2 * a.G + 2 * og) * a.k + i) * a.k + j);
        g.dx = a.gamma * g.w * ld(off, ((static_cast<size_t>(r) * 2 * a.G + 2 * og + 1) * a.k + i) * a.k + j);
      }
      if (a.mask != nullptr) m = ld(static_cast<const uint16_t*>(a.mask), (static_cast<size_t>(r) * a.k + i) * a.k + j);
      for (int su = 0; su < a.S; ++su) {
        for (int sv = 0; sv < a.S; ++sv) {
          const RoiSample sp = roi_sample(g, i, j, su, sv, a.H, a.W);
          if (!sp.any) continue;
          const int y0 = sp.y0, x0 = sp.x0;
          const bool iy0 = y0 >= 0, iy1 = y0 + 1 < a.H, ix0 = x0 >= 0, ix1 = x0 + 1 < a.W;
          const float wt[4] = {sp.w00, sp.w01, sp.w10, sp.w11};
          const bool in[4] = {iy0 && ix0, iy0 && ix1, iy1 && ix0, iy1 && ix1};
          // the four corner loads together, from valid addresses (a corner outside the
          // image reads pixel 0 and is replaced by zeros)
          uint4 cv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int yy = in[q] ? y0 + (q >> 1) : 0, xc = in[q] ? x0 + (q & 1) : 0;
            cv[q] = *reinterpret_cast<const uint4*>(img + (static_cast<size_t>(yy) * a.W + xc) * px_stride +
                                                    bin * bin_stride + c);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 v = in[q] ? cv[q] : make_uint4(0, 0, 0, 0);
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[2 * e] += wt[q] * __uint_as_float(d[e] << 16);
              acc[2 * e + 1] += wt[q] * __uint_as_float(d[e] & 0xffff0000u);
            }
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[(8 * gq + e) * ts + bin] = st<uint16_t>(m * acc[e] * inv * inv);
  }
  __syncthreads();
  const int nch = min(64, a.C - c0);
  uint16_t* out = static_cast<uint16_t*>(a.out) + (static_cast<size_t>(r) * a.C + c0) * kk;
  for (int e = threadIdx.x; e < nch * kk; e += blockDim.x) out[e] = tile[(e / kk) * ts + e % kk];
}

// Staging of the score maps for position-sensitive pooling: x [B][C*k*k][H*W] (bf16)
// -> xs [B][H*W][k*k][Cp] with Cp = C rounded up to 8 (zeros past C), so that the
// C maps of one bin at one pixel are contiguous.  One workgroup per (image, block of 64
// pixels, bin, block of 64 output channels), transposed through LDS: reads are two
// pixels (4 bytes) of one map, writes 16-byte vectors of 8 channels of one pixel.  The
// workgroups run in that order (channel blocks fastest, then bins), so consecutive ones
// fill the k*k*Cp run of the same 64 pixels, and each XCD (workgroup g runs on XCD
// g % 8) takes a contiguous run of them.
constexpr int kPsPx = 64;
__global__ __launch_bounds__(kRT) void ps_stage_kernel(const uint16_t* x, uint16_t* xs, int B, int C, int KK, int HW,
                                                       int Cp, int ptiles, int ctiles) {
  __shared__ uint32_t t[64][kPsPx / 2 + 1];   // [channel][pixel pair]
  int e = blockIdx.x;
  {   // contiguous runs of workgroups per XCD (a bijection on [0, gridDim.x))
    const int T = static_cast<int>(gridDim.x), xcd = e & 7, q = T >> 3, rr = T & 7;
    e = xcd * q + min(xcd, rr) + (e >> 3);
  }
  const int ct = e % ctiles;
  e /= ctiles;
  const int bin = e % KK;
  e /= KK;
  const int pt = e % ptiles, b = e / ptiles;
  const int c0 = ct * 64, p0 = pt * kPsPx;
  const int tid = threadIdx.x;
  // 64 channels x 32 pixel pairs
  for (int q = tid; q < 64 * (kPsPx / 2); q += kRT) {
    const int cl = q / (kPsPx / 2), pp = q - (q / (kPsPx / 2)) * (kPsPx / 2);
    const int c = c0 + cl, p = p0 + 2 * pp;
    uint32_t v = 0u;
    if (c < C && p < HW) {
      const uint16_t* src = x + (static_cast<size_t>(b) * C * KK + static_cast<size_t>(c) * KK + bin) * HW + p;
      // H*W even (checked on the host): a pair never straddles the end of a map
      v = *reinterpret_cast<const uint32_t*>(src);
    }
    t[cl][pp] = v;
  }
  __syncthreads();
  // 64 pixels x 8 groups of 8 channels
  for (int q = tid; q < kPsPx * 8; q += kRT) {
    const int pl = q >> 3, g = q & 7;
    const int p = p0 + pl, c = c0 + 8 * g;
    if (p >= HW || c >= Cp) continue;
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = t[8 * g + i][pl >> 1];
    const uint32_t sh = (pl & 1) ? 16u : 0u;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = ((h[2 * i] >> sh) & 0xffffu) | (((h[2 * i + 1] >> sh) & 0xffffu) << 16);
    *reinterpret_cast<uint4*>(xs + ((static_cast<size_t>(b) * HW + p) * KK + bin) * Cp + c) =
        make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace
}  // namespace dcn

namespace {

// the staged path: bf16, k <= 16
bool roi_staged(const dcn_roi_desc* d) { return d->dtype == DCN_BF16 && d->pooled_size <= 16; }
int64_t roi_cp(const dcn_roi_desc* d) { return (d->channels + 7) / 8 * 8; }

int roi_check(const dcn_roi_desc* d) {
  if (d == nullptr) return DCN_E_ARG;
  if (d->batch < 1 || d->channels < 1 || d->height < 1 || d->width < 1 || d->num_rois < 0 || d->pooled_size < 1 ||
      d->samples < 1 || d->pooled_size > 1024 || d->samples > 64 || !std::isfinite(d->spatial_scale) ||
      !std::isfinite(d->gamma))
    return DCN_E_ARG;
  if (d->dtype != DCN_F32 && d->dtype != DCN_BF16) return DCN_E_UNSUPPORTED;
  const double lim = 2147483647.0;
  if (static_cast<double>(d->batch) * roi_cp(d) * d->height * d->width > lim ||
      static_cast<double>(d->num_rois) * d->channels * d->pooled_size * d->pooled_size > lim ||
      static_cast<double>(d->num_rois) * 2 * d->pooled_size * d->pooled_size > lim)
    return DCN_E_UNSUPPORTED;
  return DCN_OK;
}

}  // namespace

extern "C" int dcn_roi_pool_workspace_bytes(const dcn_roi_desc* d, size_t* bytes) {
  if (bytes == nullptr) return DCN_E_ARG;
  const int rc = roi_check(d);
  if (rc != DCN_OK) return rc;
  *bytes = (roi_staged(d) && d->num_rois > 0)
               ? static_cast<size_t>(d->batch * d->height * d->width * roi_cp(d)) * 2
               : 0;
  return DCN_OK;
}

extern "C" int dcn_roi_pool(const dcn_roi_desc* d, const void* x, const float* rois, const void* offset,
                            const void* mask, void* out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  const int rc = roi_check(d);
  if (rc != DCN_OK) return rc;
  if (d->num_rois == 0) return DCN_OK;
  if (x == nullptr || rois == nullptr || out == nullptr) return DCN_E_ARG;
  size_t need = 0;
  dcn_roi_pool_workspace_bytes(d, &need);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
    return DCN_E_WORKSPACE;
  dcn::RoiArgs a{};
  a.x = x;
  a.rois = rois;
  a.offset = offset;
  a.mask = mask;
  a.out = out;
  a.B = static_cast<int>(d->batch);
  a.C = static_cast<int>(d->channels);
  a.H = static_cast<int>(d->height);
  a.W = static_cast<int>(d->width);
  a.R = static_cast<int>(d->num_rois);
  a.k = static_cast<int>(d->pooled_size);
  a.S = static_cast<int>(d->samples);
  a.scale = d->spatial_scale;
  a.gamma = d->gamma;
  a.ps = 0;
  a.G = 1;
  void* args[] = {&a};
  if (roi_staged(d)) {
    // the channels-last copy, with the forward's staging kernel (no weight to repack)
    dcn::StageArgs sa{};
    sa.x = x;
    sa.w = nullptr;
    sa.xs = workspace;
    sa.wp = nullptr;
    sa.B = a.B;
    sa.Cin = a.C;
    sa.HW = a.H * a.W;
    sa.Cp = static_cast<int>(roi_cp(d));
    sa.Cout = 0;
    sa.Mp = 0;
    sa.KK = 1;
    sa.wlayout = 0;
    if (dcn::launch_stage(dcn::V_TILE_BF16_M64_N64, sa, stream) != hipSuccess) return DCN_E_HIP;
    const uint16_t* xs = static_cast<const uint16_t*>(workspace);
    int px_stride = sa.Cp, bin_stride = 0;
    void* cargs[] = {&a, &xs, &px_stride, &bin_stride};
    const unsigned grid = static_cast<unsigned>(a.R * ((a.C + 63) / 64));
    const size_t lds = static_cast<size_t>(64) * (a.k * a.k + 1) * 2;
    return hipLaunchKernel(reinterpret_cast<const void*>(&dcn::roi_pool_cl_kernel), dim3(grid), dim3(dcn::kRT),
                           cargs, lds, stream) == hipSuccess
               ? DCN_OK
               : DCN_E_HIP;
  }
  const long long n = static_cast<long long>(a.R) * a.C * a.k * a.k;
  const void* fn = d->dtype == DCN_BF16 ? reinterpret_cast<const void*>(&dcn::roi_pool_kernel<uint16_t>)
                                        : reinterpret_cast<const void*>(&dcn::roi_pool_kernel<float>);
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>((n + dcn::kRT - 1) / dcn::kRT)), dim3(dcn::kRT), args, 0,
                         stream) == hipSuccess
             ? DCN_OK
             : DCN_E_HIP;
}

// ---- deformable position-sensitive RoI pooling: the one-thread-per-output kernel with
// the bin's own score map as its plane (no workspace)
namespace {

int ps_roi_check(const dcn_ps_roi_desc* d) {
  if (d == nullptr) return DCN_E_ARG;
  const int64_t G = d->offset_groups > 1 ? d->offset_groups : 1;
  if (d->batch < 1 || d->out_channels < 1 || d->height < 1 || d->width < 1 || d->num_rois < 0 ||
      d->pooled_size < 1 || d->samples < 1 || d->pooled_size > 1024 || d->samples > 64 || d->offset_groups < 0 ||
      d->out_channels % G != 0 || !std::isfinite(d->spatial_scale) || !std::isfinite(d->gamma))
    return DCN_E_ARG;
  if (d->dtype != DCN_F32 && d->dtype != DCN_BF16) return DCN_E_UNSUPPORTED;
  const double lim = 2147483647.0, kk = static_cast<double>(d->pooled_size) * d->pooled_size;
  if (static_cast<double>(d->batch) * d->out_channels * kk * d->height * d->width > lim ||
      static_cast<double>(d->num_rois) * d->out_channels * kk > lim ||
      static_cast<double>(d->num_rois) * 2 * G * kk > lim || static_cast<double>(d->out_channels) * kk > lim)
    return DCN_E_UNSUPPORTED;
  return DCN_OK;
}

}  // namespace

namespace {

// the staged path of position-sensitive pooling: bf16, k <= 16, H*W even, and every
// 8-channel group in one offset group (one group, or C/G a multiple of 8)
bool ps_staged(const dcn_ps_roi_desc* d) {
  const int64_t G = d->offset_groups > 1 ? d->offset_groups : 1;
  return d->dtype == DCN_BF16 && d->pooled_size <= 16 && (d->height * d->width) % 2 == 0 &&
         (G == 1 || (d->out_channels / G) % 8 == 0);
}
int64_t ps_cp(const dcn_ps_roi_desc* d) { return (d->out_channels + 7) / 8 * 8; }

}  // namespace

extern "C" int dcn_ps_roi_pool_workspace_bytes(const dcn_ps_roi_desc* d, size_t* bytes) {
  if (bytes == nullptr) return DCN_E_ARG;
  const int rc = ps_roi_check(d);
  if (rc != DCN_OK) return rc;
  const int64_t kk = d->pooled_size * d->pooled_size;
  *bytes = (ps_staged(d) && d->num_rois > 0)
               ? static_cast<size_t>(d->batch * d->height * d->width) * static_cast<size_t>(kk * ps_cp(d)) * 2
               : 0;
  return DCN_OK;
}

extern "C" int dcn_ps_roi_pool(const dcn_ps_roi_desc* d, const void* x, const float* rois, const void* offset,
                               const void* mask, void* out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  const int rc = ps_roi_check(d);
  if (rc != DCN_OK) return rc;
  if (d->num_rois == 0) return DCN_OK;
  if (x == nullptr || rois == nullptr || out == nullptr) return DCN_E_ARG;
  size_t need = 0;
  dcn_ps_roi_pool_workspace_bytes(d, &need);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
    return DCN_E_WORKSPACE;
  dcn::RoiArgs a{};
  a.x = x;
  a.rois = rois;
  a.offset = offset;
  a.mask = mask;
  a.out = out;
  a.B = static_cast<int>(d->batch);
  a.C = static_cast<int>(d->out_channels);
  a.H = static_cast<int>(d->height);
  a.W = static_cast<int>(d->width);
  a.R = static_cast<int>(d->num_rois);
  a.k = static_cast<int>(d->pooled_size);
  a.S = static_cast<int>(d->samples);
  a.scale = d->spatial_scale;
  a.gamma = d->gamma;
  a.ps = 1;
  a.G = d->offset_groups > 1 ? static_cast<int>(d->offset_groups) : 1;
  if (need > 0) {
    // the score maps channels-last, bin-major, then the pooling from that copy
    const int KK = a.k * a.k, HW = a.H * a.W, Cp = static_cast<int>(ps_cp(d));
    const int ptiles = (HW + dcn::kPsPx - 1) / dcn::kPsPx, ctiles = (Cp + 63) / 64;
    const uint16_t* xin = static_cast<const uint16_t*>(x);
    uint16_t* xs = static_cast<uint16_t*>(workspace);
    int B = a.B, C = a.C;
    void* sargs[] = {&xin, &xs, &B, &C, const_cast<int*>(&KK), const_cast<int*>(&HW), const_cast<int*>(&Cp),
                     const_cast<int*>(&ptiles), const_cast<int*>(&ctiles)};
    const unsigned sgrid = static_cast<unsigned>(a.B * KK * ptiles * ctiles);
    if (hipLaunchKernel(reinterpret_cast<const void*>(&dcn::ps_stage_kernel), dim3(sgrid), dim3(dcn::kRT), sargs, 0,
                        stream) != hipSuccess)
      return DCN_E_HIP;
    const uint16_t* xsc = xs;
    int px_stride = KK * Cp, bin_stride = Cp;
    void* cargs[] = {&a, &xsc, &px_stride, &bin_stride};
    const unsigned grid = static_cast<unsigned>(a.R * ((a.C + 63) / 64));
    const size_t lds = static_cast<size_t>(64) * (KK + 1) * 2;
    return hipLaunchKernel(reinterpret_cast<const void*>(&dcn::roi_pool_cl_kernel), dim3(grid), dim3(dcn::kRT),
                           cargs, lds, stream) == hipSuccess
               ? DCN_OK
               : DCN_E_HIP;
  }
  void* args[] = {&a};
  const long long n = static_cast<long long>(a.R) * a.C * a.k * a.k;
  const void* fn = d->dtype == DCN_BF16 ? reinterpret_cast<const void*>(&dcn::roi_pool_kernel<uint16_t>)
                                        : reinterpret_cast<const void*>(&dcn::roi_pool_kernel<float>);
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>((n + dcn::kRT - 1) / dcn::kRT)), dim3(dcn::kRT), args, 0,
                         stream) == hipSuccess
             ? DCN_OK
             : DCN_E_HIP;
}
