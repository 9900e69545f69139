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

struct RoiArgs {
  const void* x;        // [B][C][H][W]
  const float* rois;    // [R][5]: batch index, x1, y1, x2, y2
  const void* offset;   // [R][2][k][k] or null
  const void* mask;     // [R][k][k] or null
  void* out;            // [R][C][k][k]
  int B, C, H, W, R, k, S;
  float scale, gamma;
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
  const float* roi = a.rois + static_cast<size_t>(r) * 5;
  const float bi = roi[0];
  T* out = static_cast<T*>(a.out);
  if (!(bi >= 0.f && bi < static_cast<float>(a.B))) {   // no such image (or NaN): zeros
    out[e] = st<T>(0.f);
    return;
  }
  const int b = static_cast<int>(bi);
  const float x1 = roi[1] * a.scale, y1 = roi[2] * a.scale;
  const float w = (roi[3] - roi[1]) * a.scale, h = (roi[4] - roi[2]) * a.scale;
  const float bw = w / static_cast<float>(a.k), bh = h / static_cast<float>(a.k);
  float dy = 0.f, dx = 0.f, m = 1.f;
  if (a.offset != nullptr) {
    const T* off = static_cast<const T*>(a.offset);
    dy = a.gamma * h * ld(off, ((static_cast<size_t>(r) * 2 + 0) * a.k + i) * a.k + j);
    dx = a.gamma * w * ld(off, ((static_cast<size_t>(r) * 2 + 1) * a.k + i) * a.k + j);
  }
  if (a.mask != nullptr) m = ld(static_cast<const T*>(a.mask), (static_cast<size_t>(r) * a.k + i) * a.k + j);
  const T* plane = static_cast<const T*>(a.x) + (static_cast<size_t>(b) * a.C + c) * a.H * a.W;
  const float inv = 1.f / static_cast<float>(a.S);
  float acc = 0.f;
  for (int u = 0; u < a.S; ++u) {
    const float py = y1 + (static_cast<float>(i) + (static_cast<float>(u) + 0.5f) * inv) * bh + dy;
    for (int v = 0; v < a.S; ++v) {
      const float px = x1 + (static_cast<float>(j) + (static_cast<float>(v) + 0.5f) * inv) * bw + dx;
      // no neighbour inside (or NaN): nothing to add
      if (!(py > -1.f && py < static_cast<float>(a.H) && px > -1.f && px < static_cast<float>(a.W))) continue;
      const float y0f = floorf(py), x0f = floorf(px);
      const float ly = py - y0f, lx = px - x0f;
      const int y0 = static_cast<int>(y0f), x0 = static_cast<int>(x0f);
      const bool iy0 = y0 >= 0, iy1 = y0 + 1 < a.H, ix0 = x0 >= 0, ix1 = x0 + 1 < a.W;
      const int q = y0 * a.W + x0;
      const float v00 = (iy0 && ix0) ? ld(plane, q) : 0.f;
      const float v01 = (iy0 && ix1) ? ld(plane, q + 1) : 0.f;
      const float v10 = (iy1 && ix0) ? ld(plane, q + a.W) : 0.f;
      const float v11 = (iy1 && ix1) ? ld(plane, q + a.W + 1) : 0.f;
      acc += (1.f - ly) * ((1.f - lx) * v00 + lx * v01) + ly * ((1.f - lx) * v10 + lx * v11);
    }
  }
  out[e] = st<T>(m * acc * inv * inv);
}

// bf16 with a channels-last copy xs [B][H][W][Cp] of the input: one workgroup per (RoI,
// block of 64 channels).  A unit of work is (bin, 8 channels): eight neighbouring lanes
// take the eight 8-channel groups of one bin, so each corner is one 128-byte read of
// 64 channels of one pixel.  The k*k x 64 results go through LDS, channel-major, and are
// stored as one contiguous run of out[r][c0 .. c0+63][k][k].
__global__ __launch_bounds__(kRT) void roi_pool_cl_kernel(RoiArgs a, const uint16_t* xs, int Cp) {
  extern __shared__ uint16_t tile[];   // [64 channels][bin], stride k*k + 1
  const int ncb = (a.C + 63) / 64;
  const int r = blockIdx.x / ncb, c0 = (blockIdx.x - r * ncb) * 64;
  const int kk = a.k * a.k, ts = kk + 1;
  const float* roi = a.rois + static_cast<size_t>(r) * 5;
  const float bi = roi[0];
  const bool batch_ok = bi >= 0.f && bi < static_cast<float>(a.B);
  const int b = batch_ok ? static_cast<int>(bi) : 0;
  const float x1 = roi[1] * a.scale, y1 = roi[2] * a.scale;
  const float w = (roi[3] - roi[1]) * a.scale, h = (roi[4] - roi[2]) * a.scale;
  const float bw = w / static_cast<float>(a.k), bh = h / static_cast<float>(a.k);
  const float inv = 1.f / static_cast<float>(a.S);
  const uint16_t* img = xs + static_cast<size_t>(b) * a.H * a.W * Cp;
  for (int u = threadIdx.x; u < kk * 8; u += blockDim.x) {
    const int bin = u >> 3, gq = u & 7, c = c0 + 8 * gq;
    const int i = bin / a.k, j = bin - (bin / a.k) * a.k;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    float m = 0.f;
    if (batch_ok && c < a.C) {
      float dy = 0.f, dx = 0.f;
      m = 1.f;
      if (a.offset != nullptr) {
        const uint16_t* off = static_cast<const uint16_t*>(a.offset);
        dy = a.gamma * h * ld(off, ((static_cast<size_t>(r) * 2 + 0) * a.k + i) * a.k + j);
        dx = a.gamma * w * ld(off, ((static_cast<size_t>(r) * 2 + 1) * a.k + i) * a.k + j);
      }
      if (a.mask != nullptr) m = ld(static_cast<const uint16_t*>(a.mask), (static_cast<size_t>(r) * a.k + i) * a.k + j);
      for (int su = 0; su < a.S; ++su) {
        const float py = y1 + (static_cast<float>(i) + (static_cast<float>(su) + 0.5f) * inv) * bh + dy;
        for (int sv = 0; sv < a.S; ++sv) {
          const float px = x1 + (static_cast<float>(j) + (static_cast<float>(sv) + 0.5f) * inv) * bw + dx;
          if (!(py > -1.f && py < static_cast<float>(a.H) && px > -1.f && px < static_cast<float>(a.W))) continue;
          const float y0f = floorf(py), x0f = floorf(px);
          const float ly = py - y0f, lx = px - x0f;
          const int y0 = static_cast<int>(y0f), x0 = static_cast<int>(x0f);
          const bool iy0 = y0 >= 0, iy1 = y0 + 1 < a.H, ix0 = x0 >= 0, ix1 = x0 + 1 < a.W;
          const float wt[4] = {(1.f - ly) * (1.f - lx), (1.f - ly) * lx, ly * (1.f - lx), ly * lx};
          const bool in[4] = {iy0 && ix0, iy0 && ix1, iy1 && ix0, iy1 && ix1};
          // the four corner loads together, from valid addresses (a corner outside the
          // image reads pixel 0 and is replaced by zeros)
          uint4 cv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int yy = in[q] ? y0 + (q >> 1) : 0, xc = in[q] ? x0 + (q & 1) : 0;
            cv[q] = *reinterpret_cast<const uint4*>(img + (static_cast<size_t>(yy) * a.W + xc) * Cp + c);
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
    int Cp = sa.Cp;
    void* cargs[] = {&a, &xs, &Cp};
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
