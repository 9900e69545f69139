// dcn_backward.hip -- gfx950 gradients of the modulated deformable convolution.
//
// For an upstream gradient gy[B][Cout][Ho][Wo], with the column entry
// col[b][c*K^2+k][p] = m_k * S(x[b,c], py_k, px_k) of the forward's deformable
// im2col (p an output pixel, S the bilinear sample with zero outside the image):
//
//   gcol[b][r][p]   = sum_o W[o][r] * gy[b][o][p]              (r = c*K^2 + k)
//   grad_weight[o][r] = sum_{b,p} gy[b][o][p] * col[b][r][p]
//   grad_bias[o]    = sum_{b,p} gy[b][o][p]
//   grad_mask       = sum_c gcol * S
//   grad_offset     = sum_c gcol * m * (dS/dpy, dS/dpx)
//   grad_x          = the column gradient times m, scattered to the four neighbours
//                     of each sample with their bilinear weights
//
// The offset gradient runs through the derivative of the bilinear kernel (the
// gradient equation of the csdn.net tags page "可变形卷积：Deformable ConvNets",
// part "Deformable Convolutional Networks", section 可变形卷积); the rest is the
// chain rule through the forward sum (same page, deformable-convolution equation,
// with the DCNv2 modulation scalar of section 3.2).  At an integer position the
// derivative is the one from the right (the side floor picks); positions are formed
// in fp32 as in the forward.
//
// Kernels, in launch order:
//   prep_w   W [Cout][R] -> Wt [R][Coutp] (the column-gradient product's first operand)
//   prep_gy  gy -> gyT [B][P][Coutp] and gyP [B][Cout][Pp] (both zero-padded), and
//            the bias gradient's per-tile sums (fp32 atomics)
//   fill     zero the fp32 accumulators (one launch)
//   gemm     gcol[b] = Wt x gyT[b]^T (MFMA, both operands contiguous along the reduction)
//   sample   per (b, group, channel block, kernel point, pixel): the sample's corners
//            and weights once, then for each channel the column entry (for the
//            weight gradient), the mask and offset partial sums and the four
//            scattered input-gradient contributions (fp32 atomics)
//   gemm     grad_weight = sum_b gyP[b] x col[b]^T, the reduction split over workgroups
//            (fp32 atomics into a zeroed accumulator)
//   gather   grad_x from the boxes (tiled path)
//   convert  fp32 accumulators -> the element type (one launch)
// The gradient products run on MFMA 32x32x16 bf16 (bf16 data) or 32x32x2 fp32.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <initializer_list>
#include <tuple>

#include "dcn.h"
#include "dcn_internal.h"

namespace dcn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBT = 256;   // threads per workgroup of the elementwise kernels
constexpr int kCB = 32;    // channels per thread in the sample kernel

template <typename T>
__device__ __forceinline__ float to_f(T v);
template <>
__device__ __forceinline__ float to_f<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f<uint16_t>(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

template <typename T>
__device__ __forceinline__ T from_f(float v);
template <>
__device__ __forceinline__ float from_f<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t from_f<uint16_t>(float v) {   // round to nearest even
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

struct BwdArgs {
  const void* x;        // [B][Cin][H][W]
  const void* offset;   // [B][2GK^2][Ho][Wo]
  const void* mask;     // [B][GK^2][Ho][Wo] or null
  const void* w;        // [Cout][Cin][K][K] = [Cout][R]
  const void* gy;       // [B][Cout][Ho][Wo]
  void* wt;             // [R][Coutp]
  void* gyt;            // [B][P][Coutp]
  void* gyp;            // [B][Cout][Pp]
  void* col;            // [B][R][Pp] or null (no weight gradient)
  float* gcol;          // [B][R][P] or null (no input, offset or mask gradient)
  float* gx32;          // [B][Cin][H][W] or null
  float* goff32;        // [B][2GK^2][P] or null
  float* gm32;          // [B][GK^2][P] or null
  float* gb32;          // [Cout] or null (bias gradient accumulator)
  float* outliers;      // [1]: set to 1 when a corner outside its box went to gx32
  int B, Cin, H, W, Cout, K, KK, stride, pad, dil, Ho, Wo, P, Pp, Coutp, R, G, Cg, NCB;
  // tiled sampling (bwd_sample_tile): output tiles of kTH x kTW pixels, an LDS box of
  // BH x BW input pixels per channel (the tile's footprint plus a margin of kMargin),
  // CBL channels of boxes at a time, each group's channels split over nsplit workgroups
  // of cps channels; gbox [B][Cin][TY][TX][BH*BW] keeps every box for the gather pass
  float* gbox;
  int TY, TX, BH, BW, CBL, nsplit, cps;
  int tiles_total;      // workgroups of the tiled sampling kernel: B * G * nsplit * TY * TX
};

constexpr int kTH = 8, kTW = 8;   // output tile of the tiled sampling kernel
constexpr int kMargin = 4;        // box margin (input pixels) around the tile's footprint

template <typename T>
__global__ __launch_bounds__(kBT) void bwd_prep_w(BwdArgs a) {
  const int e = blockIdx.x * kBT + threadIdx.x;
  if (e >= a.R * a.Coutp) return;
  const int o = e % a.Coutp, r = e / a.Coutp;
  const T* w = static_cast<const T*>(a.w);
  static_cast<T*>(a.wt)[e] = o < a.Cout ? w[static_cast<size_t>(o) * a.R + r] : T(0);
}

// 32 x 32 tiles of (output channel, pixel) through LDS: gyP keeps gy's layout with
// the pixel stride padded to Pp; gyT is its transpose with the channel stride
// padded to Coutp.  Padding is written as zeros.
template <typename T>
__global__ __launch_bounds__(kBT) void bwd_prep_gy(BwdArgs a) {
  __shared__ T tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int p0 = blockIdx.x * 32, o0 = blockIdx.y * 32, b = blockIdx.z;
  const T* gy = static_cast<const T*>(a.gy) + static_cast<size_t>(b) * a.Cout * a.P;
  T* gyp = a.gyp != nullptr ? static_cast<T*>(a.gyp) + static_cast<size_t>(b) * a.Cout * a.Pp : nullptr;
  T* gyt = a.gyt != nullptr ? static_cast<T*>(a.gyt) + static_cast<size_t>(b) * a.P * a.Coutp : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = o0 + ty + 8 * i, p = p0 + tx;
    const T v = (o < a.Cout && p < a.P) ? gy[static_cast<size_t>(o) * a.P + p] : T(0);
    tile[ty + 8 * i][tx] = v;
    if (gyp != nullptr && o < a.Cout && p < a.Pp) gyp[static_cast<size_t>(o) * a.Pp + p] = v;
  }
  __syncthreads();
  if (a.gyt != nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + ty + 8 * i, o = o0 + tx;
      if (p < a.P && o < a.Coutp) gyt[static_cast<size_t>(p) * a.Coutp + o] = tile[tx][ty + 8 * i];
    }
  }
  // the bias gradient: this tile's sum over its 32 pixels of each output channel
  if (a.gb32 != nullptr && threadIdx.x < 32 && o0 + static_cast<int>(threadIdx.x) < a.Cout) {
    float sum = 0.f;
#pragma unroll 8
    for (int t = 0; t < 32; ++t) sum += to_f(tile[threadIdx.x][t]);
    unsafeAtomicAdd(a.gb32 + o0 + threadIdx.x, sum);
  }
}

// Up to six fp32 ranges zeroed (or converted) by one launch; the workgroups are
// split over the ranges in proportion to their sizes (blocks[i] workgroups for range i).
struct Ranges {
  float* p[6];
  void* dst[6];
  int n[6];
  int blocks[6];
  int count;
};

__global__ __launch_bounds__(kBT) void bwd_fill_zero_ranges(Ranges r) {
  int blk = blockIdx.x, i = 0;
  while (i + 1 < r.count && blk >= r.blocks[i]) blk -= r.blocks[i++];
  const int e = (blk * kBT + static_cast<int>(threadIdx.x)) * 4;   // four floats per thread
  if (e + 4 <= r.n[i]) *reinterpret_cast<float4*>(r.p[i] + e) = make_float4(0.f, 0.f, 0.f, 0.f);
  else
    for (int t = e; t < r.n[i]; ++t) r.p[i][t] = 0.f;
}

template <typename T>
__global__ __launch_bounds__(kBT) void bwd_convert_ranges(Ranges r) {
  int blk = blockIdx.x, i = 0;
  while (i + 1 < r.count && blk >= r.blocks[i]) blk -= r.blocks[i++];
  const int e = blk * kBT + static_cast<int>(threadIdx.x);
  if (e < r.n[i]) static_cast<T*>(r.dst[i])[e] = from_f<T>(r.p[i][e]);
}

template <typename T>
__global__ __launch_bounds__(kBT) void bwd_fill_zero_t(T* p, int n) {
  const int e = blockIdx.x * kBT + threadIdx.x;
  if (e < n) p[e] = T(0);
}

// zero columns [P, Pp) of each of the rows of col
template <typename T>
__global__ __launch_bounds__(kBT) void bwd_col_pad(T* col, int rows, int P, int Pp) {
  const int r = blockIdx.x * kBT + threadIdx.x;
  if (r >= rows) return;
  for (int p = P; p < Pp; ++p) col[static_cast<size_t>(r) * Pp + p] = T(0);
}

template <typename T>
__global__ __launch_bounds__(kBT) void bwd_convert(const float* src, T* dst, int n) {
  const int e = blockIdx.x * kBT + threadIdx.x;
  if (e < n) dst[e] = from_f<T>(src[e]);
}

// One workgroup per (b, group, channel split, output tile of kTH x kTW pixels); the
// tile's K^2 x 64 samples are spread over the threads (NS per thread), and each
// sample's corners, weights and mask are computed once.  The input gradient is
// gathered, not scattered: once per workgroup the (sample, corner) pairs that land
// in the LDS box around the tile are sorted by box pixel (a count, a prefix sum and
// a placement), and then for each channel
//   1. each thread forms its samples' column entries (stored for the weight
//      gradient), reads their column gradients, accumulates the mask and offset sums,
//      and leaves gcol * m of each sample in LDS;
//   2. each thread sums, for its box pixels, gcol * m * (corner weight) over the pairs
//      sorted to that pixel and stores the sum to gbox.
// A corner outside the box (but inside the image) is added to the fp32 accumulator
// with a global atomic add.  The gather pass then sums the boxes covering each input
// pixel.  (LDS float atomics measured far slower than this on gfx950.)
template <typename T, int NS, int CQ>
__global__ __launch_bounds__(kBT) void bwd_sample_tile(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  constexpr int NE = NS * kBT * 4;                        // (sample, corner) pairs
  float* ent_w = reinterpret_cast<float*>(lds);           // [NE] corner weight
  uint16_t* ent_s = reinterpret_cast<uint16_t*>(lds + NE * 4);   // [NE] sample
  int* start = reinterpret_cast<int*>(lds + NE * 6);      // [BP + 1]
  const int tid = threadIdx.x;
  // Workgroups go to the eight XCDs in turn (workgroup w to XCD w % 8), and each XCD has
  // its own L2.  Neighbouring tiles share cache lines of gcol, x and col (a line holds
  // 32 fp32 pixels of a gcol row, four tiles' worth), so consecutive logical tiles are
  // given to workgroups of one XCD: logical index = XCD * per + (workgroup / 8).
  const int per = (a.tiles_total + 7) / 8;
  int t = static_cast<int>(blockIdx.x % 8) * per + static_cast<int>(blockIdx.x / 8);
  if (t >= a.tiles_total) return;   // the last XCD's spare workgroups (uniform)
  const int tx = t % a.TX;
  t /= a.TX;
  const int ty = t % a.TY;
  t /= a.TY;
  const int sp = t % a.nsplit;
  t /= a.nsplit;
  const int g = t % a.G, b = t / a.G;
  const int oy0 = ty * kTH, ox0 = tx * kTW;
  const int by0 = oy0 * a.stride - a.pad - kMargin, bx0 = ox0 * a.stride - a.pad - kMargin;
  const int BP = a.BH * a.BW, GKK = a.G * a.KK, HW = a.H * a.W;
  float* tgs = reinterpret_cast<float*>(lds + NE * 6 + ((BP + 1) * 4 + 15) / 16 * 16);   // [2][CQ][NS * kBT]
  const T* x = static_cast<const T*>(a.x);
  const T* off = static_cast<const T*>(a.offset);
  T* col = static_cast<T*>(a.col);
  const bool grads = a.gcol != nullptr;
  const bool scat = a.gx32 != nullptr;

  // per-sample state
  int p_[NS], pq_[NS], k_[NS], q00_[NS], bl_[NS], fl_[NS], o_[NS][4];
  float m_[NS], w_[NS][4], lx_[NS], ly_[NS], gm_[NS], goy_[NS], gox_[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int s = tid + i * kBT;
    const int k = s / (kTH * kTW), pl = s - k * (kTH * kTW);
    const int oy = oy0 + pl / kTW, ox = ox0 + pl % kTW;
    const bool valid = k < a.KK && oy < a.Ho && ox < a.Wo;
    p_[i] = valid ? oy * a.Wo + ox : -1;
    pq_[i] = valid ? p_[i] : 0;
    k_[i] = valid ? k : 0;
    o_[i][0] = o_[i][1] = o_[i][2] = o_[i][3] = 0;
    gm_[i] = goy_[i] = gox_[i] = 0.f;
    fl_[i] = 0;
    q00_[i] = 0;
    bl_[i] = -1;
    m_[i] = 0.f;
    lx_[i] = ly_[i] = 0.f;
    w_[i][0] = w_[i][1] = w_[i][2] = w_[i][3] = 0.f;
    if (!valid) continue;
    const int p = p_[i], gk = g * a.KK + k, ki = k / a.K, kj = k - (k / a.K) * a.K;
    const float dy = to_f(off[(static_cast<size_t>(b) * 2 * GKK + 2 * gk) * a.P + p]);
    const float dx = to_f(off[(static_cast<size_t>(b) * 2 * GKK + 2 * gk + 1) * a.P + p]);
    const float py = static_cast<float>(oy * a.stride - a.pad + ki * a.dil) + dy;
    const float px = static_cast<float>(ox * a.stride - a.pad + kj * a.dil) + dx;
    m_[i] = a.mask != nullptr ? to_f(static_cast<const T*>(a.mask)[(static_cast<size_t>(b) * GKK + gk) * a.P + p]) : 1.f;
    // a position with no neighbour in the image (or NaN) has none; at py == -1 the cell
    // is [-1, 0): row 0 has weight 0 but its derivative counts
    const bool any = py >= -1.f && py < static_cast<float>(a.H) && px >= -1.f && px < static_cast<float>(a.W);
    if (!any) continue;
    const float y0f = floorf(py), x0f = floorf(px);
    const float ly = py - y0f, lx = px - x0f;
    const int y0 = static_cast<int>(y0f), x0 = static_cast<int>(x0f);
    const bool iy0 = y0 >= 0, iy1 = y0 + 1 < a.H, ix0 = x0 >= 0, ix1 = x0 + 1 < a.W;
    fl_[i] = (iy0 && ix0 ? 1 : 0) | (iy0 && ix1 ? 2 : 0) | (iy1 && ix0 ? 4 : 0) | (iy1 && ix1 ? 8 : 0);
    q00_[i] = y0 * a.W + x0;
    o_[i][0] = (fl_[i] & 1) ? q00_[i] : 0;
    o_[i][1] = (fl_[i] & 2) ? q00_[i] + 1 : 0;
    o_[i][2] = (fl_[i] & 4) ? q00_[i] + a.W : 0;
    o_[i][3] = (fl_[i] & 8) ? q00_[i] + a.W + 1 : 0;
    const int yb = y0 - by0, xb = x0 - bx0;
    bl_[i] = (yb >= 0 && yb + 1 < a.BH && xb >= 0 && xb + 1 < a.BW) ? yb * a.BW + xb : -1;
    ly_[i] = ly;
    lx_[i] = lx;
    w_[i][0] = (1.f - ly) * (1.f - lx);
    w_[i][1] = (1.f - ly) * lx;
    w_[i][2] = ly * (1.f - lx);
    w_[i][3] = ly * lx;
  }

  // sort the in-box (sample, corner) pairs by box pixel: count, prefix sum, place
  if (scat) {
    for (int j = tid; j <= BP; j += kBT) start[j] = 0;
    __syncthreads();
    int rank[NS][4];
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        rank[i][n] = -1;
        if (bl_[i] >= 0 && (fl_[i] & (1 << n))) {
          const int j = bl_[i] + (n & 1) + (n >> 1) * a.BW;
          rank[i][n] = atomicAdd(&start[j + 1], 1);
        }
      }
    __syncthreads();
    if (tid < 64) {   // inclusive scan of start[1..BP] by one wave, 64 bins per pass
      int carry = 0;
      for (int j0 = 1; j0 <= BP; j0 += 64) {
        const int j = j0 + tid;
        int v = j <= BP ? start[j] : 0;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int u = __shfl_up(v, d);
          if (tid >= d) v += u;
        }
        if (j <= BP) start[j] = v + carry;
        carry += __shfl(v, 63);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        if (rank[i][n] >= 0) {
          const int j = bl_[i] + (n & 1) + (n >> 1) * a.BW;
          const int e = start[j] + rank[i][n];
          ent_s[e] = static_cast<uint16_t>(tid + i * kBT);
          ent_w[e] = w_[i][n];
        }
    __syncthreads();
  }

  const int cg0 = g * a.Cg + sp * a.cps, cg1 = min(cg0 + a.cps, (g + 1) * a.Cg);
  const size_t cstride = static_cast<size_t>(a.TY) * a.TX * BP;   // gbox: next channel, same tile
  float* gdst = scat ? a.gbox + (((static_cast<size_t>(b) * a.Cin + cg0) * a.TY + ty) * a.TX + tx) * BP : nullptr;
  // CQ channels per step: every load of the step first (from valid addresses: a corner
  // outside the image reads the plane's first element and is replaced by 0
  // afterwards), then the samples' work, one barrier, and the gather of the CQ
  // channels' boxes, which reads each sorted pair once for all of them.  The two
  // halves of tgs alternate between steps, so a thread still gathering step t reads a
  // half that step t+1 does not write.
  for (int c = cg0; c < cg1; c += CQ) {
    const int nq = min(CQ, cg1 - c);
    float* tg_s = tgs + (((c - cg0) / CQ) & 1) * (CQ * NS * kBT);
    float v[CQ][NS][4], gcv[CQ][NS];
#pragma unroll
    for (int q = 0; q < CQ; ++q) {
      const int cq = min(c + q, cg1 - 1);   // past the split's last channel: a repeat, not used
      const size_t pl = (static_cast<size_t>(b) * a.Cin + cq) * HW;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
#pragma unroll
        for (int n = 0; n < 4; ++n) v[q][i][n] = to_f(x[pl + o_[i][n]]);
        gcv[q][i] = grads ? a.gcol[(static_cast<size_t>(b) * a.R + cq * a.KK + k_[i]) * a.P + pq_[i]] : 0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < CQ; ++q) {
      if (q >= nq) break;
      const size_t pl = (static_cast<size_t>(b) * a.Cin + c + q) * HW;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int f = fl_[i];
        const float v00 = (f & 1) ? v[q][i][0] : 0.f, v01 = (f & 2) ? v[q][i][1] : 0.f;
        const float v10 = (f & 4) ? v[q][i][2] : 0.f, v11 = (f & 8) ? v[q][i][3] : 0.f;
        const float sv = w_[i][0] * v00 + w_[i][1] * v01 + w_[i][2] * v10 + w_[i][3] * v11;
        const size_t r = static_cast<size_t>(b) * a.R + (c + q) * a.KK + k_[i];
        if (col != nullptr && p_[i] >= 0) col[r * a.Pp + p_[i]] = from_f<T>(m_[i] * sv);
        if (!grads) continue;
        const float gc = gcv[q][i];
        gm_[i] += gc * sv;
        goy_[i] += gc * ((1.f - lx_[i]) * (v10 - v00) + lx_[i] * (v11 - v01));
        gox_[i] += gc * ((1.f - ly_[i]) * (v01 - v00) + ly_[i] * (v11 - v10));
        if (!scat) continue;
        const float tg = gc * m_[i];
        tg_s[q * (NS * kBT) + tid + i * kBT] = tg;
        if (bl_[i] < 0 && f != 0) {   // corners outside the box
          *a.outliers = 1.f;
          float* gx = a.gx32 + pl + q00_[i];
          if (f & 1) unsafeAtomicAdd(gx, tg * w_[i][0]);
          if (f & 2) unsafeAtomicAdd(gx + 1, tg * w_[i][1]);
          if (f & 4) unsafeAtomicAdd(gx + a.W, tg * w_[i][2]);
          if (f & 8) unsafeAtomicAdd(gx + a.W + 1, tg * w_[i][3]);
        }
      }
    }
    if (scat) {
      __syncthreads();
      for (int j = tid; j < BP; j += kBT) {
        float acc[CQ];
#pragma unroll
        for (int q = 0; q < CQ; ++q) acc[q] = 0.f;
        for (int e = start[j]; e < start[j + 1]; ++e) {
          const int sj = ent_s[e];
          const float w = ent_w[e];
#pragma unroll
          for (int q = 0; q < CQ; ++q) acc[q] += tg_s[q * (NS * kBT) + sj] * w;
        }
#pragma unroll
        for (int q = 0; q < CQ; ++q)
          if (q < nq) gdst[q * cstride + j] = acc[q];
      }
      gdst += CQ * cstride;
    }
  }
  if (grads) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (p_[i] < 0) continue;
      const int gk = g * a.KK + k_[i];
      if (a.goff32 != nullptr) {
        float* go = a.goff32 + (static_cast<size_t>(b) * 2 * GKK + 2 * gk) * a.P + p_[i];
        unsafeAtomicAdd(go, goy_[i] * m_[i]);
        unsafeAtomicAdd(go + a.P, gox_[i] * m_[i]);
      }
      if (a.gm32 != nullptr) unsafeAtomicAdd(a.gm32 + (static_cast<size_t>(b) * GKK + gk) * a.P + p_[i], gm_[i]);
    }
  }
}

// grad_x[b][c][y][x] = the fp32 accumulator (corners outside their box) plus the
// entries of every box that covers (y, x): tile ty's box starts at row
// ty*kTH*stride - pad - kMargin and has BH rows (likewise columns).
template <typename T>
__global__ __launch_bounds__(kBT) void bwd_gather_x(BwdArgs a, T* grad_x) {
  const long long e = static_cast<long long>(blockIdx.x) * kBT + threadIdx.x;
  const long long n = static_cast<long long>(a.B) * a.Cin * a.H * a.W;
  if (e >= n) return;
  const int xx = static_cast<int>(e % a.W);
  const int yy = static_cast<int>((e / a.W) % a.H);
  const long long bc = e / (static_cast<long long>(a.H) * a.W);
  const int sy = kTH * a.stride, sx = kTW * a.stride;
  const int ry = yy + a.pad + kMargin, rx = xx + a.pad + kMargin;   // >= 0
  const int ty1 = min(ry / sy, a.TY - 1), tx1 = min(rx / sx, a.TX - 1);
  const int BP = a.BH * a.BW;
  // the fp32 accumulator holds anything only if some corner fell outside its box
  float acc = *a.outliers != 0.f ? a.gx32[e] : 0.f;
  const float* base = a.gbox + static_cast<size_t>(bc) * a.TY * a.TX * BP;
  for (int ty = ty1; ty >= 0; --ty) {
    const int yb = ry - ty * sy;   // row inside tile ty's box
    if (yb >= a.BH) break;
    for (int tx = tx1; tx >= 0; --tx) {
      const int xb = rx - tx * sx;
      if (xb >= a.BW) break;
      acc += base[(static_cast<size_t>(ty) * a.TX + tx) * BP + yb * a.BW + xb];
    }
  }
  grad_x[e] = from_f<T>(acc);
}

// One thread per (b, group, channel block, kernel point, pixel), pixels fastest.
// Threads with a pixel in the padding [P, Pp) write the zero padding of col.
template <typename T>
__global__ __launch_bounds__(kBT) void bwd_sample(BwdArgs a) {
  const long long e = static_cast<long long>(blockIdx.x) * kBT + threadIdx.x;
  const long long total = static_cast<long long>(a.B) * a.G * a.NCB * a.KK * a.Pp;
  if (e >= total) return;
  const int p = static_cast<int>(e % a.Pp);
  long long t = e / a.Pp;
  const int k = static_cast<int>(t % a.KK);
  t /= a.KK;
  const int cb = static_cast<int>(t % a.NCB);
  t /= a.NCB;
  const int g = static_cast<int>(t % a.G), b = static_cast<int>(t / a.G);
  const int c0 = g * a.Cg + cb * kCB, c1 = min(c0 + kCB, (g + 1) * a.Cg);
  T* col = static_cast<T*>(a.col);
  if (p >= a.P) {
    if (col != nullptr)
      for (int c = c0; c < c1; ++c) col[(static_cast<size_t>(b) * a.R + c * a.KK + k) * a.Pp + p] = T(0);
    return;
  }
  const int gk = g * a.KK + k, GKK = a.G * a.KK;
  const int oy = p / a.Wo, ox = p - (p / a.Wo) * a.Wo, i = k / a.K, j = k - (k / a.K) * a.K;
  const T* off = static_cast<const T*>(a.offset);
  const float dy = to_f(off[(static_cast<size_t>(b) * 2 * GKK + 2 * gk) * a.P + p]);
  const float dx = to_f(off[(static_cast<size_t>(b) * 2 * GKK + 2 * gk + 1) * a.P + p]);
  const float py = static_cast<float>(oy * a.stride - a.pad + i * a.dil) + dy;
  const float px = static_cast<float>(ox * a.stride - a.pad + j * a.dil) + dx;
  const float m = a.mask != nullptr ? to_f(static_cast<const T*>(a.mask)[(static_cast<size_t>(b) * GKK + gk) * a.P + p])
                                    : 1.f;
  // corners and weights; a position with no neighbour in the image (or NaN) has none.
  // At py == -1 the cell is [-1, 0): row 0 has weight 0 but its derivative counts.
  const bool any = py >= -1.f && py < static_cast<float>(a.H) && px >= -1.f && px < static_cast<float>(a.W);
  const float y0f = any ? floorf(py) : 0.f, x0f = any ? floorf(px) : 0.f;
  const float ly = py - y0f, lx = px - x0f;
  const int y0 = static_cast<int>(y0f), x0 = static_cast<int>(x0f);
  const bool iy0 = any && y0 >= 0, iy1 = any && y0 + 1 < a.H, ix0 = any && x0 >= 0, ix1 = any && x0 + 1 < a.W;
  const bool in00 = iy0 && ix0, in01 = iy0 && ix1, in10 = iy1 && ix0, in11 = iy1 && ix1;
  const float w00 = (1.f - ly) * (1.f - lx), w01 = (1.f - ly) * lx, w10 = ly * (1.f - lx), w11 = ly * lx;
  const int q00 = y0 * a.W + x0;
  const int HW = a.H * a.W;
  const T* x = static_cast<const T*>(a.x);
  const bool grads = a.gcol != nullptr;
  float gm = 0.f, goy = 0.f, gox = 0.f;
  for (int c = c0; c < c1; ++c) {
    const size_t pl = (static_cast<size_t>(b) * a.Cin + c) * HW;
    const float v00 = in00 ? to_f(x[pl + q00]) : 0.f;
    const float v01 = in01 ? to_f(x[pl + q00 + 1]) : 0.f;
    const float v10 = in10 ? to_f(x[pl + q00 + a.W]) : 0.f;
    const float v11 = in11 ? to_f(x[pl + q00 + a.W + 1]) : 0.f;
    const float s = w00 * v00 + w01 * v01 + w10 * v10 + w11 * v11;
    const size_t r = static_cast<size_t>(b) * a.R + c * a.KK + k;
    if (col != nullptr) col[r * a.Pp + p] = from_f<T>(m * s);
    if (grads) {
      const float gc = a.gcol[r * a.P + p];
      gm += gc * s;
      goy += gc * ((1.f - lx) * (v10 - v00) + lx * (v11 - v01));
      gox += gc * ((1.f - ly) * (v01 - v00) + ly * (v11 - v10));
      if (a.gx32 != nullptr) {
        const float tg = gc * m;
        float* gx = a.gx32 + pl + q00;
        if (in00) unsafeAtomicAdd(gx, tg * w00);
        if (in01) unsafeAtomicAdd(gx + 1, tg * w01);
        if (in10) unsafeAtomicAdd(gx + a.W, tg * w10);
        if (in11) unsafeAtomicAdd(gx + a.W + 1, tg * w11);
      }
    }
  }
  if (grads) {
    if (a.goff32 != nullptr) {
      float* go = a.goff32 + (static_cast<size_t>(b) * 2 * GKK + 2 * gk) * a.P + p;
      unsafeAtomicAdd(go, goy * m);
      unsafeAtomicAdd(go + a.P, gox * m);
    }
    if (a.gm32 != nullptr) unsafeAtomicAdd(a.gm32 + (static_cast<size_t>(b) * GKK + gk) * a.P + p, gm);
  }
}

// C[z] (+)= sum over the reduction of A[m][k] * Bm[n][k]: both operands row-major with
// the reduction contiguous (rows padded with zeros to Kd, a multiple of 8).  The
// reduction runs over nseg segments of Kd (operand strides sAs, sBs), split evenly
// over ksplit workgroups per output tile (atomics into a zeroed C when ksplit > 1).
// blockIdx.z = zb * ksplit + ks, zb selecting independent problems (strides sAz, sBz,
// sCz).  A 128 x 128 output tile per workgroup, four waves of 64 x 64, 32-deep chunks
// staged through LDS with the next chunk's loads in flight during the multiply.
template <typename T>
struct GemmArgs {
  const T* A;
  const T* Bm;
  float* C;
  int M, N, Kd, lda, ldb, ldc, nseg, ksplit;
  long long sAs, sBs, sAz, sBz, sCz;
};

constexpr int kGM = 128, kGN = 128, kGK = 32;

template <typename T>
__global__ __launch_bounds__(256) void bwd_gemm_nt(GemmArgs<T> g) {
  constexpr bool kBF = sizeof(T) == 2;
  constexpr int VE = 16 / static_cast<int>(sizeof(T));   // elements per 16-byte vector
  constexpr int VPR = kGK / VE;                           // vectors per tile row
  constexpr int NV = kGM * VPR / 256;                     // vectors per thread and operand
  constexpr int LDT = kGK + VE;                           // LDS row stride in elements
  __shared__ __attribute__((aligned(16))) T As[kGM * LDT];
  __shared__ __attribute__((aligned(16))) T Bs[kGN * LDT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lh = lane >> 5, wm = wave >> 1, wn = wave & 1;
  // Output tiles in row-major order (N fastest), handed out so that each XCD (workgroup
  // w runs on XCD w % 8, each with its own L2) takes a contiguous run of tiles, which
  // share their A rows (and neighbouring runs their B rows) in that L2.
  const int ntn = (g.N + kGN - 1) / kGN, ntiles = ntn * ((g.M + kGM - 1) / kGM);
  const int xper = (ntiles + 7) / 8;
  const int lt = static_cast<int>(blockIdx.x % 8) * xper + static_cast<int>(blockIdx.x / 8);
  if (lt >= ntiles) return;   // spare workgroups of the last XCD (uniform)
  const int m0 = (lt / ntn) * kGM, n0 = (lt % ntn) * kGN;
  const int zb = blockIdx.z / g.ksplit, ks = blockIdx.z - zb * g.ksplit;
  const T* A = g.A + zb * g.sAz;
  const T* Bm = g.Bm + zb * g.sBz;
  float* C = g.C + zb * g.sCz;
  const int kchunks = (g.Kd + kGK - 1) / kGK;
  const int total = kchunks * g.nseg;
  const int per = (total + g.ksplit - 1) / g.ksplit;
  const int t0 = ks * per, t1 = min(total, t0 + per);
  floatx16 acc[2][2];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;
  uint4 ra[NV], rb[NV];
  auto gload = [&](int t) {
    const int seg = t / kchunks, kc = t - seg * kchunks;
    const T* Ap = A + seg * g.sAs;
    const T* Bp = Bm + seg * g.sBs;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int idx = tid + v * 256, row = idx / VPR, k = kc * kGK + (idx % VPR) * VE;
      const int ma = m0 + row, nb = n0 + row;
      ra[v] = (ma < g.M && k < g.Kd) ? *reinterpret_cast<const uint4*>(Ap + static_cast<size_t>(ma) * g.lda + k)
                                     : make_uint4(0, 0, 0, 0);
      rb[v] = (nb < g.N && k < g.Kd) ? *reinterpret_cast<const uint4*>(Bp + static_cast<size_t>(nb) * g.ldb + k)
                                     : make_uint4(0, 0, 0, 0);
    }
  };
  if (t0 < t1) gload(t0);
  for (int t = t0; t < t1; ++t) {
    __syncthreads();
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int idx = tid + v * 256, row = idx / VPR, kv = idx % VPR;
      *reinterpret_cast<uint4*>(As + row * LDT + kv * VE) = ra[v];
      *reinterpret_cast<uint4*>(Bs + row * LDT + kv * VE) = rb[v];
    }
    __syncthreads();
    if (t + 1 < t1) gload(t + 1);
    if constexpr (kBF) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 av[2], bv[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          av[q] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + q * 32 + l32) * LDT + h * 16 + lh * 8);
          bv[q] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 64 + q * 32 + l32) * LDT + h * 16 + lh * 8);
        }
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
          for (int tn = 0; tn < 2; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[tm], bv[tn], acc[tm][tn], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < kGK / 2; ++kk) {
        float av[2], bv[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          av[q] = As[(wm * 64 + q * 32 + l32) * LDT + 2 * kk + lh];
          bv[q] = Bs[(wn * 64 + q * 32 + l32) * LDT + 2 * kk + lh];
        }
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
          for (int tn = 0; tn < 2; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[tm], bv[tn], acc[tm][tn], 0, 0, 0);
      }
    }
  }
  if (t0 >= t1) return;
  // accumulator element r of a 32x32 block: row 8*(r/4) + 4*lh + r%4, column l32
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + tm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int cc = n0 + wn * 64 + tn * 32 + l32;
        if (row < g.M && cc < g.N) {
          float* dst = C + static_cast<size_t>(row) * g.ldc + cc;
          if (g.ksplit > 1) unsafeAtomicAdd(dst, acc[tm][tn][r]);
          else *dst = acc[tm][tn][r];
        }
      }
}

int64_t rup(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Workspace layout of one backward call.
struct BwdPlan {
  int64_t Ho = 0, Wo = 0, P = 0, Pp = 0, Coutp = 0, R = 0, G = 1;
  size_t o_wt = 0, o_gyt = 0, o_gyp = 0, o_col = 0, o_gcol = 0, o_gx = 0, o_gw = 0, o_goff = 0, o_gm = 0, o_gb = 0;
  size_t o_flag = 0;
  int64_t TY = 0, TX = 0, BH = 0, BW = 0;
  int CBL = 0;
  bool tiled = false;
  size_t o_gbox = 0;
  size_t bytes = 0;
};

int bwd_plan(const dcn_desc* d, BwdPlan* p) {
  int rc = check_desc(d, &p->Ho, &p->Wo);
  if (rc != DCN_OK) return rc;
  const int64_t B = d->batch, Cin = d->in_channels, Cout = d->out_channels, KK = d->kernel_size * d->kernel_size;
  p->G = d->offset_groups > 1 ? d->offset_groups : 1;
  p->P = p->Ho * p->Wo;
  p->Pp = rup(p->P, 8);
  p->Coutp = rup(Cout > 0 ? Cout : 1, 8);
  p->R = Cin * KK;
  const double lim = 2147483647.0;
  const double Bd = static_cast<double>(B);
  if (Bd * p->R * p->Pp > lim || Bd * Cin * d->height * d->width > lim || Bd * p->Coutp * p->Pp > lim ||
      static_cast<double>(p->R) * p->Coutp > lim || Bd * 2 * p->G * KK * p->P > lim ||
      static_cast<double>(Cout) * p->R > lim)
    return DCN_E_UNSUPPORTED;
  const size_t es = d->dtype == DCN_BF16 ? 2 : 4;
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o += align256(n);
    return at;
  };
  p->o_wt = take(static_cast<size_t>(p->R * p->Coutp) * es);
  p->o_gyt = take(static_cast<size_t>(B * p->P * p->Coutp) * es);
  p->o_gyp = take(static_cast<size_t>(B * Cout * p->Pp) * es);
  p->o_col = take(static_cast<size_t>(B * p->R * p->Pp) * es);
  p->o_gcol = take(static_cast<size_t>(B * p->R * p->P) * 4);
  p->o_gx = take(static_cast<size_t>(B * Cin * d->height * d->width) * 4);
  p->o_gw = take(static_cast<size_t>(Cout * p->R) * 4);
  p->o_goff = take(static_cast<size_t>(B * 2 * p->G * KK * p->P) * 4);
  p->o_gm = take(static_cast<size_t>(B * p->G * KK * p->P) * 4);
  p->o_gb = take(static_cast<size_t>(Cout) * 4);
  p->o_flag = take(4);
  // tiled sampling: K^2 <= 28 (seven samples per thread at most) and a box of at
  // least four channels in 64 KB of LDS
  p->TY = (p->Ho + kTH - 1) / kTH;
  p->TX = (p->Wo + kTW - 1) / kTW;
  p->BH = (kTH - 1) * d->stride + (d->kernel_size - 1) * d->dilation + 2 + 2 * kMargin;
  p->BW = (kTW - 1) * d->stride + (d->kernel_size - 1) * d->dilation + 2 + 2 * kMargin;
  const double box_elems = static_cast<double>(B) * Cin * p->TY * p->TX * p->BH * p->BW;
  p->CBL = 1;
  p->tiled = KK <= 28 && p->BH * p->BW <= 1536 && box_elems <= lim;
  if (p->tiled) p->o_gbox = take(static_cast<size_t>(box_elems) * 4);
  p->bytes = o;
  return DCN_OK;
}

hipError_t launch1(const void* fn, int64_t n, void** args, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>((n + kBT - 1) / kBT)), dim3(kBT), args, 0, s);
}

// ranges[i] = (fp32 buffer, destination or null, elements); null buffers are skipped
hipError_t launch_ranges(const void* fn, int per_thread, std::initializer_list<std::tuple<float*, void*, int64_t>> list,
                         hipStream_t s) {
  Ranges r{};
  int total = 0;
  for (const auto& t : list) {
    if (std::get<0>(t) == nullptr || std::get<2>(t) <= 0) continue;
    r.p[r.count] = std::get<0>(t);
    r.dst[r.count] = std::get<1>(t);
    r.n[r.count] = static_cast<int>(std::get<2>(t));
    r.blocks[r.count] = static_cast<int>((std::get<2>(t) + kBT * per_thread - 1) / (kBT * per_thread));
    total += r.blocks[r.count];
    ++r.count;
  }
  if (r.count == 0) return hipSuccess;
  void* args[] = {&r};
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(total)), dim3(kBT), args, 0, s);
}

template <typename T>
hipError_t convert(const float* src, void* dst, int64_t n, hipStream_t s) {
  T* d = static_cast<T*>(dst);
  int nn = static_cast<int>(n);
  void* args[] = {&src, &d, &nn};
  return launch1(reinterpret_cast<const void*>(&bwd_convert<T>), n, args, s);
}

template <typename T>
hipError_t gemm(const GemmArgs<T>& g, int zb, hipStream_t s) {
  GemmArgs<T> gg = g;
  void* args[] = {&gg};
  const int ntiles = ((g.N + kGN - 1) / kGN) * ((g.M + kGM - 1) / kGM);
  const dim3 grid(static_cast<unsigned>((ntiles + 7) / 8 * 8), 1, static_cast<unsigned>(zb * g.ksplit));
  return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_gemm_nt<T>), grid, dim3(256), args, 0, s);
}

#define BWD_TRY(e)                          \
  do {                                      \
    if ((e) != hipSuccess) return DCN_E_HIP; \
  } while (0)

template <typename T>
int run_backward(const dcn_desc* d, const BwdPlan& p, const void* x, const void* offset, const void* mask,
                 const void* weight, const void* grad_out, void* grad_x, void* grad_offset, void* grad_mask,
                 void* grad_weight, void* grad_bias, unsigned char* ws, hipStream_t s) {
  BwdArgs a{};
  a.x = x;
  a.offset = offset;
  a.mask = mask;
  a.w = weight;
  a.gy = grad_out;
  a.B = static_cast<int>(d->batch);
  a.Cin = static_cast<int>(d->in_channels);
  a.H = static_cast<int>(d->height);
  a.W = static_cast<int>(d->width);
  a.Cout = static_cast<int>(d->out_channels);
  a.K = static_cast<int>(d->kernel_size);
  a.KK = a.K * a.K;
  a.stride = static_cast<int>(d->stride);
  a.pad = static_cast<int>(d->pad);
  a.dil = static_cast<int>(d->dilation);
  a.Ho = static_cast<int>(p.Ho);
  a.Wo = static_cast<int>(p.Wo);
  a.P = static_cast<int>(p.P);
  a.Pp = static_cast<int>(p.Pp);
  a.Coutp = static_cast<int>(p.Coutp);
  a.R = static_cast<int>(p.R);
  a.G = static_cast<int>(p.G);
  a.Cg = a.Cin / a.G;
  a.NCB = (a.Cg + kCB - 1) / kCB;
  const bool need_gcol = grad_x != nullptr || grad_offset != nullptr || (grad_mask != nullptr && mask != nullptr);
  a.wt = ws + p.o_wt;
  a.gyt = need_gcol ? static_cast<void*>(ws + p.o_gyt) : nullptr;
  a.gyp = grad_weight != nullptr ? static_cast<void*>(ws + p.o_gyp) : nullptr;
  a.gb32 = grad_bias != nullptr ? reinterpret_cast<float*>(ws + p.o_gb) : nullptr;
  a.outliers = reinterpret_cast<float*>(ws + p.o_flag);
  a.col = grad_weight != nullptr ? static_cast<void*>(ws + p.o_col) : nullptr;
  a.gcol = need_gcol ? reinterpret_cast<float*>(ws + p.o_gcol) : nullptr;
  a.gx32 = grad_x != nullptr ? reinterpret_cast<float*>(ws + p.o_gx) : nullptr;
  a.goff32 = grad_offset != nullptr ? reinterpret_cast<float*>(ws + p.o_goff) : nullptr;
  a.gm32 = (grad_mask != nullptr && mask != nullptr) ? reinterpret_cast<float*>(ws + p.o_gm) : nullptr;
  float* gw32 = reinterpret_cast<float*>(ws + p.o_gw);
  const int64_t nx = static_cast<int64_t>(a.B) * a.Cin * a.H * a.W;
  const int64_t noff = static_cast<int64_t>(a.B) * 2 * a.G * a.KK * a.P;
  const int64_t nm = noff / 2;
  const int64_t nw = static_cast<int64_t>(a.Cout) * a.R;
  void* args[] = {&a};

  if (need_gcol) {
    BWD_TRY(launch1(reinterpret_cast<const void*>(&bwd_prep_w<T>), static_cast<int64_t>(a.R) * a.Coutp, args, s));
  }
  // every fp32 accumulator zeroed by one launch (before prep_gy adds the bias sums)
  BWD_TRY(launch_ranges(reinterpret_cast<const void*>(&bwd_fill_zero_ranges), 4,
                        {{a.gx32, nullptr, nx}, {a.goff32, nullptr, noff}, {a.gm32, nullptr, nm},
                         {grad_weight != nullptr ? gw32 : nullptr, nullptr, nw}, {a.gb32, nullptr, a.Cout},
                         {a.outliers, nullptr, 1}},
                        s));
  if (need_gcol || grad_weight != nullptr || grad_bias != nullptr) {
    const dim3 grid(static_cast<unsigned>((a.Pp + 31) / 32), static_cast<unsigned>((a.Coutp + 31) / 32),
                    static_cast<unsigned>(a.B));
    BWD_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&bwd_prep_gy<T>), grid, dim3(kBT), args, 0, s));
  }
  if (need_gcol) {
    GemmArgs<T> g{};
    g.A = static_cast<const T*>(a.wt);
    g.Bm = static_cast<const T*>(a.gyt);
    g.C = a.gcol;
    g.M = a.R;
    g.N = a.P;
    g.Kd = a.Coutp;
    g.lda = g.ldb = a.Coutp;
    g.ldc = a.P;
    g.nseg = 1;
    g.ksplit = 1;
    g.sAz = 0;
    g.sBz = static_cast<long long>(a.P) * a.Coutp;
    g.sCz = static_cast<long long>(a.R) * a.P;
    BWD_TRY(gemm<T>(g, a.B, s));
  }
  if ((need_gcol || grad_weight != nullptr) && p.tiled) {
    a.gbox = reinterpret_cast<float*>(ws + p.o_gbox);
    a.TY = static_cast<int>(p.TY);
    a.TX = static_cast<int>(p.TX);
    a.BH = static_cast<int>(p.BH);
    a.BW = static_cast<int>(p.BW);
    a.CBL = p.CBL;
    // split each group's channels until there are about four workgroups per CU
    const int64_t wgs = static_cast<int64_t>(a.B) * a.G * a.TY * a.TX;
    int ns = 1;
    while (wgs * ns < 1024 && (a.Cg + ns * 2 - 1) / (ns * 2) >= 16) ns *= 2;
    a.cps = (a.Cg + ns - 1) / ns;
    a.nsplit = (a.Cg + a.cps - 1) / a.cps;
    if (grad_weight != nullptr && a.Pp > a.P) {   // zero padding of the columns
      const int64_t n = static_cast<int64_t>(a.B) * a.R;
      T* colp = static_cast<T*>(a.col);
      int rows = static_cast<int>(n), P = a.P, Pp = a.Pp;
      void* pargs[] = {&colp, &rows, &P, &Pp};
      BWD_TRY(launch1(reinterpret_cast<const void*>(&bwd_col_pad<T>), n, pargs, s));
    }
    // LDS: the sorted pairs (weight, sample), the bin starts, two halves of gcol * m
    // (three samples per thread: four channels per step; seven: one)
    const int nsmp = a.KK <= 12 ? 3 : 7, cq = a.KK <= 12 ? 4 : 1;
    const size_t lds = static_cast<size_t>(nsmp) * kBT * 4 * 6 + ((a.BH * a.BW + 1) * 4 + 15) / 16 * 16 +
                       static_cast<size_t>(2) * cq * nsmp * kBT * 4;
    a.tiles_total = static_cast<int>(wgs * a.nsplit);
    const unsigned grid = static_cast<unsigned>((a.tiles_total + 7) / 8 * 8);
    const void* fn = a.KK <= 12 ? reinterpret_cast<const void*>(&bwd_sample_tile<T, 3, 4>)
                                : reinterpret_cast<const void*>(&bwd_sample_tile<T, 7, 1>);
    BWD_TRY(hipLaunchKernel(fn, dim3(grid), dim3(kBT), args, lds, s));
  } else if (need_gcol || grad_weight != nullptr) {
    const int64_t n = static_cast<int64_t>(a.B) * a.G * a.NCB * a.KK * a.Pp;
    BWD_TRY(launch1(reinterpret_cast<const void*>(&bwd_sample<T>), n, args, s));
  }
  if (grad_weight != nullptr) {
    GemmArgs<T> g{};
    g.A = static_cast<const T*>(a.gyp);
    g.Bm = static_cast<const T*>(a.col);
    g.C = gw32;
    g.M = a.Cout;
    g.N = a.R;
    g.Kd = a.Pp;
    g.lda = g.ldb = a.Pp;
    g.ldc = a.R;
    g.nseg = a.B;
    g.sAs = static_cast<long long>(a.Cout) * a.Pp;
    g.sBs = static_cast<long long>(a.R) * a.Pp;
    // split the reduction until the output tiles and splits give about one workgroup per CU
    // (more splits measured slower: more fp32 atomics into the accumulator)
    const int tiles = ((a.Cout + kGM - 1) / kGM) * ((a.R + kGN - 1) / kGN);
    const int chunks = ((a.Pp + kGK - 1) / kGK) * a.B;
    int ks = 1;
    while (tiles * ks < 256 && ks * 2 <= chunks / 4) ks *= 2;
    g.ksplit = ks;
    BWD_TRY(gemm<T>(g, 1, s));
  }
  if (a.gx32 != nullptr) {
    if (p.tiled) {
      T* gxo = static_cast<T*>(grad_x);
      void* gargs[] = {&a, &gxo};
      BWD_TRY(launch1(reinterpret_cast<const void*>(&bwd_gather_x<T>), nx, gargs, s));
    } else {
      BWD_TRY(convert<T>(a.gx32, grad_x, nx, s));
    }
  }
  // the other fp32 accumulators to the element type, one launch
  BWD_TRY(launch_ranges(reinterpret_cast<const void*>(&bwd_convert_ranges<T>), 1,
                        {{grad_weight != nullptr ? gw32 : nullptr, grad_weight, nw}, {a.goff32, grad_offset, noff},
                         {a.gm32, grad_mask, nm}, {a.gb32, grad_bias, a.Cout}},
                        s));
  return DCN_OK;
}

// Outputs of an empty problem (B == 0 or Cout == 0) that still have elements: the
// sums over nothing are zero.
template <typename T>
int zero_outputs(const dcn_desc* d, const BwdPlan& p, void* grad_x, void* grad_offset, void* grad_mask,
                 const void* mask, void* grad_weight, void* grad_bias, hipStream_t s) {
  const int64_t B = d->batch, KK = d->kernel_size * d->kernel_size;
  struct Out {
    void* ptr;
    int64_t n;
  } outs[] = {{grad_x, B * d->in_channels * d->height * d->width},
              {grad_offset, B * 2 * p.G * KK * p.P},
              {mask != nullptr ? grad_mask : nullptr, B * p.G * KK * p.P},
              {grad_weight, d->out_channels * p.R},
              {grad_bias, d->out_channels}};
  for (const Out& o : outs) {
    if (o.ptr == nullptr || o.n == 0) continue;
    T* ptr = static_cast<T*>(o.ptr);
    int n = static_cast<int>(o.n);
    void* args[] = {&ptr, &n};
    BWD_TRY(launch1(reinterpret_cast<const void*>(&bwd_fill_zero_t<T>), o.n, args, s));
  }
  return DCN_OK;
}

}  // namespace
}  // namespace dcn

extern "C" int dcn_backward_workspace_bytes(const dcn_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return DCN_E_ARG;
  dcn::BwdPlan p;
  const int rc = dcn::bwd_plan(desc, &p);
  if (rc != DCN_OK) return rc;
  *bytes = (desc->batch == 0 || desc->out_channels == 0) ? 0 : p.bytes;
  return DCN_OK;
}

extern "C" int dcn_backward(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                            const void* weight, const void* grad_out, void* grad_x, void* grad_offset,
                            void* grad_mask, void* grad_weight, void* grad_bias, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  dcn::BwdPlan p;
  const int rc = dcn::bwd_plan(desc, &p);
  if (rc != DCN_OK) return rc;
  const bool bf16 = desc->dtype == DCN_BF16;
  if (desc->batch == 0 || desc->out_channels == 0)
    return bf16 ? dcn::zero_outputs<uint16_t>(desc, p, grad_x, grad_offset, grad_mask, mask, grad_weight, grad_bias,
                                              stream)
                : dcn::zero_outputs<float>(desc, p, grad_x, grad_offset, grad_mask, mask, grad_weight, grad_bias,
                                           stream);
  if (x == nullptr || offset == nullptr || weight == nullptr || grad_out == nullptr) return DCN_E_ARG;
  if (workspace == nullptr || workspace_bytes < p.bytes || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return DCN_E_WORKSPACE;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  return bf16 ? dcn::run_backward<uint16_t>(desc, p, x, offset, mask, weight, grad_out, grad_x, grad_offset, grad_mask,
                                            grad_weight, grad_bias, ws, stream)
              : dcn::run_backward<float>(desc, p, x, offset, mask, weight, grad_out, grad_x, grad_offset, grad_mask,
                                         grad_weight, grad_bias, ws, stream);
}
