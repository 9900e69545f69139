// dcn_backward.hip -- gfx950 gradients of the modulated deformable convolution.
//
// For an upstream gradient gy[B][Cout][Ho][Wo], with the column entry
// col[b][c*K^2+k][p] = m_k * S(x[b,c], py_k, px_k) of the forward's deformable
// im2col (p an output pixel, S the bilinear sample with zero outside the image):
//
//   gcol[b][p][k][c]  = sum_o W[o][c][k] * gy[b][o][p]
//   grad_weight[o][r] = sum_{b,p} gy[b][o][p] * col[b][r][p]
//   grad_bias[o]      = sum_{b,p} gy[b][o][p]
//   grad_mask         = sum_c gcol * S
//   grad_offset       = sum_c gcol * m * (dS/dpy, dS/dpx)
//   grad_x            = the column gradient times m, carried to the four neighbours
//                       of each sample with their bilinear weights
//
// The offset gradient runs through the derivative of the bilinear kernel (the
// gradient equation of the csdn.net tags page "可变形卷积：Deformable ConvNets",
// part "Deformable Convolutional Networks", section 可变形卷积); the rest is the
// chain rule through the forward sum (same page, deformable-convolution equation,
// with the DCNv2 modulation scalar of section 3.2).  At an integer position the
// derivative is the one from the right (the side floor picks); positions are formed
// in fp32 as in the forward.
//
// Launches, in order:
//   stage    x -> xs [B][H][W][Cp], channels last (the forward's staging kernel)
//   prep_1   W [Cout][Cin][K^2] -> Wt [K^2][Cin][Coutp] (the column-gradient product's
//            second operand, rows in the column gradient's channel-fastest order), and
//            the bias accumulator and the pair counters zeroed
//   prep_2   gy -> gyT [B][P][Coutp] and, when P is not a multiple of 8, gyP
//            [B][Cout][Pp] (both zero-padded; otherwise gy itself serves as gyP), with
//            the bias gradient's per-tile sums (fp32 atomics); and the pair count: per
//            sample (b, group, kernel point, pixel) each corner inside the image counted
//            at its input pixel
//   scan     exclusive prefix sums of the counts: per block of 2048 (also copied to the
//            per-pixel cursors), then the block sums
//   gemm     gcol[b] = gyT[b] x Wt^T, channels fastest: [B][P][K^2][Cin] (MFMA), rounded
//            to the element type
//   sample   per (b, group, kernel point, 32 output pixels): the corners from xs as
//            16-byte channel vectors; the column entries, transposed through LDS to
//            col [B][R][Pp] for the weight gradient; the offset and mask gradients summed
//            over the group's channels across the lanes of the sample and written once;
//            and each in-image corner's pair (column-gradient row, m * corner weight)
//            placed in its input pixel's list at the slot its cursor hands out
//   gather   grad_x per input pixel: the sum over its pairs of weight * column-gradient
//            row, transposed through LDS to [B][Cin][H][W]
//   gemm     grad_weight = sum_b gyP[b] x col[b]^T, the reduction split over workgroups,
//            each split's partial sum to its own fp32 slice
//   reduce   the partial sums added in split order and rounded to the element type; the
//            bias accumulator converted
// The gradient products run on MFMA 32x32x16 bf16 (bf16 data) or 32x32x2 fp32.  The
// input, offset, mask and weight gradients take no atomics: each is summed by one thread,
// one group of lanes or one pass in a fixed order, and rounded to the element type once.

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

constexpr int kBT = 256;     // threads per workgroup
constexpr int kSP = 32;      // output pixels per workgroup of the sampling kernel (one kernel point)
constexpr int kGH = 1, kGW = 8;   // input tile (rows x columns) of a workgroup of the gather kernel
constexpr int kGP = kGH * kGW;
constexpr int kCC = 256;     // channels per chunk of the sampling and gather kernels (32 lanes x 8)
constexpr int kScanB = 2048; // counts per block of the first scan pass (256 threads x 8)
static_assert(kSP * 4 <= kBT, "the sampling kernel places four corners per sample with one thread each");

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

// A workgroup barrier that orders LDS traffic only: global loads and stores issued
// before it stay in flight across it (a plain __syncthreads also waits for those).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup id -> work item, so that consecutive items run on the same XCD (workgroups
// are dealt to the 8 XCDs round-robin; XCD x takes the contiguous item range
// [x*q + min(x,r), ... + q + (x<r)) of T = 8q + r items; a bijection on [0, T)).
__device__ __forceinline__ int xcd_item(int g, int T) {
  const int xcd = g & 7, idx = g >> 3;
  const int q = T >> 3, r = T & 7;
  return xcd * q + min(xcd, r) + idx;
}

struct BwdArgs {
  const void* xs;       // staged x, [B][H][W][Cp] (channels >= Cin zero)
  const void* offset;   // [B][2GK^2][Ho][Wo]
  const void* mask;     // [B][GK^2][Ho][Wo] or null
  const void* w;        // [Cout][Cin][K][K] = [Cout][R]
  const void* gy;       // [B][Cout][Ho][Wo]
  void* wt;             // [K^2][Cin][Coutp]
  void* gyt;            // [B][P][Coutp]
  void* gyp;            // [B][Cout][Pp]
  void* col;            // [B][R][Pp] or null (no weight gradient)
  void* gcol;           // [B][P][K^2][Cin] in the element type, or null (no input, offset or
                        // mask gradient)
  float* gb32;          // [Cout] or null (bias gradient accumulator)
  void* grad_offset;    // [B][2GK^2][Ho][Wo] or null
  void* grad_mask;      // [B][GK^2][Ho][Wo] or null
  void* grad_x;         // [B][Cin][H][W] or null
  int* cnt;             // [B*G*H*W + 1]: pairs per input pixel, then their block-local
                        // exclusive prefix sums
  int* bsum;            // [ceil((B*G*H*W + 1) / kScanB)]: block sums, then their exclusive sums
  int* cur;             // [B*G*H*W + 1]: each pixel's next free slot (block-local, as cnt)
  int2* pairs;          // [B*G*K^2*P*4]: (column-gradient row, bits of m * corner weight)
  int B, Cin, H, W, Cout, K, KK, stride, pad, dil, Ho, Wo, P, Pp, Coutp, R, G, Cg, Cp;
  int lg;               // lanes per sample (sampling) or pixel (gather): a power of two
                        // <= 32, eight channels per lane
  int npb;              // kSP-pixel blocks of the output plane
  int nqy, nqx;         // kGH x kGW tiles of the input plane (rows, columns)
  int ncc;              // 256-channel chunks of a group
  int nsamp;            // B * G * K^2 * P
  int gyp_copy;         // 1: gyp is a padded copy to write (Pp > P); 0: gyp is gy
};

// Wt[k*Cin + c][o] = W[o][c*K^2 + k] (zero for o >= Cout): 32 x 32 tiles of (o, r)
// through LDS, read along r and written along o.
template <typename T>
__device__ __forceinline__ void prep_w_tile(const BwdArgs& a, T (*tile)[33], int bx, int by) {
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int r0 = bx * 32, o0 = by * 32;
  const T* w = static_cast<const T*>(a.w);
  T* wt = static_cast<T*>(a.wt);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int o = o0 + ty + 8 * i, r = r0 + tx;
    tile[ty + 8 * i][tx] = (o < a.Cout && r < a.R) ? w[static_cast<size_t>(o) * a.R + r] : T(0);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + ty + 8 * i, o = o0 + tx;
    if (r < a.R && o < a.Coutp) {
      const int c = r / a.KK, k = r - (r / a.KK) * a.KK;
      wt[(static_cast<size_t>(k) * a.Cin + c) * a.Coutp + o] = tile[tx][ty + 8 * i];
    }
  }
}

// 64 x 64 tiles of (output channel, pixel) through LDS: gyP keeps gy's layout with the
// pixel stride padded to Pp (written only when Pp > P; otherwise gy itself serves); gyT
// is its transpose with the channel stride padded to Coutp.  Padding is written as
// zeros.  With vec (P a multiple of 16 bytes' worth and gy 16-byte aligned) rows are
// read as 16-byte vectors; gyT rows are written as 16-byte vectors of channels.  Also
// the bias gradient: this tile's sum over its pixels of each output channel (fp32
// atomics).
constexpr int kGT = 64;   // tile edge of the grad_out transposes
template <typename T>
__device__ __forceinline__ void prep_gy_tile(const BwdArgs& a, T* tile, int bx, int by, int b, bool vec) {
  constexpr int VE = 16 / static_cast<int>(sizeof(T)), TPV = kGT + VE;   // LDS pitch
  const int tid = threadIdx.x;
  const int p0 = bx * kGT, o0 = by * kGT;
  const T* gy = static_cast<const T*>(a.gy) + static_cast<size_t>(b) * a.Cout * a.P;
  T* gyp = a.gyp != nullptr && a.gyp_copy ? static_cast<T*>(a.gyp) + static_cast<size_t>(b) * a.Cout * a.Pp : nullptr;
  T* gyt = a.gyt != nullptr ? static_cast<T*>(a.gyt) + static_cast<size_t>(b) * a.P * a.Coutp : nullptr;
  // read: rows o of kGT pixels, VE pixels per item
  for (int idx = tid; idx < kGT * (kGT / VE); idx += kBT) {
    const int ol = idx / (kGT / VE), pl = (idx % (kGT / VE)) * VE;
    const int o = o0 + ol, p = p0 + pl;
    T v[VE];
    if (vec && o < a.Cout && p < a.P) {
      const uint4 q = *reinterpret_cast<const uint4*>(gy + static_cast<size_t>(o) * a.P + p);
      __builtin_memcpy(v, &q, 16);
    } else {
#pragma unroll
      for (int j = 0; j < VE; ++j) v[j] = (o < a.Cout && p + j < a.P) ? gy[static_cast<size_t>(o) * a.P + p + j] : T(0);
    }
    uint4 q;
    __builtin_memcpy(&q, v, 16);
    *reinterpret_cast<uint4*>(tile + ol * TPV + pl) = q;
    if (gyp != nullptr && o < a.Cout)
#pragma unroll
      for (int j = 0; j < VE; ++j)
        if (p + j < a.Pp) gyp[static_cast<size_t>(o) * a.Pp + p + j] = v[j];
  }
  __syncthreads();
  if (gyt != nullptr) {   // rows p of kGT channels, VE channels per item (Coutp: a multiple of 8)
    for (int idx = tid; idx < kGT * (kGT / VE); idx += kBT) {
      const int pl = idx / (kGT / VE), ol = (idx % (kGT / VE)) * VE;
      const int p = p0 + pl, o = o0 + ol;
      if (p >= a.P || o >= a.Coutp) continue;
      T v[VE];
#pragma unroll
      for (int j = 0; j < VE; ++j) v[j] = tile[(ol + j) * TPV + pl];
      uint4 q;
      __builtin_memcpy(&q, v, 16);
      *reinterpret_cast<uint4*>(gyt + static_cast<size_t>(p) * a.Coutp + o) = q;
    }
  }
  if (a.gb32 != nullptr && tid < kGT && o0 + tid < a.Cout) {
    float sum = 0.f;
#pragma unroll 8
    for (int t = 0; t < kGT; ++t) sum += to_f(tile[tid * TPV + t]);   // pixels past P are zero
    unsafeAtomicAdd(a.gb32 + o0 + tid, sum);
  }
}

// Up to six fp32 ranges zeroed by one launch; the workgroups are
// split over the ranges in proportion to their sizes (blocks[i] workgroups for range i).
struct Ranges {
  float* p[6];
  int n[6];
  int blocks[6];
  int count;
};

__device__ __forceinline__ void fill_zero_block(const Ranges& r, int blk) {
  int i = 0;
  while (i + 1 < r.count && blk >= r.blocks[i]) blk -= r.blocks[i++];
  const int e = (blk * kBT + static_cast<int>(threadIdx.x)) * 4;   // four floats per thread
  if (e + 4 <= r.n[i]) *reinterpret_cast<float4*>(r.p[i] + e) = make_float4(0.f, 0.f, 0.f, 0.f);
  else
    for (int t = e; t < r.n[i]; ++t) r.p[i][t] = 0.f;
}

template <typename T>
__global__ __launch_bounds__(kBT) void bwd_fill_zero_t(T* p, int n) {
  const int e = blockIdx.x * kBT + threadIdx.x;
  if (e < n) p[e] = T(0);
}

// Data-parallel-primitive lane moves: v from lane (lane permuted by CTRL) of the same row
// of 16 lanes.  0xB1: quad_perm [1,0,3,2] (lane ^ 1); 0x4E: quad_perm [2,3,0,1] (lane ^ 2);
// 0x141: row_half_mirror (lane 7 - i within each 8 lanes); 0x140: row_mirror (lane 15 - i).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
// The sum of v over an aligned group of lg lanes (a power of two <= 32), in every lane of
// the group: each step adds the value of a lane in the other half of a group twice the
// size, whose lanes already agree.
__device__ __forceinline__ float group_sum(float v, int lg) {
  if (lg >= 2) v += dpp_move<0xB1>(v);
  if (lg >= 4) v += dpp_move<0x4E>(v);
  if (lg >= 8) v += dpp_move<0x141>(v);
  if (lg >= 16) v += dpp_move<0x140>(v);
  if (lg >= 32) v += __shfl_xor(v, 16);
  return v;
}

// One sample's geometry: its corners inside the image (bit n of fl: corner n of 00, 01,
// 10, 11), the flat index of corner 00, the four bilinear weights, the cell
// fractions and the mask.  A position with no neighbour in the image (or NaN) has no
// corner; at py == -1 the cell is [-1, 0): row 0 has weight 0 but its derivative counts.
struct Geo {
  int fl, q00;
  float w00, w01, w10, w11, ly, lx, m;
};

template <typename T>
__device__ __forceinline__ Geo sample_geo(const BwdArgs& a, int b, int g, int k, int p) {
  Geo e;
  const int GKK = a.G * a.KK, gk = g * a.KK + k;
  const int oy = p / a.Wo, ox = p - (p / a.Wo) * a.Wo, ki = k / a.K, kj = k - (k / a.K) * a.K;
  const T* off = static_cast<const T*>(a.offset);
  const float dy = to_f(off[(static_cast<size_t>(b) * 2 * GKK + 2 * gk) * a.P + p]);
  const float dx = to_f(off[(static_cast<size_t>(b) * 2 * GKK + 2 * gk + 1) * a.P + p]);
  const float py = static_cast<float>(oy * a.stride - a.pad + ki * a.dil) + dy;
  const float px = static_cast<float>(ox * a.stride - a.pad + kj * a.dil) + dx;
  e.m = a.mask != nullptr ? to_f(static_cast<const T*>(a.mask)[(static_cast<size_t>(b) * GKK + gk) * a.P + p]) : 1.f;
  const bool any = py >= -1.f && py < static_cast<float>(a.H) && px >= -1.f && px < static_cast<float>(a.W);
  const float y0f = any ? floorf(py) : 0.f, x0f = any ? floorf(px) : 0.f;
  const float ly = any ? py - y0f : 0.f, lx = any ? px - x0f : 0.f;
  const int y0 = static_cast<int>(y0f), x0 = static_cast<int>(x0f);
  const bool iy0 = any && y0 >= 0, iy1 = any && y0 + 1 < a.H, ix0 = any && x0 >= 0, ix1 = any && x0 + 1 < a.W;
  e.fl = (iy0 && ix0 ? 1 : 0) | (iy0 && ix1 ? 2 : 0) | (iy1 && ix0 ? 4 : 0) | (iy1 && ix1 ? 8 : 0);
  e.q00 = y0 * a.W + x0;
  e.ly = ly;
  e.lx = lx;
  e.w00 = (1.f - ly) * (1.f - lx);
  e.w01 = (1.f - ly) * lx;
  e.w10 = ly * (1.f - lx);
  e.w11 = ly * lx;
  return e;
}

__device__ __forceinline__ int corner_dq(int n, int W) { return (n & 1) + (n >> 1) * W; }
__device__ __forceinline__ float corner_w(const Geo& e, int n) {
  return n == 0 ? e.w00 : n == 1 ? e.w01 : n == 2 ? e.w10 : e.w11;
}

// One thread per sample s = ((b*G + g)*K^2 + k)*P + p: each corner inside the image is
// counted at its input pixel (increments whose old value nobody waits for).
template <typename T>
__device__ __forceinline__ void count_block(const BwdArgs& a, int blk) {
  const int s = blk * kBT + threadIdx.x;
  if (s >= a.nsamp) return;
  const int p = s % a.P;
  int t = s / a.P;
  const int k = t % a.KK;
  t /= a.KK;
  const int g = t % a.G, b = t / a.G;
  const Geo e = sample_geo<T>(a, b, g, k, p);
  int* c = a.cnt + (b * a.G + g) * a.H * a.W;
#pragma unroll
  for (int n = 0; n < 4; ++n)
    if ((e.fl >> n) & 1) atomicAdd(c + e.q00 + corner_dq(n, a.W), 1);
}

// Two launches share the small independent steps: the first the weight transpose and
// the zero fill (bias accumulator, pair counters), the second the grad_out transposes
// (with the bias sums) and the pair count.  Workgroups [0, n1) take the first step,
// the rest the second.
struct PrepLaunch {
  BwdArgs a;
  Ranges r;            // ranges to zero
  int wx, wy;          // weight-transpose tiles (0 x 0: none)
  int gx, gy, gz;      // grad_out tiles (0: none)
  int gy_vec;          // grad_out rows readable as 16-byte vectors
};

template <typename T>
__global__ __launch_bounds__(kBT) void bwd_prep_1(PrepLaunch L) {
  __shared__ T tile[32][33];
  const int n1 = L.wx * L.wy, blk = blockIdx.x;
  if (blk < n1) prep_w_tile<T>(L.a, tile, blk % L.wx, blk / L.wx);
  else fill_zero_block(L.r, blk - n1);
}

template <typename T>
__global__ __launch_bounds__(kBT) void bwd_prep_2(PrepLaunch L) {
  __shared__ __attribute__((aligned(16))) T tile[kGT * (kGT + 16 / sizeof(T))];
  const int n1 = L.gx * L.gy * L.gz, blk = blockIdx.x;
  if (blk < n1) prep_gy_tile<T>(L.a, tile, blk % L.gx, (blk / L.gx) % L.gy, blk / (L.gx * L.gy), L.gy_vec);
  else count_block<T>(L.a, blk - n1);
}

// Exclusive prefix sums of cnt[0, n) within blocks of kScanB (in place, and copied to
// cur); each block's total to bsum[block].
__global__ __launch_bounds__(kBT) void bwd_scan_blocks(int* cnt, int n, int* bsum, int* cur) {
  __shared__ int wsum[kBT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int base = blockIdx.x * kScanB + tid * 8;
  int v[8], run = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = base + i;
    const int c = j < n ? cnt[j] : 0;
    v[i] = run;
    run += c;
  }
  int inc = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(inc, d);
    if (lane >= d) inc += u;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  int woff = 0;
  for (int w = 0; w < wv; ++w) woff += wsum[w];
  const int off = woff + inc - run;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = base + i;
    if (j < n) cnt[j] = cur[j] = v[i] + off;
  }
  if (tid == kBT - 1) bsum[blockIdx.x] = woff + inc;
}

// Exclusive prefix sums of bsum[0, nb) in place, one workgroup.
__global__ __launch_bounds__(kBT) void bwd_scan_top(int* bsum, int nb) {
  __shared__ int wsum[kBT / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;
  for (int j0 = 0; j0 < nb; j0 += kBT) {
    const int j = j0 + tid;
    const int v = j < nb ? bsum[j] : 0;
    int inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(inc, d);
      if (lane >= d) inc += u;
    }
    if (lane == 63) wsum[wv] = inc;
    __syncthreads();
    int woff = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kBT / 64; ++w) {
      if (w < wv) woff += wsum[w];
      total += wsum[w];
    }
    if (j < nb) bsum[j] = carry + woff + inc - v;
    carry += total;
    __syncthreads();
  }
}

// first pair of input pixel i (flat over (b, group, pixel)); i + 1 gives the end
__device__ __forceinline__ int pair_start(const BwdArgs& a, int i) { return a.cnt[i] + a.bsum[i / kScanB]; }

// eight values from 8 consecutive elements (16- or 32-byte aligned) as fp32
__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(u[i] << 16);
    v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 q0 = *reinterpret_cast<const float4*>(p), q1 = *reinterpret_cast<const float4*>(p + 4);
  v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w;
  v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
}
__device__ __forceinline__ void store8(uint16_t* p, const float v[8]) {
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    u[i] = static_cast<uint32_t>(from_f<uint16_t>(v[2 * i])) | (static_cast<uint32_t>(from_f<uint16_t>(v[2 * i + 1])) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(u[0], u[1], u[2], u[3]);
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// One workgroup per (b, group, kSP output pixels, kernel point), kernel points fastest
// and consecutive items on one XCD (the kernel points of a pixel block read neighbouring
// corners).  Small items keep the dispatcher's tail short and, with few registers (no
// sample's loads kept across another's), five waves per SIMD in flight.  First, four
// threads per sample: the sample's geometry (to LDS) and, one corner each, a slot for
// its pair in its input pixel's list from the pixel's cursor (the pair is stored after
// the channel work, whose first loads overlap these).  Then a sample is taken by lg lanes, eight channels
// each (16-byte channel vectors of xs and of its column-gradient row), all its loads
// issued together; with 256 channels, 32 lanes and eight samples at a time.  The group's
// channels go in chunks of 256: the chunk's column entries of the block wait in LDS
// ([pixel][channel]) and leave as row segments of col (kSP pixels of one (channel,
// kernel point) row).  The corner sums of a chunk are summed over the sample's lanes,
// and carried from chunk to chunk in LDS by the sample's first lane.
template <typename T>
__global__ __launch_bounds__(kBT) void bwd_sample_cl(BwdArgs a) {
  constexpr int ES = sizeof(T), VE = 16 / ES;   // elements per 16-byte vector
  constexpr int TP = kCC + VE;                   // LDS pitch of one pixel's entries
  __shared__ __attribute__((aligned(16))) T tile[kSP * TP];
  __shared__ float sacc[4][kSP];   // corner sums of the chunks so far
  __shared__ float sgeo[7][kSP];   // w00, w01, w10, w11, ly, lx, m of each sample
  __shared__ int sfl[kSP], sq[kSP];
  const int tid = threadIdx.x;
  int t = xcd_item(blockIdx.x, a.B * a.G * a.npb * a.KK);
  const int k = t % a.KK;
  t /= a.KK;
  const int pb = t % a.npb;
  t /= a.npb;
  const int g = t % a.G, b = t / a.G;
  const int GKK = a.G * a.KK, gk = g * a.KK + k;
  // this thread's pair: sample tid / 4, corner tid % 4 (pos < 0: none)
  int pos = -1, prow = 0;
  float pw = 0.f;
  if (tid < 4 * kSP) {
    const int pl = tid >> 2, n = tid & 3, p = pb * kSP + pl;
    if (p < a.P) {
      const Geo e = sample_geo<T>(a, b, g, k, p);
      if (n == 0) {
        sgeo[0][pl] = e.w00;
        sgeo[1][pl] = e.w01;
        sgeo[2][pl] = e.w10;
        sgeo[3][pl] = e.w11;
        sgeo[4][pl] = e.ly;
        sgeo[5][pl] = e.lx;
        sgeo[6][pl] = e.m;
        sfl[pl] = e.fl;
        sq[pl] = e.q00;
      }
      if (a.pairs != nullptr && ((e.fl >> n) & 1)) {
        const int i = (b * a.G + g) * a.H * a.W + e.q00 + corner_dq(n, a.W);
        pos = atomicAdd(a.cur + i, 1) + a.bsum[i / kScanB];
        prow = (b * a.P + p) * a.KK + k;
        pw = e.m * corner_w(e, n);
      }
    }
  }
  lds_barrier();
  const int LG = a.lg, li = tid & (LG - 1), si = tid / LG, SPI = kBT / LG;
  const int nit = (kSP + SPI - 1) / SPI;
  const bool grads = a.gcol != nullptr;
  const bool vec = a.Cg % 8 == 0;
  const int c8 = li * 8;   // lg * 8 >= the chunk's channels: one octet per lane at most
  T* col = static_cast<T*>(a.col);
  const T* xs = static_cast<const T*>(a.xs) + static_cast<size_t>(b) * a.H * a.W * a.Cp + g * a.Cg;
  struct Ld {
    float v[4][8], gc[8];
  };
  for (int cc0 = 0; cc0 < a.Cg; cc0 += kCC) {
    const int ccn = min(kCC, a.Cg - cc0);
    const bool act = c8 < ccn;
    // the corners and column gradients of the sample of iteration it (zeros where none)
    // The loads are unconditional (a corner outside the image, a lane past the chunk's
    // channels or a missing sample reads pixel 0 / channel 0 and is zeroed afterwards):
    // a load under a lane-dependent branch would be waited for before the branch ends.
    auto load = [&](int it, Ld& L) {
      const int pl = it * SPI + si, p = pb * kSP + pl;
      const bool ok = act && pl < kSP && p < a.P;
      const int fl = ok ? sfl[pl] : 0, q00 = ok ? sq[pl] : 0;
      const int ce = act ? c8 : 0;
      const T* xq = xs + cc0 + ce;
      // element indices within the image's xs and within gcol fit 32 bits (checked by the plan)
      const uint32_t grow = ok ? static_cast<uint32_t>((b * a.P + p) * a.KK + k) : 0u;
      const T* gcr = static_cast<const T*>(a.gcol) + (grow * static_cast<uint32_t>(a.Cin) + g * a.Cg + cc0 + ce);
      if (vec) {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const bool on = (fl >> n) & 1;
          const uint32_t q = on ? static_cast<uint32_t>(q00 + corner_dq(n, a.W)) : 0u;
          load8(xq + q * static_cast<uint32_t>(a.Cp), L.v[n]);
#pragma unroll
          for (int j = 0; j < 8; ++j) L.v[n][j] = on ? L.v[n][j] : 0.f;
        }
        if (grads) {   // uniform
          load8(gcr, L.gc);
#pragma unroll
          for (int j = 0; j < 8; ++j) L.gc[j] = ok ? L.gc[j] : 0.f;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) L.gc[j] = 0.f;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool in = ok && c8 + j < ccn;
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const bool on = in && ((fl >> n) & 1);
            const uint32_t e = on ? static_cast<uint32_t>(q00 + corner_dq(n, a.W)) * static_cast<uint32_t>(a.Cp) + j : 0u;
            const float v = to_f(xq[e]);
            L.v[n][j] = on ? v : 0.f;
          }
          const float gv = grads ? to_f(gcr[in ? j : 0]) : 0.f;
          L.gc[j] = in ? gv : 0.f;
        }
      }
    };
    // Column entries to LDS; the four corner sums sum_c gc * v_corner over the sample's
    // lanes, kept (more chunks to come) or turned into the gradients.  The mask and
    // offset gradients are linear in the corner values, so each is the same combination
    // of the corner sums: grad_mask = sum_n w_n * S_n, and the position derivatives
    // (1 - lx)(S10 - S00) + lx (S11 - S01) and (1 - ly)(S01 - S00) + ly (S11 - S10).
    auto work = [&](int it, const Ld& L) {
      const int pl = it * SPI + si, p = pb * kSP + pl;
      if (pl >= kSP || p >= a.P) return;   // uniform over the sample's lanes
      const float w00 = sgeo[0][pl], w01 = sgeo[1][pl], w10 = sgeo[2][pl], w11 = sgeo[3][pl];
      const float m = sgeo[6][pl];
      if (col != nullptr && act) {
        const float m00 = m * w00, m01 = m * w01, m10 = m * w10, m11 = m * w11;
        float cv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) cv[j] = m00 * L.v[0][j] + m01 * L.v[1][j] + m10 * L.v[2][j] + m11 * L.v[3][j];
        T* dst = tile + pl * TP + c8;
        if (vec) {
          store8(dst, cv);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c8 + j < ccn) dst[j] = from_f<T>(cv[j]);
        }
      }
      if (!grads) return;
      float sc[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += L.gc[j] * L.v[n][j];
        sc[n] = acc;
      }
#pragma unroll
      for (int n = 0; n < 4; ++n) sc[n] = group_sum(sc[n], LG);
      if (li != 0) return;
      if (cc0 > 0)
#pragma unroll
        for (int n = 0; n < 4; ++n) sc[n] += sacc[n][pl];
      if (cc0 + kCC < a.Cg) {
#pragma unroll
        for (int n = 0; n < 4; ++n) sacc[n][pl] = sc[n];
        return;
      }
      const float ly = sgeo[4][pl], lx = sgeo[5][pl];
      if (a.grad_offset != nullptr) {
        const float goy = (1.f - lx) * (sc[2] - sc[0]) + lx * (sc[3] - sc[1]);
        const float gox = (1.f - ly) * (sc[1] - sc[0]) + ly * (sc[3] - sc[2]);
        T* go = static_cast<T*>(a.grad_offset) + (static_cast<size_t>(b) * 2 * GKK + 2 * gk) * a.P + p;
        go[0] = from_f<T>(goy * m);
        go[a.P] = from_f<T>(gox * m);
      }
      if (a.grad_mask != nullptr)
        static_cast<T*>(a.grad_mask)[(static_cast<size_t>(b) * GKK + gk) * a.P + p] =
            from_f<T>(w00 * sc[0] + w01 * sc[1] + w10 * sc[2] + w11 * sc[3]);
    };
    for (int it = 0; it < nit; ++it) {
      Ld L;
      load(it, L);
      work(it, L);
    }
    if (col != nullptr) {
      lds_barrier();
      // rows (channel, kernel point) of col: 16 bytes (VE pixels) per thread, the pieces
      // of one row on neighbouring lanes, so that a store instruction writes whole row
      // segments (few, large write requests) rather than 16 bytes in each of 64 rows
      const int ng = kSP / VE;
      for (int idx = tid; idx < ccn * ng; idx += kBT) {
        const int pg = idx % ng, c = idx / ng;
        const int p0 = pb * kSP + pg * VE;
        if (p0 >= a.Pp) continue;
        T vals[VE];
#pragma unroll
        for (int j = 0; j < VE; ++j) vals[j] = p0 + j < a.P ? tile[(pg * VE + j) * TP + c] : T(0);
        const uint32_t r = static_cast<uint32_t>(b * a.R + (g * a.Cg + cc0 + c) * a.KK + k);
        uint4 q;
        __builtin_memcpy(&q, vals, 16);
        *reinterpret_cast<uint4*>(col + (r * static_cast<uint32_t>(a.Pp) + p0)) = q;
      }
      lds_barrier();
    }
  }
  if (pos >= 0) a.pairs[pos] = make_int2(prow, __float_as_int(pw));
}

// One workgroup per (b, group, 256-channel chunk, kGH x kGW input pixels), tiles in
// raster order and consecutive tiles on one XCD, so that the rows of a sample's corners
// are fetched by neighbouring workgroups of one L2.  First each pixel's pair range (to
// LDS); then lg lanes per pixel, eight channels each: the pixel's pairs loaded by its
// lanes at once (one pair per lane, then passed round by lane shuffles), their
// column-gradient rows eight at a time, and the sum of weight * row; the chunk's sums
// leave through LDS ([channel][pixel]) as kGW-pixel row segments per channel.
template <typename T>
__global__ __launch_bounds__(kBT) void bwd_gather_cl(BwdArgs a) {
  constexpr int GP = kGP + 1;   // LDS pitch of one channel's pixels
  __shared__ T tile[kCC * GP];
  __shared__ int sst[2 * kGP];  // pair range of each pixel
  const int tid = threadIdx.x, HW = a.H * a.W;
  int t = xcd_item(blockIdx.x, a.B * a.G * a.ncc * a.nqy * a.nqx);
  const int tx = t % a.nqx;
  t /= a.nqx;
  const int ty = t % a.nqy;
  t /= a.nqy;
  const int ci = t % a.ncc;
  t /= a.ncc;
  const int g = t % a.G, b = t / a.G;
  const int ib = (b * a.G + g) * HW;
  const int y0 = ty * kGH, x0 = tx * kGW;
  if (tid < kGP) {
    const int y = y0 + tid / kGW, x = x0 + tid % kGW;
    const bool in = y < a.H && x < a.W;
    const int i = ib + y * a.W + x;
    sst[2 * tid] = in ? pair_start(a, i) : 0;
    sst[2 * tid + 1] = in ? pair_start(a, i + 1) : 0;
  }
  lds_barrier();
  const int cc0 = ci * kCC, ccn = min(kCC, a.Cg - cc0);
  const int LG = a.lg, li = tid & (LG - 1), si = tid / LG, SPI = kBT / LG;
  const int nit = (kGP + SPI - 1) / SPI;
  const bool vec = a.Cg % 8 == 0;
  const T* gsrc = static_cast<const T*>(a.gcol) + g * a.Cg + cc0;
  const int lbase = threadIdx.x & 63 & ~(LG - 1);   // the group's first lane in the wave
  for (int it = 0; it < nit; ++it) {
    const int pl = it * SPI + si;
    if (pl >= kGP) continue;
    const int e0 = sst[2 * pl], e1 = sst[2 * pl + 1];   // empty outside the image
    // every lane of the pixel takes part in loading and passing round the pairs, also
    // the lanes past the chunk's channels (lg * 8 >= the chunk's channels)
    const int c8 = li * 8;
    const bool act = c8 < ccn;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    for (int eb = e0; eb < e1; eb += LG) {
      const int nb = min(LG, e1 - eb);
      const int2 mine = li < nb ? a.pairs[eb + li] : make_int2(0, 0);
      if (vec) {
        for (int u0 = 0; u0 < nb; u0 += 8) {
          float v[8][8], wm[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int src = lbase + min(u0 + u, nb - 1);
            const int row = __shfl(mine.x, src);
            wm[u] = u0 + u < nb ? __int_as_float(__shfl(mine.y, src)) : 0.f;
            // unconditional (row is a valid pair's, c8 clamped): its data only feed lanes
            // whose sums are stored
            load8(gsrc + (static_cast<uint32_t>(row) * static_cast<uint32_t>(a.Cin) + (act ? c8 : 0)), v[u]);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] += wm[u] * v[u][j];
        }
      } else {
        for (int u = 0; u < nb; ++u) {
          const int row = __shfl(mine.x, lbase + u);
          const float wm = __int_as_float(__shfl(mine.y, lbase + u));
          const T* src = gsrc + (static_cast<uint32_t>(row) * static_cast<uint32_t>(a.Cin) + c8);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (c8 + j < ccn) acc[j] += wm * to_f(src[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c8 + j < ccn) tile[(c8 + j) * GP + pl] = from_f<T>(acc[j]);
  }
  lds_barrier();
  T* gx = static_cast<T*>(a.grad_x) + (static_cast<size_t>(b) * a.Cin + g * a.Cg + cc0) * HW;
  for (int idx = tid; idx < ccn * kGP; idx += kBT) {
    const int c = idx / kGP, px = idx - (idx / kGP) * kGP;
    const int y = y0 + px / kGW, x = x0 + px % kGW;
    if (y < a.H && x < a.W) gx[static_cast<size_t>(c) * HW + y * a.W + x] = tile[c * GP + px];
  }
}

// C = sum over the reduction of A[m][k] * Bm[n][k]: both operands row-major with the
// reduction contiguous (rows padded with zeros to Kd, a multiple of 8).  The reduction
// runs over nseg segments of Kd (operand strides sAs, sBs), split evenly over ksplit
// workgroups per output tile; split ks writes its partial sum to C + ks * sCk (a later
// pass adds the partials in a fixed order).  blockIdx.z = zb * ksplit + ks, zb
// selecting independent problems (strides sAz, sBz, sCz).  A 128 x 128 output tile per
// workgroup, four waves of 64 x 64; chunks of 128 bytes of the reduction per row (64
// bf16 or 32 fp32 values) in two LDS buffers: while the waves multiply one, the next
// chunk goes from registers into the other and the one after is loaded into
// registers, one barrier per chunk.
template <typename T>
struct GemmArgs {
  const T* A;
  const T* Bm;
  void* C;       // fp32, or the element type with c_elem
  int M, N, Kd, lda, ldb, ldc, nseg, ksplit;
  int mfast;   // 1: output tiles in column-major order (M fastest)
  int c_elem;  // 1: C in the element type T (rounded once), else fp32
  long long sAs, sBs, sAz, sBz, sCz, sCk;
};

constexpr int kGM = 128, kGN = 128;
constexpr int kGKB = 128;   // bytes of the reduction per tile row and chunk

template <typename T>
__global__ __launch_bounds__(256) void bwd_gemm_nt(GemmArgs<T> g) {
  constexpr bool kBF = sizeof(T) == 2;
  constexpr int GK = kGKB / static_cast<int>(sizeof(T));  // reduction depth of a chunk
  constexpr int VE = 16 / static_cast<int>(sizeof(T));    // elements per 16-byte vector
  constexpr int VPR = GK / VE;                            // vectors per tile row (8)
  constexpr int NV = kGM * VPR / 256;                     // vectors per thread and operand (4)
  constexpr int LDT = GK + VE;                            // LDS row stride: 144 bytes
  __shared__ __attribute__((aligned(16))) T As[2][kGM * LDT];
  __shared__ __attribute__((aligned(16))) T Bs[2][kGN * LDT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lh = lane >> 5, wm = wave >> 1, wn = wave & 1;
  // Output tiles in row-major order (N fastest; M fastest with mfast), handed out so that
  // each XCD (workgroup w runs on XCD w % 8, each with its own L2) takes a contiguous run
  // of tiles, which share their A rows (B rows with mfast) in that L2.
  const int ntn = (g.N + kGN - 1) / kGN, ntm = (g.M + kGM - 1) / kGM, ntiles = ntn * ntm;
  const int xper = (ntiles + 7) / 8;
  const int lt = static_cast<int>(blockIdx.x % 8) * xper + static_cast<int>(blockIdx.x / 8);
  if (lt >= ntiles) return;   // spare workgroups of the last XCD (uniform)
  const int m0 = (g.mfast ? lt % ntm : lt / ntn) * kGM, n0 = (g.mfast ? lt / ntm : lt % ntn) * kGN;
  const int zb = blockIdx.z / g.ksplit, ks = blockIdx.z - zb * g.ksplit;
  const T* A = g.A + zb * g.sAz;
  const T* Bm = g.Bm + zb * g.sBz;
  const size_t c0 = zb * g.sCz + ks * g.sCk;
  const int kchunks = (g.Kd + GK - 1) / GK;
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
      const int idx = tid + v * 256, row = idx / VPR, k = kc * GK + (idx % VPR) * VE;
      const int ma = m0 + row, nb = n0 + row;
      ra[v] = (ma < g.M && k < g.Kd) ? *reinterpret_cast<const uint4*>(Ap + static_cast<size_t>(ma) * g.lda + k)
                                     : make_uint4(0, 0, 0, 0);
      rb[v] = (nb < g.N && k < g.Kd) ? *reinterpret_cast<const uint4*>(Bp + static_cast<size_t>(nb) * g.ldb + k)
                                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int idx = tid + v * 256, row = idx / VPR, kv = idx % VPR;
      *reinterpret_cast<uint4*>(&As[buf][row * LDT + kv * VE]) = ra[v];
      *reinterpret_cast<uint4*>(&Bs[buf][row * LDT + kv * VE]) = rb[v];
    }
  };
  auto mma = [&](int buf) {
    const T* as = As[buf];
    const T* bs = Bs[buf];
    if constexpr (kBF) {
#pragma unroll
      for (int h = 0; h < GK / 16; ++h) {
        bf16x8 av[2], bv[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          av[q] = *reinterpret_cast<const bf16x8*>(as + (wm * 64 + q * 32 + l32) * LDT + h * 16 + lh * 8);
          bv[q] = *reinterpret_cast<const bf16x8*>(bs + (wn * 64 + q * 32 + l32) * LDT + h * 16 + lh * 8);
        }
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
          for (int tn = 0; tn < 2; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[tm], bv[tn], acc[tm][tn], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < GK / 2; ++kk) {
        float av[2], bv[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          av[q] = as[(wm * 64 + q * 32 + l32) * LDT + 2 * kk + lh];
          bv[q] = bs[(wn * 64 + q * 32 + l32) * LDT + 2 * kk + lh];
        }
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
          for (int tn = 0; tn < 2; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[tm], bv[tn], acc[tm][tn], 0, 0, 0);
      }
    }
  };
  if (t0 < t1) {
    gload(t0);
    sstore(0);
    if (t0 + 1 < t1) gload(t0 + 1);
  }
  lds_barrier();
  for (int t = t0; t < t1; ++t) {
    const int cur = (t - t0) & 1;
    mma(cur);
    if (t + 1 < t1) {
      sstore(cur ^ 1);   // no wave still reads this buffer: all passed the last barrier
      if (t + 2 < t1) gload(t + 2);
    }
    lds_barrier();
  }
  // accumulator element r of a 32x32 block: row 8*(r/4) + 4*lh + r%4, column l32 (an
  // empty split writes zeros)
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + tm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int cc = n0 + wn * 64 + tn * 32 + l32;
        if (row < g.M && cc < g.N) {
          const size_t e = c0 + static_cast<size_t>(row) * g.ldc + cc;
          if (g.c_elem) static_cast<T*>(g.C)[e] = from_f<T>(acc[tm][tn][r]);
          else static_cast<float*>(g.C)[e] = acc[tm][tn][r];
        }
      }
}

// bf16 operands: the same product with the chunks moved by buffer->LDS loads straight
// into a ring of kDS LDS stages, three chunks ahead of the multiply and no registers
// held for them.  A chunk is 32 values (64 bytes) of the reduction for the tile's 128
// rows of each operand; lane s of a 1 KB load fills 16-byte slot s of a 16-row block,
// and the slots of a row are XOR-swizzled with (row / 4) % 4, so that the multiply's
// 16-byte reads of 16 rows at one reduction offset fall in distinct banks.  Rows past
// M or N and reduction indices past Kd read zeros (the load's offset is past the
// buffer).  With c_elem the tile leaves through LDS as 16-byte row pieces.
constexpr int kDK = 32;   // reduction values per chunk
constexpr int kDS = 4;    // LDS stages
constexpr int kDRB = kDK * 2;   // bytes of a row in a chunk
constexpr uint32_t kDOOB = 0xfffffff0u;   // a byte offset past every operand (operands < 2 GiB)

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// a barrier after this wave's LDS operations completed (the direct loads into LDS are
// waited for separately with wait_vm)
__device__ __forceinline__ void barrier_lds_done() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ __launch_bounds__(256) void bwd_gemm_dma(GemmArgs<uint16_t> g, uint32_t a_bytes, uint32_t b_bytes) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kDS][2][kGM * kDRB];   // [stage][A, B][row][128 B]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lh = lane >> 5, wm = wave >> 1, wn = wave & 1;
  const int ntn = (g.N + kGN - 1) / kGN, ntm = (g.M + kGM - 1) / kGM, ntiles = ntn * ntm;
  const int xper = (ntiles + 7) / 8;
  const int lt = static_cast<int>(blockIdx.x % 8) * xper + static_cast<int>(blockIdx.x / 8);
  if (lt >= ntiles) return;   // spare workgroups of the last XCD (uniform)
  const int m0 = (g.mfast ? lt % ntm : lt / ntn) * kGM, n0 = (g.mfast ? lt / ntm : lt % ntn) * kGN;
  const int zb = blockIdx.z / g.ksplit, ks = blockIdx.z - zb * g.ksplit;
  const __amdgpu_buffer_rsrc_t ra = gemm_rsrc(g.A + zb * g.sAz, a_bytes);
  const __amdgpu_buffer_rsrc_t rb = gemm_rsrc(g.Bm + zb * g.sBz, b_bytes);
  const int kchunks = (g.Kd + kDK - 1) / kDK;
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
  // this lane's slot in a 16-row block: row s / 4, physical piece s % 4
  const int srow = lane >> 2, sphys = lane & 3;
  // chunk t into stage st: four 1 KB loads per wave (two 16-row blocks of each operand)
  auto issue = [&](int t, int st) {
    const int seg = t / kchunks, kc = t - seg * kchunks;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = wave * 2 + i, row = blk * 16 + srow;
      const int k = kc * kDK + (sphys ^ ((row >> 2) & 3)) * 8;
      const int ma = m0 + row, nb = n0 + row;
      const uint32_t va = ma < g.M && k < g.Kd
                              ? static_cast<uint32_t>((seg * g.sAs + static_cast<long long>(ma) * g.lda + k) * 2)
                              : kDOOB;
      const uint32_t vb = nb < g.N && k < g.Kd
                              ? static_cast<uint32_t>((seg * g.sBs + static_cast<long long>(nb) * g.ldb + k) * 2)
                              : kDOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(smem[st][0] + blk * 1024), 16, va, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(smem[st][1] + blk * 1024), 16, vb, 0, 0, 0);
    }
  };
  auto mma = [&](int st) {
    const unsigned char* as = smem[st][0];
    const unsigned char* bs = smem[st][1];
#pragma unroll
    for (int h = 0; h < kDK / 16; ++h) {
      const int kv = 2 * h + lh;
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int ra_ = wm * 64 + q * 32 + l32, rb_ = wn * 64 + q * 32 + l32;
        av[q] = *reinterpret_cast<const bf16x8*>(as + ra_ * kDRB + ((kv ^ ((ra_ >> 2) & 3)) << 4));
        bv[q] = *reinterpret_cast<const bf16x8*>(bs + rb_ * kDRB + ((kv ^ ((rb_ >> 2) & 3)) << 4));
      }
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[tm], bv[tn], acc[tm][tn], 0, 0, 0);
    }
  };
#pragma unroll
  for (int j = 0; j < kDS - 1; ++j)
    if (t0 + j < t1) issue(t0 + j, j);
  for (int t = t0; t < t1; ++t) {
    // this wave's loads of chunk t are done when at most (chunks issued after t) x 4 remain
    static_assert(kDS == 4, "the wait below allows two chunks after t");
    const int after = min(t1 - 1 - t, kDS - 2);
    if (after >= 2) wait_vm<8>();
    else if (after == 1) wait_vm<4>();
    else wait_vm<0>();
    barrier_lds_done();   // every wave's chunk t is in LDS; stage (t - 1) % kDS is free
    if (t + kDS - 1 < t1) issue(t + kDS - 1, (t + kDS - 1 - t0) % kDS);
    mma((t - t0) % kDS);
  }
  // accumulator element r of a 32x32 block: row 8*(r/4) + 4*lh + r%4, column l32
  const size_t c0 = zb * g.sCz + ks * g.sCk;
  if (!g.c_elem || g.ldc % 8 != 0) {
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 64 + tm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          const int cc = n0 + wn * 64 + tn * 32 + l32;
          if (row < g.M && cc < g.N) {
            const size_t e = c0 + static_cast<size_t>(row) * g.ldc + cc;
            if (g.c_elem) static_cast<uint16_t*>(g.C)[e] = from_f<uint16_t>(acc[tm][tn][r]);
            else static_cast<float*>(g.C)[e] = acc[tm][tn][r];
          }
        }
    return;
  }
  // through LDS: the tile as bf16 [128][136], then 16-byte pieces of rows
  uint16_t* ct = reinterpret_cast<uint16_t*>(&smem[0][0][0]);
  constexpr int CP = kGN + 8;
  wait_vm<0>();
  barrier_lds_done();
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + tm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        ct[row * CP + wn * 64 + tn * 32 + l32] = from_f<uint16_t>(acc[tm][tn][r]);
      }
  barrier_lds_done();
  uint16_t* C = static_cast<uint16_t*>(g.C) + c0;
#pragma unroll
  for (int i = 0; i < kGM * kGN / 8 / 256; ++i) {
    const int idx = tid + i * 256, row = idx >> 4, pc = (idx & 15) * 8;
    const int gr = m0 + row, gc = n0 + pc;
    if (gr >= g.M || gc >= g.N) continue;
    if (gc + 8 <= g.N) {
      *reinterpret_cast<uint4*>(C + static_cast<size_t>(gr) * g.ldc + gc) = *reinterpret_cast<const uint4*>(ct + row * CP + pc);
    } else {
      for (int j = 0; j < g.N - gc; ++j) C[static_cast<size_t>(gr) * g.ldc + gc + j] = ct[row * CP + pc + j];
    }
  }
}

// The weight gradient's partial sums added in split order and rounded to the element
// type; the bias accumulator converted by the threads past the weight's elements.
template <typename T>
__global__ __launch_bounds__(kBT) void bwd_reduce_w(const float* part, int nsplit, int n, T* out, const float* gb32,
                                                    T* gbo, int nb) {
  const int e = blockIdx.x * kBT + threadIdx.x;
  if (e < n) {
    if (out == nullptr) return;
    float s = part[e];
    for (int k = 1; k < nsplit; ++k) s += part[static_cast<size_t>(k) * n + e];
    out[e] = from_f<T>(s);
  } else if (e - n < nb && gbo != nullptr) {
    gbo[e - n] = from_f<T>(gb32[e - n]);
  }
}

int64_t rup(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Workspace layout of one backward call.
struct BwdPlan {
  int64_t Ho = 0, Wo = 0, P = 0, Pp = 0, Coutp = 0, R = 0, G = 1, Cp = 0, ncnt = 0, nblk = 0, nsamp = 0;
  int wks = 1;   // splits of the weight gradient's reduction (partial sums in the workspace)
  size_t o_wt = 0, o_gyt = 0, o_gyp = 0, o_col = 0, o_gcol = 0, o_xs = 0, o_gw = 0, o_gb = 0;
  size_t o_cnt = 0, o_bsum = 0, o_cur = 0, o_pairs = 0;
  size_t bytes = 0;
};

int bwd_plan(const dcn_desc* d, BwdPlan* p) {
  int rc = check_desc(d, &p->Ho, &p->Wo);
  if (rc != DCN_OK) return rc;
  const int64_t B = d->batch, Cin = d->in_channels, Cout = d->out_channels, KK = d->kernel_size * d->kernel_size;
  const int64_t HW = d->height * d->width;
  p->G = d->offset_groups > 1 ? d->offset_groups : 1;
  p->P = p->Ho * p->Wo;
  p->Pp = rup(p->P, 8);
  p->Coutp = rup(Cout > 0 ? Cout : 1, 8);
  p->R = Cin * KK;
  p->Cp = rup(Cin, 8);
  p->nsamp = B * p->G * KK * p->P;
  p->ncnt = B * p->G * HW + 1;
  p->nblk = (p->ncnt + kScanB - 1) / kScanB;
  const double lim = 2147483647.0;
  const double Bd = static_cast<double>(B);
  if (Bd * p->R * p->Pp > lim || Bd * Cin * HW > lim || Bd * p->Coutp * p->Pp > lim ||
      static_cast<double>(p->R) * p->Coutp > lim || Bd * 2 * p->G * KK * p->P > lim ||
      static_cast<double>(Cout) * p->R > lim || Bd * HW * p->Cp > lim || 4.0 * p->nsamp > lim ||
      static_cast<double>(p->ncnt) > lim)
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
  p->o_gcol = take(static_cast<size_t>(B * p->P * p->R) * es);
  p->o_xs = take(static_cast<size_t>(B * HW * p->Cp) * es);
  // split the weight gradient's reduction (B segments of Pp) until the output tiles and
  // splits give about one workgroup per CU, with at least four chunks per split
  {
    const int64_t tiles = ((Cout + kGM - 1) / kGM) * ((p->R + kGN - 1) / kGN);
    const int64_t chunks = (p->Pp + kGKB / static_cast<int64_t>(es) - 1) / (kGKB / static_cast<int64_t>(es)) * B;
    while (tiles * p->wks < 256 && p->wks * 2 <= chunks / 4) p->wks *= 2;
  }
  p->o_gw = take(static_cast<size_t>(Cout * p->R) * 4 * p->wks);
  p->o_gb = take(static_cast<size_t>(Cout) * 4);
  p->o_cnt = take(static_cast<size_t>(p->ncnt) * 4);
  p->o_bsum = take(static_cast<size_t>(p->nblk) * 4);
  p->o_cur = take(static_cast<size_t>(p->ncnt) * 4);
  p->o_pairs = take(static_cast<size_t>(p->nsamp) * 4 * 8);
  p->bytes = o;
  return DCN_OK;
}

hipError_t launch1(const void* fn, int64_t n, void** args, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>((n + kBT - 1) / kBT)), dim3(kBT), args, 0, s);
}

// ranges[i] = (fp32 buffer, elements) to zero, four floats per thread; null buffers
// are skipped.  Returns the workgroups the ranges take.
int make_ranges(Ranges* r, std::initializer_list<std::tuple<float*, int64_t>> list) {
  *r = Ranges{};
  int total = 0;
  for (const auto& t : list) {
    if (std::get<0>(t) == nullptr || std::get<1>(t) <= 0) continue;
    r->p[r->count] = std::get<0>(t);
    r->n[r->count] = static_cast<int>(std::get<1>(t));
    r->blocks[r->count] = static_cast<int>((std::get<1>(t) + kBT * 4 - 1) / (kBT * 4));
    total += r->blocks[r->count];
    ++r->count;
  }
  return total;
}

// bf16 products with a short reduction per workgroup (at most 256 values: the column
// gradients' 256 output channels on c4) whose operands are under 2 GiB take the LDS-ring
// kernel (a_bytes and b_bytes: the extent of A and Bm over the segments); the others,
// whose long reductions the register-staged kernel's 128-byte chunks run through with
// half the barriers, take that one (c4: column gradients 31 -> 26 us on the ring, the
// weight gradient 28 -> 36 us).
template <typename T>
hipError_t gemm(const GemmArgs<T>& g, int zb, hipStream_t s) {
  GemmArgs<T> gg = g;
  const int ntiles = ((g.N + kGN - 1) / kGN) * ((g.M + kGM - 1) / kGM);
  const dim3 grid(static_cast<unsigned>((ntiles + 7) / 8 * 8), 1, static_cast<unsigned>(zb * g.ksplit));
  const double ab = 2.0 * ((g.nseg - 1) * static_cast<double>(g.sAs) + static_cast<double>(g.M) * g.lda);
  const double bb = 2.0 * ((g.nseg - 1) * static_cast<double>(g.sBs) + static_cast<double>(g.N) * g.ldb);
  const int per_split = (g.nseg * ((g.Kd + 31) / 32) + g.ksplit - 1) / g.ksplit;   // 32-value chunks
  if (sizeof(T) == 2 && per_split <= 8 && ab < 2147483648.0 && bb < 2147483648.0) {
    uint32_t a_bytes = static_cast<uint32_t>(ab), b_bytes = static_cast<uint32_t>(bb);
    void* args[] = {&gg, &a_bytes, &b_bytes};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_gemm_dma), grid, dim3(256), args, 0, s);
  }
  void* args[] = {&gg};
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
  constexpr bool kBF16 = sizeof(T) == 2;
  BwdArgs a{};
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
  a.Cp = static_cast<int>(p.Cp);
  a.nsamp = static_cast<int>(p.nsamp);
  // lanes per sample or pixel: eight channels each, enough for a chunk (kCC = 32 * 8)
  const int cch = std::min(a.Cg, kCC);
  a.lg = 1;
  while (a.lg < 32 && a.lg * 8 < cch) a.lg *= 2;
  a.npb = (a.P + kSP - 1) / kSP;
  a.nqy = (a.H + kGH - 1) / kGH;
  a.nqx = (a.W + kGW - 1) / kGW;
  a.ncc = (a.Cg + kCC - 1) / kCC;
  const bool need_gcol = grad_x != nullptr || grad_offset != nullptr || (grad_mask != nullptr && mask != nullptr);
  const bool sample = need_gcol || grad_weight != nullptr;
  a.xs = ws + p.o_xs;
  a.wt = ws + p.o_wt;
  a.gyt = need_gcol ? static_cast<void*>(ws + p.o_gyt) : nullptr;
  // grad_out with its pixel stride padded to Pp: grad_out itself when P is a multiple of 8
  a.gyp_copy = a.Pp > a.P ? 1 : 0;
  a.gyp = grad_weight == nullptr ? nullptr : a.gyp_copy ? static_cast<void*>(ws + p.o_gyp) : const_cast<void*>(grad_out);
  a.col = grad_weight != nullptr ? static_cast<void*>(ws + p.o_col) : nullptr;
  a.gcol = need_gcol ? static_cast<void*>(ws + p.o_gcol) : nullptr;
  a.gb32 = grad_bias != nullptr ? reinterpret_cast<float*>(ws + p.o_gb) : nullptr;
  a.grad_offset = grad_offset;
  a.grad_mask = mask != nullptr ? grad_mask : nullptr;
  a.grad_x = grad_x;
  if (grad_x != nullptr) {
    a.cnt = reinterpret_cast<int*>(ws + p.o_cnt);
    a.bsum = reinterpret_cast<int*>(ws + p.o_bsum);
    a.cur = reinterpret_cast<int*>(ws + p.o_cur);
    a.pairs = reinterpret_cast<int2*>(ws + p.o_pairs);
  }
  float* gw32 = reinterpret_cast<float*>(ws + p.o_gw);   // [wks][Cout][R] partial sums
  const int64_t nw = static_cast<int64_t>(a.Cout) * a.R;
  void* args[] = {&a};

  if (sample) {   // x channels last, with the forward's staging kernel (no weight to repack)
    StageArgs sa{};
    sa.x = x;
    sa.xs = ws + p.o_xs;
    sa.B = a.B;
    sa.Cin = a.Cin;
    sa.HW = a.H * a.W;
    sa.Cp = a.Cp;
    sa.KK = 1;
    BWD_TRY(launch_stage(kBF16 ? V_TILE_BF16_M64_N64 : V_TILE_F32_M64_N64, sa, s));
  }
  {
    // the weight transpose and the zero fill (bias accumulator, pair counters: before the
    // bias sums and the count), then the grad_out transposes and the pair count
    PrepLaunch L{};
    L.a = a;
    if (need_gcol) {
      L.wx = (a.R + 31) / 32;
      L.wy = (a.Coutp + 31) / 32;
    }
    const int nfill = make_ranges(&L.r, {{a.gb32, a.Cout}, {reinterpret_cast<float*>(a.cnt), p.ncnt}});
    const int n1 = L.wx * L.wy + nfill;
    void* largs[] = {&L};
    if (n1 > 0)
      BWD_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&bwd_prep_1<T>), dim3(n1), dim3(kBT), largs, 0, s));
    if (sample || grad_bias != nullptr) {
      L.gx = (a.Pp + kGT - 1) / kGT;
      L.gy = (a.Coutp + kGT - 1) / kGT;
      L.gz = a.B;
      L.gy_vec = a.P % (16 / static_cast<int>(sizeof(T))) == 0 && reinterpret_cast<uintptr_t>(grad_out) % 16 == 0;
    }
    const int ncount = grad_x != nullptr ? (a.nsamp + kBT - 1) / kBT : 0;
    const int n2 = L.gx * L.gy * L.gz + ncount;
    if (n2 > 0)
      BWD_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&bwd_prep_2<T>), dim3(n2), dim3(kBT), largs, 0, s));
  }
  if (grad_x != nullptr) {
    int n = static_cast<int>(p.ncnt), nb = static_cast<int>(p.nblk);
    void* s1[] = {&a.cnt, &n, &a.bsum, &a.cur};
    BWD_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&bwd_scan_blocks), dim3(nb), dim3(kBT), s1, 0, s));
    void* s2[] = {&a.bsum, &nb};
    BWD_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&bwd_scan_top), dim3(1), dim3(kBT), s2, 0, s));
  }
  if (need_gcol) {   // gcol[b][p][r'] = sum_o gyT[b][p][o] * Wt[r'][o], r' = k*Cin + c
    GemmArgs<T> g{};
    g.A = static_cast<const T*>(a.gyt);
    g.Bm = static_cast<const T*>(a.wt);
    g.C = a.gcol;
    g.c_elem = 1;
    g.M = a.P;
    g.N = a.R;
    g.Kd = a.Coutp;
    g.lda = g.ldb = a.Coutp;
    g.ldc = a.R;
    g.nseg = 1;
    g.ksplit = 1;
    g.sAz = static_cast<long long>(a.P) * a.Coutp;
    g.sBz = 0;
    g.sCz = static_cast<long long>(a.P) * a.R;
    BWD_TRY(gemm<T>(g, a.B, s));
  }
  if (sample) {
    const unsigned grid = static_cast<unsigned>(a.B * a.G * a.npb * a.KK);
    BWD_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&bwd_sample_cl<T>), dim3(grid), dim3(kBT), args, 0, s));
  }
  if (grad_x != nullptr) {
    const unsigned grid = static_cast<unsigned>(a.B * a.G * a.ncc * a.nqy * a.nqx);
    BWD_TRY(hipLaunchKernel(reinterpret_cast<const void*>(&bwd_gather_cl<T>), dim3(grid), dim3(kBT), args, 0, s));
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
    g.ksplit = p.wks;
    g.sCk = nw;
    g.mfast = 1;   // the tiles of one column block (all output channels) share its col rows
    BWD_TRY(gemm<T>(g, 1, s));
  }
  // the weight gradient's partial sums added and the bias accumulator converted, one launch
  if (grad_weight != nullptr || grad_bias != nullptr) {
    const float* part = gw32;
    int nsplit = p.wks, n = grad_weight != nullptr ? static_cast<int>(nw) : 0, nb = grad_bias != nullptr ? a.Cout : 0;
    T* out = static_cast<T*>(grad_weight);
    T* gbo = static_cast<T*>(grad_bias);
    const float* gb = a.gb32;
    void* rargs[] = {&part, &nsplit, &n, &out, &gb, &gbo, &nb};
    BWD_TRY(launch1(reinterpret_cast<const void*>(&bwd_reduce_w<T>), static_cast<int64_t>(n) + nb, rargs, s));
  }
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
