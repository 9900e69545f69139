// dcn_kernels.hip -- gfx950 kernels of the deformable convolution forward.
//
// Two launches per call:
//   stage_x / pack_w : x from [B][Cin][H][W] to channels-last [B][H][W][Cp] and the
//                      weight from [Cout][Cin][K][K] to [Mp][K^2][Cp] (zero padding up
//                      to Cp channels and Mp rows), so that the samples of one kernel
//                      point form a contiguous reduction run of Cp channels;
//   dcn_fused        : one workgroup per (MT output channels) x (NT output pixels)
//                      tile.  For each reduction chunk (kernel point k, CK channels):
//                      the sampling positions and bilinear corner weights of
//                      (pixel, k) times the mask (computed once per k, kept in
//                      registers), coalesced 16-byte gathers of the four corner
//                      channel vectors from the channels-last copy, fp32
//                      interpolation, rounding to the element type, a column tile
//                      in LDS; MFMA against the weight tile; fp32 accumulators; bias
//                      added in the epilogue and the result stored as [B][Cout][Ho][Wo].
//
// The computation follows the deformable-convolution equation (csdn.net tags page
// "可变形卷积：Deformable ConvNets", part "Deformable Convolutional Networks",
// section on deformable convolution), with the modulation scalar of DCNv2 (same
// page, section 3.2) and bilinear interpolation from the four integer neighbours
// (same page, bilinear-interpolation equation).  The im2col -> GEMM -> reduce
// split of a convolution (same page, supplement on im2col) is realised with the
// column matrix kept in LDS only: it never goes to HBM.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dcn_internal.h"

namespace dcn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // four wave64 per workgroup

// ---------------------------------------------------------------------------
// element helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

template <bool BF16>
__device__ __forceinline__ float load_scalar(const void* p, int idx) {
  if constexpr (BF16) {
    const uint16_t v = reinterpret_cast<const uint16_t*>(p)[idx];
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  } else {
    return reinterpret_cast<const float*>(p)[idx];
  }
}

template <bool BF16>
__device__ __forceinline__ void store_scalar(void* p, int idx, float v) {
  if constexpr (BF16) {
    reinterpret_cast<uint16_t*>(p)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  } else {
    reinterpret_cast<float*>(p)[idx] = v;
  }
}

// Workgroup id -> tile id, so that consecutive tiles run on the same XCD.
// Workgroups are dealt to the 8 XCDs round-robin in id order; this gives XCD x
// the contiguous tile range [x*q + min(x,r), ... + q + (x<r)) of T = 8q + r
// tiles.  It is a bijection on [0, T) for any T.
__device__ __forceinline__ int xcd_tile(int g, int T) {
  const int xcd = g & 7, idx = g >> 3;
  const int q = T >> 3, r = T & 7;
  return xcd * q + min(xcd, r) + idx;
}

// ---------------------------------------------------------------------------
// staging
// ---------------------------------------------------------------------------

// Weight repack, one thread per (row o, channel c): the K*K values of (o, c) are
// contiguous in w, and for each kernel point neighbouring threads write neighbouring
// channels.  Layout 0: wp[o][k][c]; layout 1 (box kernel): wp[c/32 * KK + k][o][c%32];
// layout 2 (offset/mask convolution): wp[(k * Cp + c) / 16][o][c%16].
// Rows >= Cout and channels >= Cin are written as 0.
template <typename T>
__device__ __forceinline__ void pack_weight(const StageArgs& a, int wg, int nwg) {
  // the two do not overlap (the workspace is the caller's scratch), so every load of
  // a row can be issued before its stores
  const T* __restrict__ w = reinterpret_cast<const T*>(a.w);
  T* __restrict__ wp = reinterpret_cast<T*>(a.wp);
  const int total = a.Mp * a.Cp;
  for (int e = wg * kThreads + static_cast<int>(threadIdx.x); e < total; e += nwg * kThreads) {
    const int o = e / a.Cp, c = e - (e / a.Cp) * a.Cp;
    const bool live = o < a.Cout && c < a.Cin;
    const T* src = w + (static_cast<size_t>(o) * a.Cin + c) * a.KK;
    // nine kernel points at a time: all loads in flight before the stores
    for (int k0 = 0; k0 < a.KK; k0 += 9) {
      T v[9];
#pragma unroll
      for (int j = 0; j < 9; ++j) v[j] = (live && k0 + j < a.KK) ? src[k0 + j] : T(0);
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        const int k = k0 + j;
        if (k >= a.KK) break;
        const size_t dst = a.wlayout == 0 ? (static_cast<size_t>(o) * a.KK + k) * a.Cp + c
                           : a.wlayout == 1
                               ? ((static_cast<size_t>(c >> 5) * a.KK + k) * a.Mp + o) * 32 + (c & 31)
                               : ((static_cast<size_t>(k) * (a.Cp >> 4) + (c >> 4)) * a.Mp + o) * 16 + (c & 15);
        wp[dst] = v[j];
      }
    }
  }
}

// The step-major weight layout from bf16 with Cin a multiple of 8 and a 16-byte aligned
// w: one thread per (row o, 8 channels), whose 8*K*K values are contiguous in w
// (nine 16-byte loads for 3x3); for each kernel point the 8 channels' values are
// gathered into one 16-byte store.
__device__ __forceinline__ bool pack_weight_v8_ok(const StageArgs& a) {
  return a.wlayout == 1 && a.KK == 9 && a.Cin % 8 == 0 && reinterpret_cast<uintptr_t>(a.w) % 16 == 0;
}
__device__ __forceinline__ void pack_weight_v8(const StageArgs& a, int wg, int nwg) {
  const uint4* w = reinterpret_cast<const uint4*>(a.w);
  uint4* wp = reinterpret_cast<uint4*>(a.wp);
  const int groups = a.Cp / 8, total = a.Mp * groups;
  for (int e = wg * kThreads + static_cast<int>(threadIdx.x); e < total; e += nwg * kThreads) {
    const int o = e / groups, c = (e - (e / groups) * groups) * 8;
    uint32_t d[36];   // 72 bf16: channel i, kernel point k at element 9i + k
    if (o < a.Cout && c < a.Cin) {
      const uint4* src = w + (static_cast<size_t>(o) * a.Cin + c) * 9 / 8;
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        const uint4 q = src[j];
        d[4 * j] = q.x; d[4 * j + 1] = q.y; d[4 * j + 2] = q.z; d[4 * j + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 36; ++j) d[j] = 0;
    }
    uint4* dst = wp + ((static_cast<size_t>(c >> 5) * 9) * a.Mp + o) * 4 + ((c & 31) >> 3);
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      uint32_t r[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int e0 = 18 * m + k, e1 = e0 + 9;   // channels 2m and 2m+1
        // byte selectors of v_perm: 0-3 pick from the second operand, 4-7 from the first
        const uint32_t s0 = (e0 & 1) ? 0x0302u : 0x0100u, s1 = (e1 & 1) ? 0x0706u : 0x0504u;
        r[m] = __builtin_amdgcn_perm(d[e1 >> 1], d[e0 >> 1], (s1 << 16) | s0);
      }
      dst[static_cast<size_t>(k) * a.Mp * 4] = make_uint4(r[0], r[1], r[2], r[3]);
    }
  }
}

// One launch stages both operands of the fused kernel.
//   Workgroups [0, nw):  w[o][c][k] -> wp[o][k][c] (or the step-major layout of the
//                        box kernel) for o < Mp, k < KK, c < Cp, zero outside
//                        Cout x Cin.
//   Workgroups [nw, ..): x[b][c][s] -> xs[b][s][c] for s in [0, H*W), c in [0, Cp),
//                        channels >= Cin written as 0.  Each moves a 64-channel x
//                        64-pixel tile (128 pixels for bf16 with 16-byte reads)
//                        through LDS: global reads are VEC pixels of one channel
//                        (VEC = 16 bytes' worth when H*W allows the alignment, fewer
//                        otherwise), global writes are 16-byte channel vectors of one
//                        pixel.
// bf16 with 16-byte reads (H*W a multiple of 8): the transpose goes through LDS as
// channel pairs.  Thread (channel pair cp, pixel group pg) reads 8 pixels of channels
// 2cp and 2cp+1 (eight lanes cover 128 contiguous bytes of one channel), packs each
// pixel's two channels into one dword and writes the eight dwords to tile[p][cp].
// The 16-byte group of 4 channel pairs is XOR-swizzled with the pixel group, so the
// dword writes of a wave and the 16-byte reads of one pixel's 8 channels both hit
// distinct banks; a thread then writes 8 channels of one pixel as one 16-byte store
// (eight lanes cover the 128 bytes of the tile's 64 channels of that pixel).
constexpr int kPairPx = 128;   // pixels per tile of the channel-pair transpose
__device__ __forceinline__ void stage_x_bf16_v8(const StageArgs& a, uint32_t* tile, int b, int s0, int c0) {
  const int tid = threadIdx.x;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(a.x) + static_cast<size_t>(b) * a.Cin * a.HW;
  uint16_t* xs = reinterpret_cast<uint16_t*>(a.xs) + static_cast<size_t>(b) * a.HW * a.Cp;
#pragma unroll
  for (int u = 0; u < kPairPx / 64; ++u) {
    const int pg = (tid & 7) + 8 * u, cp = tid >> 3;
    const int c = c0 + 2 * cp, sp = s0 + 8 * pg;
    uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
    if (sp < a.HW) {   // H*W is a multiple of 8: the vector is all in or all out
      const uint16_t* src = x + static_cast<size_t>(c) * a.HW + sp;
      if (c < a.Cin) lo = *reinterpret_cast<const uint4*>(src);
      if (c + 1 < a.Cin) hi = *reinterpret_cast<const uint4*>(src + a.HW);
    }
    const uint32_t l[4] = {lo.x, lo.y, lo.z, lo.w}, h[4] = {hi.x, hi.y, hi.z, hi.w};
    uint32_t* t = tile + (8 * pg) * 32 + (((cp >> 2) ^ (pg & 7)) << 2) + (cp & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t[(2 * i) * 32] = __builtin_amdgcn_perm(h[i], l[i], 0x05040100u);      // pixel 2i
      t[(2 * i + 1) * 32] = __builtin_amdgcn_perm(h[i], l[i], 0x07060302u);  // pixel 2i+1
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPairPx / 32; ++j) {
    const int g = tid & 7, p = (tid >> 3) + 32 * j;
    const int sp = s0 + p, c = c0 + 8 * g;
    if (sp >= a.HW || c >= a.Cp) continue;
    const uint4 q = *reinterpret_cast<const uint4*>(tile + p * 32 + ((g ^ ((p >> 3) & 7)) << 2));
    *reinterpret_cast<uint4*>(xs + static_cast<size_t>(sp) * a.Cp + c) = q;
  }
}

template <bool BF16, int VEC>
__global__ __launch_bounds__(kThreads) void stage_kernel(StageArgs a, int nx, int s_tiles, int c_tiles) {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  constexpr int ES = sizeof(T);
  constexpr int OUTV = 16 / ES;                  // elements per 16-byte channel vector
  constexpr bool kPairs = BF16 && VEC == 8;
  __shared__ __attribute__((aligned(16))) T tile[64][kPairs ? kPairPx : 64 + 2];   // [channel][pixel]
  const int tid = threadIdx.x;
  // the weight workgroups come first, so that they run beside the first x tiles
  // rather than after the last
  const int nw2 = a.w2 != nullptr ? a.nw2 : 0;
  const int nw = static_cast<int>(gridDim.x) - nx - nw2;
  if (nw2 > 0 && static_cast<int>(blockIdx.x) >= nw && static_cast<int>(blockIdx.x) < nw + nw2) {
    // the second weight
    StageArgs a2 = a;
    a2.w = a.w2;
    a2.wp = a.wp2;
    a2.Cout = a.Cout2;
    a2.Mp = a.Mp2;
    a2.wlayout = a.wlayout2;
    if constexpr (BF16) {
      if (pack_weight_v8_ok(a2)) {
        pack_weight_v8(a2, static_cast<int>(blockIdx.x) - nw, nw2);
        return;
      }
    }
    pack_weight<T>(a2, static_cast<int>(blockIdx.x) - nw, nw2);
    return;
  }
  if (static_cast<int>(blockIdx.x) < nw) {
    if constexpr (BF16) {
      if (pack_weight_v8_ok(a)) {
        pack_weight_v8(a, static_cast<int>(blockIdx.x), nw);
        return;
      }
    }
    pack_weight<T>(a, static_cast<int>(blockIdx.x), nw);
    return;
  }
  // The x tiles run in (image, pixel block, channel block) order, channel blocks fastest,
  // and each XCD (workgroup g runs on XCD g % 8; the weight workgroups before them are
  // a multiple of 8) takes a contiguous run of them: a band of input rows of one image,
  // the band the fused kernel's workgroups on that XCD read (they take contiguous runs
  // of output tiles in the same raster order).
  const int bx = xcd_tile(static_cast<int>(blockIdx.x) - nw - nw2, nx);
  const int per_img = s_tiles * c_tiles;
  const int b = bx / per_img;
  const int r = bx - b * per_img;
  const int st = r / c_tiles, ct = r - (r / c_tiles) * c_tiles;
  const int s0 = st * (kPairs ? kPairPx : 64), c0 = ct * 64;
  if constexpr (kPairs) {
    stage_x_bf16_v8(a, reinterpret_cast<uint32_t*>(&tile[0][0]), b, s0, c0);
    return;
  }
  const T* x = reinterpret_cast<const T*>(a.x) + static_cast<size_t>(b) * a.Cin * a.HW;
  T* xs = reinterpret_cast<T*>(a.xs) + static_cast<size_t>(b) * a.HW * a.Cp;
  // read: 64 channels x (64 / VEC) vectors of VEC pixels
  for (int e = tid; e < 64 * (64 / VEC); e += kThreads) {
    const int cl = e / (64 / VEC), sv = e - (e / (64 / VEC)) * (64 / VEC);
    const int c = c0 + cl, sp = s0 + sv * VEC;
    T v[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = T(0);
    if (c < a.Cin) {
      const T* src = x + static_cast<size_t>(c) * a.HW + sp;
      if (sp + VEC <= a.HW) {
        if constexpr (VEC * ES == 16) {
          const uint4 q = *reinterpret_cast<const uint4*>(src);
          __builtin_memcpy(v, &q, 16);
        } else if constexpr (VEC * ES == 8) {
          const uint2 q = *reinterpret_cast<const uint2*>(src);
          __builtin_memcpy(v, &q, 8);
        } else if constexpr (VEC * ES == 4) {
          const uint32_t q = *reinterpret_cast<const uint32_t*>(src);
          __builtin_memcpy(v, &q, 4);
        } else {
#pragma unroll
          for (int i = 0; i < VEC; ++i) v[i] = src[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i)
          if (sp + i < a.HW) v[i] = src[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) tile[cl][sv * VEC + i] = v[i];
  }
  __syncthreads();
  // write: 64 pixels x (64 / OUTV) vectors of OUTV channels
  for (int e = tid; e < 64 * (64 / OUTV); e += kThreads) {
    const int sl = e / (64 / OUTV), cv = e - (e / (64 / OUTV)) * (64 / OUTV);
    const int sp = s0 + sl, c = c0 + cv * OUTV;
    if (sp >= a.HW || c >= a.Cp) continue;
    T v[OUTV];
#pragma unroll
    for (int i = 0; i < OUTV; ++i) v[i] = tile[cv * OUTV + i][sl];
    uint4 q;
    __builtin_memcpy(&q, v, 16);
    *reinterpret_cast<uint4*>(xs + static_cast<size_t>(sp) * a.Cp + c) = q;
  }
}

// ---------------------------------------------------------------------------
// fused deformable im2col + MFMA + bias
// ---------------------------------------------------------------------------

template <bool BF16, int MT, int NT>
struct TileCfg {
  static constexpr int ES = BF16 ? 2 : 4;          // element bytes
  static constexpr int CK = 32;                     // channels per reduction chunk
  static constexpr int VEC = 16 / ES;               // elements per 16-byte unit
  static constexpr int UPR = CK / VEC;              // 16-byte units per tile row
  static constexpr int ROWB = CK * ES + 16;         // LDS row stride in bytes (padded)
  static constexpr int G_UNITS = NT * UPR;          // column-tile units per chunk
  static constexpr int GU = (G_UNITS + kThreads - 1) / kThreads;
  static constexpr int A_UNITS = MT * UPR;          // weight-tile units per chunk
  static constexpr int AU = (A_UNITS + kThreads - 1) / kThreads;
  static constexpr int WAVES_M = 2, WAVES_N = 2;
  static constexpr int WM = MT / WAVES_M, WN = NT / WAVES_N;
  static constexpr int FM = WM / 16, FN = WN / 16;  // 16x16 MFMA fragments per wave
  static constexpr int BUF_BYTES = (MT + NT) * ROWB;
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
};

template <bool BF16, int MT, int NT>
__global__ __launch_bounds__(kThreads) void dcn_fused_kernel(FusedArgs a) {
  using C = TileCfg<BF16, MT, NT>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][C::BUF_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.m_tiles * a.n_tiles;
  const int t = xcd_tile(blockIdx.x, T);
  const int m0 = (t % a.m_tiles) * MT;
  const int n0 = (t / a.m_tiles) * NT;
  const int KK = a.KK, Cp = a.Cp;
  const int cch = Cp / C::CK;          // channel chunks per kernel point
  const int nq = KK * cch;             // reduction chunks

  const unsigned char* xs = reinterpret_cast<const unsigned char*>(a.xs);
  const unsigned char* wp = reinterpret_cast<const unsigned char*>(a.wp);

  // --- gather units owned by this thread: (pixel of the tile, 16-byte sub-block)
  int g_pl[C::GU], g_sub[C::GU], g_b[C::GU], g_oy[C::GU], g_ox[C::GU], g_rem[C::GU];
  bool g_on[C::GU];
#pragma unroll
  for (int u = 0; u < C::GU; ++u) {
    const int unit = tid + u * kThreads;
    g_pl[u] = unit / C::UPR;
    g_sub[u] = unit % C::UPR;
    const int n = n0 + g_pl[u];
    g_on[u] = unit < C::G_UNITS && n < a.N;
    const int nn = g_on[u] ? n : 0;
    g_b[u] = nn / a.HoWo;
    g_rem[u] = nn - g_b[u] * a.HoWo;
    g_oy[u] = g_rem[u] / a.Wo;
    g_ox[u] = g_rem[u] - g_oy[u] * a.Wo;
  }

  // corner table of the current kernel point: element offsets into xs (or -1)
  // and bilinear weights times the mask (0 for a corner outside the image)
  int c_off[C::GU][4];
  float c_w[C::GU][4];

  // Offset group of a unit in channel chunk cc: every 16-byte unit lies in one group
  // (Cg is a multiple of VEC); channels past Cin (zero weights) use the last group.
  auto corners = [&](int k, int cc) {
    const int i = k / a.K, j = k - (k / a.K) * a.K;
#pragma unroll
    for (int u = 0; u < C::GU; ++u) {
#pragma unroll
      for (int q = 0; q < 4; ++q) { c_off[u][q] = -1; c_w[u][q] = 0.f; }
      if (!g_on[u]) continue;
      const int grp = a.G == 1 ? 0 : min((cc * C::CK + g_sub[u] * C::VEC) / a.Cg, a.G - 1);
      const int gk = grp * KK + k;
      const int ob = (g_b[u] * 2 * KK * a.G + 2 * gk) * a.HoWo + g_rem[u];
      const float dy = a.offset ? load_scalar<BF16>(a.offset, ob) : 0.f;
      const float dx = a.offset ? load_scalar<BF16>(a.offset, ob + a.HoWo) : 0.f;
      const float m = a.mask ? load_scalar<BF16>(a.mask, (g_b[u] * KK * a.G + gk) * a.HoWo + g_rem[u]) : 1.f;
      // integer and fractional parts of the offset are exact in fp32, so the
      // neighbour rows/columns and the interpolation fractions are exact too.
      const float fy = floorf(dy), fx = floorf(dx);
      const float ly = dy - fy, lx = dx - fx;
      const float y0 = static_cast<float>(g_oy[u] * a.stride - a.pad + i * a.dil) + fy;
      const float x0 = static_cast<float>(g_ox[u] * a.stride - a.pad + j * a.dil) + fx;
      // inside tests on floats first: NaN and huge values fail every test
      const bool vy0 = (y0 >= 0.f) && (y0 <= static_cast<float>(a.H - 1));
      const bool vy1 = (y0 >= -1.f) && (y0 <= static_cast<float>(a.H - 2));
      const bool vx0 = (x0 >= 0.f) && (x0 <= static_cast<float>(a.W - 1));
      const bool vx1 = (x0 >= -1.f) && (x0 <= static_cast<float>(a.W - 2));
      if (!((vy0 || vy1) && (vx0 || vx1))) continue;
      const int iy = static_cast<int>(y0), ix = static_cast<int>(x0);
      const int base = ((g_b[u] * a.H + iy) * a.W + ix) * Cp;
      const float hy = 1.f - ly, hx = 1.f - lx;
      if (vy0 && vx0) { c_off[u][0] = base;                  c_w[u][0] = hy * hx * m; }
      if (vy0 && vx1) { c_off[u][1] = base + Cp;             c_w[u][1] = hy * lx * m; }
      if (vy1 && vx0) { c_off[u][2] = base + a.W * Cp;       c_w[u][2] = ly * hx * m; }
      if (vy1 && vx1) { c_off[u][3] = base + a.W * Cp + Cp;  c_w[u][3] = ly * lx * m; }
    }
  };

  uint4 graw[C::GU][4];
  uint4 araw[C::AU];

  // global loads for chunk q into registers
  auto issue = [&](int q) {
    const int k = q / cch, cc = q - (q / cch) * cch;
    if (cc == 0 || a.G > 1) corners(k, cc);
#pragma unroll
    for (int u = 0; u < C::GU; ++u) {
      const int ch = cc * C::CK + g_sub[u] * C::VEC;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        graw[u][q4] = make_uint4(0u, 0u, 0u, 0u);
        if (c_off[u][q4] >= 0)
          graw[u][q4] = *reinterpret_cast<const uint4*>(xs + static_cast<size_t>(c_off[u][q4] + ch) * C::ES);
      }
    }
#pragma unroll
    for (int u = 0; u < C::AU; ++u) {
      const int unit = tid + u * kThreads;
      if (unit < C::A_UNITS) {
        const int row = unit / C::UPR, sub = unit % C::UPR;
        const size_t e = (static_cast<size_t>(m0 + row) * KK + k) * Cp + cc * C::CK + sub * C::VEC;
        araw[u] = *reinterpret_cast<const uint4*>(wp + e * C::ES);
      }
    }
  };

  // interpolate the gathered corners and write both tiles to LDS buffer `buf`
  auto commit = [&](int buf) {
    unsigned char* As = lds[buf];
    unsigned char* Bs = lds[buf] + MT * C::ROWB;
#pragma unroll
    for (int u = 0; u < C::GU; ++u) {
      const int unit = tid + u * kThreads;
      if (unit >= C::G_UNITS) continue;
      uint4 res;
      const float w0 = c_w[u][0], w1 = c_w[u][1], w2 = c_w[u][2], w3 = c_w[u][3];
      if constexpr (BF16) {
        const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&graw[u][0]);
        const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&graw[u][1]);
        const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&graw[u][2]);
        const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&graw[u][3]);
        uint32_t* o = reinterpret_cast<uint32_t*>(&res);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float lo = w0 * bf16_lo(r0[e]);
          lo = fmaf(w1, bf16_lo(r1[e]), lo);
          lo = fmaf(w2, bf16_lo(r2[e]), lo);
          lo = fmaf(w3, bf16_lo(r3[e]), lo);
          float hi = w0 * bf16_hi(r0[e]);
          hi = fmaf(w1, bf16_hi(r1[e]), hi);
          hi = fmaf(w2, bf16_hi(r2[e]), hi);
          hi = fmaf(w3, bf16_hi(r3[e]), hi);
          o[e] = pack_bf16x2(lo, hi);
        }
      } else {
        const float* r0 = reinterpret_cast<const float*>(&graw[u][0]);
        const float* r1 = reinterpret_cast<const float*>(&graw[u][1]);
        const float* r2 = reinterpret_cast<const float*>(&graw[u][2]);
        const float* r3 = reinterpret_cast<const float*>(&graw[u][3]);
        float* o = reinterpret_cast<float*>(&res);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = w0 * r0[e];
          v = fmaf(w1, r1[e], v);
          v = fmaf(w2, r2[e], v);
          v = fmaf(w3, r3[e], v);
          o[e] = v;
        }
      }
      *reinterpret_cast<uint4*>(Bs + g_pl[u] * C::ROWB + g_sub[u] * 16) = res;
    }
#pragma unroll
    for (int u = 0; u < C::AU; ++u) {
      const int unit = tid + u * kThreads;
      if (unit < C::A_UNITS) {
        const int row = unit / C::UPR, sub = unit % C::UPR;
        *reinterpret_cast<uint4*>(As + row * C::ROWB + sub * 16) = araw[u];
      }
    }
  };

  floatx4 acc[C::FM][C::FN];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int wave_m = wave % C::WAVES_M, wave_n = wave / C::WAVES_M;
  const int lrow = lane & 15, lgrp = lane >> 4;

  auto mma = [&](int buf) {
    const unsigned char* As = lds[buf];
    const unsigned char* Bs = lds[buf] + MT * C::ROWB;
    if constexpr (BF16) {
      // 16x16x32: lane supplies 8 consecutive reduction values of row/column lane%16
      bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
        af[fm] = *reinterpret_cast<const bf16x8*>(As + (wave_m * C::WM + fm * 16 + lrow) * C::ROWB + lgrp * 16);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        bfr[fn] = *reinterpret_cast<const bf16x8*>(Bs + (wave_n * C::WN + fn * 16 + lrow) * C::ROWB + lgrp * 16);
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
    } else {
      // 16x16x4 fp32, eight steps per 32-channel chunk: at step s lane l supplies
      // reduction index (l/16)*8 + s of its row (A) and column (B)
      floatx4 a8[C::FM][2], b8[C::FN][2];
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const unsigned char* p = As + (wave_m * C::WM + fm * 16 + lrow) * C::ROWB + lgrp * 32;
        a8[fm][0] = *reinterpret_cast<const floatx4*>(p);
        a8[fm][1] = *reinterpret_cast<const floatx4*>(p + 16);
      }
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const unsigned char* p = Bs + (wave_n * C::WN + fn * 16 + lrow) * C::ROWB + lgrp * 32;
        b8[fn][0] = *reinterpret_cast<const floatx4*>(p);
        b8[fn][1] = *reinterpret_cast<const floatx4*>(p + 16);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(a8[fm][s >> 2][s & 3], b8[fn][s >> 2][s & 3],
                                                               acc[fm][fn], 0, 0, 0);
    }
  };

  // --- main loop: loads for chunk q+1 are in flight while chunk q multiplies
  issue(0);
  commit(0);
  __syncthreads();
  for (int q = 0; q < nq; ++q) {
    const bool more = q + 1 < nq;
    if (more) issue(q + 1);
    mma(q & 1);
    if (more) commit((q + 1) & 1);
    __syncthreads();
  }

  // --- epilogue: bias, rounding, NCHW store.  D fragment: lane l holds rows
  // 4*(l/16)+i, column l%16.
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int n = n0 + wave_n * C::WN + fn * 16 + lrow;
      if (n >= a.N) continue;
      const int b = n / a.HoWo, rem = n - (n / a.HoWo) * a.HoWo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = m0 + wave_m * C::WM + fm * 16 + lgrp * 4 + i;
        if (o >= a.Cout) continue;
        float v = acc[fm][fn][i];
        if (a.bias) v += load_scalar<BF16>(a.bias, o);
        if (a.om_split == 0) {
          store_scalar<BF16>(a.out, (b * a.Cout + o) * a.HoWo + rem, v);
        } else if (o < a.om_split) {   // offset channels
          store_scalar<BF16>(a.out, (b * a.om_split + o) * a.HoWo + rem, v);
        } else {                       // mask channels: sigmoid
          store_scalar<BF16>(a.out2, (b * (a.Cout - a.om_split) + o - a.om_split) * a.HoWo + rem,
                             1.f / (1.f + expf(-v)));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// variant table and launchers
// ---------------------------------------------------------------------------

static const VariantInfo kVariants[V_COUNT] = {
    {"tile_f32_m64_n64", 0, 64, 64, 32, 1},
    {"tile_f32_m128_n64", 0, 128, 64, 32, 1},
    {"tile_bf16_m64_n64", 1, 64, 64, 32, 1},
    {"tile_bf16_m128_n64", 1, 128, 64, 32, 1},
    {"tile_bf16_m128_n32", 1, 128, 32, 32, 1},
    {"tile_bf16_m256_n64", 1, 256, 64, 32, 1},
    {"box_bf16_m128", 1, 128, 0, 32, 1},
    {"box_bf16_m256", 1, 256, 0, 32, 1},
    {"direct_f32", 0, 64, 64, 1, 0},
    {"direct_bf16", 1, 64, 64, 1, 0},
    {"om_bf16", 1, 32, 32, 32, 1},
};

const VariantInfo& variant_info(int v) { return kVariants[v]; }

hipError_t launch_stage(int variant, const StageArgs& a, hipStream_t stream) {
  const VariantInfo& vi = kVariants[variant];
  if (!vi.staged) return hipSuccess;
  const uintptr_t xa = reinterpret_cast<uintptr_t>(a.x);
  // widest global read that every channel plane (starting at x + c*H*W elements)
  // keeps aligned, given the caller's x pointer
  auto fits = [&](int vec, int es) { return a.HW % vec == 0 && xa % static_cast<uintptr_t>(vec * es) == 0; };
  const int spx = vi.is_bf16 && fits(8, 2) ? kPairPx : 64;   // pixels per x tile
  const int s_tiles = (a.HW + spx - 1) / spx, c_tiles = (a.Cp + 63) / 64;
  const int nx = s_tiles * c_tiles * a.B;
  const bool wv8 = vi.is_bf16 && a.wlayout == 1 && a.KK == 9 && a.Cin % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(a.w) % 16 == 0;   // pack_weight_v8_ok
  const int wunits = wv8 ? a.Mp * (a.Cp / 8) : a.Mp * a.Cp;
  // (rounded up to a multiple of 8, so the x tiles' workgroups start on XCD 0; a
  // weight workgroup past the last unit has nothing to do)
  const int nw = a.w != nullptr ? (min((wunits + kThreads - 1) / kThreads, 1024) + 7) / 8 * 8 : 0;
  StageArgs sa = a;
  sa.nw2 = 0;
  if (a.w2 != nullptr) {
    const bool wv8b = vi.is_bf16 && a.wlayout2 == 1 && a.KK == 9 && a.Cin % 8 == 0 &&
                      reinterpret_cast<uintptr_t>(a.w2) % 16 == 0;
    const int wunits2 = wv8b ? a.Mp2 * (a.Cp / 8) : a.Mp2 * a.Cp;
    sa.nw2 = (min((wunits2 + kThreads - 1) / kThreads, 1024) + 7) / 8 * 8;
  }
  const dim3 grid(nx + nw + sa.nw2);
  void* args[] = {&sa, const_cast<int*>(&nx), const_cast<int*>(&s_tiles), const_cast<int*>(&c_tiles)};
  const void* fn;
  if (vi.is_bf16)
    fn = fits(8, 2)   ? reinterpret_cast<const void*>(&stage_kernel<true, 8>)
       : fits(4, 2)   ? reinterpret_cast<const void*>(&stage_kernel<true, 4>)
       : fits(2, 2)   ? reinterpret_cast<const void*>(&stage_kernel<true, 2>)
                      : reinterpret_cast<const void*>(&stage_kernel<true, 1>);
  else
    fn = fits(4, 4)   ? reinterpret_cast<const void*>(&stage_kernel<false, 4>)
       : fits(2, 4)   ? reinterpret_cast<const void*>(&stage_kernel<false, 2>)
                      : reinterpret_cast<const void*>(&stage_kernel<false, 1>);
  return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, stream);
}

template <bool BF16, int MT, int NT>
static hipError_t launch_tile(const FusedArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<FusedArgs*>(&a)};
  const dim3 grid(a.m_tiles * a.n_tiles);
  return hipLaunchKernel(reinterpret_cast<const void*>(&dcn_fused_kernel<BF16, MT, NT>), grid, dim3(kThreads),
                         args, 0, stream);
}

hipError_t launch_fused(int variant, const FusedArgs& a, hipStream_t stream) {
  switch (variant) {
    case V_TILE_F32_M64_N64: return launch_tile<false, 64, 64>(a, stream);
    case V_TILE_F32_M128_N64: return launch_tile<false, 128, 64>(a, stream);
    case V_TILE_BF16_M64_N64: return launch_tile<true, 64, 64>(a, stream);
    case V_TILE_BF16_M128_N64: return launch_tile<true, 128, 64>(a, stream);
    case V_TILE_BF16_M128_N32: return launch_tile<true, 128, 32>(a, stream);
    case V_TILE_BF16_M256_N64: return launch_tile<true, 256, 64>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dcn
