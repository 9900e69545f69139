// dcn_direct.hip -- gfx950 kernel for deformable convolutions with a tiny reduction
// (at most 4 input channels, K*K in {1, 4, 9}), such as a first layer on RGB input.
//
// With Cin*K*K <= 36 the column of a workgroup's pixels is a few KB, so there is no
// staging copy and the output write dominates the traffic.  A workgroup owns 64
// output pixels and up to 64 output channels:
//   * each of its four waves samples a share of the kernel points: it reads the
//     offsets and the mask of its pixels (consecutive lanes, consecutive pixels),
//     forms the sampling position and the four bilinear weights times the mask (zero
//     for a neighbour outside the image), interpolates the Cin input channels from x
//     in its given [B][Cin][H][W] layout (x is small; its reads are cache hits) and
//     puts the column entries, in fp32, in LDS.  The weight rows are loaded at the
//     same time as the offsets;
//   * after a barrier each wave multiplies one 32 x 32 block (output channels x
//     pixels) on the matrix cores, MFMA 32x32x2 in fp32 (a bf16 input is exact in
//     fp32, so one contraction serves both element types), adds the bias and stores;
//     a store instruction writes 32 consecutive pixels of two output channels.
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
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Raw buffer loads with 32-bit byte offsets (the host keeps every tensor the kernel
// reads under 2 GiB).  An offset past the end reads 0 without touching memory, which
// is how neighbours outside the image are read: no branch around the load.
constexpr uint32_t kOutside = 0x80000000u;
// cache-policy bits of a buffer store: nontemporal
constexpr int kNonTemporal = 2;

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
  constexpr int RP = (RMAX + 1) & ~1;   // reduction length padded to the MFMA's k = 2
  // column [r][pixel] and weight rows [r][output channel - o0], zero past Cin*K*K
  // (one padding column keeps the 32 lanes of a weight read on distinct banks)
  __shared__ float colbuf[RP][64];
  __shared__ float wsm[RP][65];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int RK = a.Cin * KKT;
  const int o0 = blockIdx.y * 64, o1 = min(o0 + 64, a.Cout);
  const uint32_t HW = static_cast<uint32_t>(a.H) * static_cast<uint32_t>(a.W);
  const auto rx = rsrc(a.x, static_cast<uint32_t>(a.B) * a.Cin * HW * ES);
  const auto ro = rsrc(a.offset, static_cast<uint32_t>(a.B) * 2 * KKT * a.HoWo * ES);
  const auto rm = rsrc(a.mask ? a.mask : a.offset, static_cast<uint32_t>(a.B) * KKT * a.HoWo * ES);
  // weight rows: the loads are issued here and stored to LDS after the offsets' loads
  // have gone out too, so the two latencies overlap
  constexpr int NW = (64 * RP + 255) / 256;
  float wv[NW];
  {
    const auto rw = rsrc(a.w, static_cast<uint32_t>(a.Cout) * RK * ES);
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int e = tid + t * 256;
      const int ol = e / RP, r = e - (e / RP) * RP;
      wv[t] = ldb_if<BF16>(rw, e < 64 * RP && o0 + ol < a.Cout && r < RK, static_cast<uint32_t>(o0 + ol) * RK + r);
    }
  }
  const int n = blockIdx.x * 64 + lane;
  const bool live = n < a.N;
  const int nn = live ? n : 0;
  const int b = nn / a.HoWo, rem = nn - (nn / a.HoWo) * a.HoWo;
  const int oy = rem / a.Wo, ox = rem - (rem / a.Wo) * a.Wo;

  // ---- column of the workgroup's 64 pixels: wave w samples kernel points k = w, w+4, ...
  // Offsets and mask first, then the positions, then every input load (no lane-dependent
  // branches: neighbours outside the image read as zero), then the interpolation.  Only
  // the last round of kernel points can be short of a point for some waves; those skip it.
  constexpr int KPW = (KKT + 3) / 4;   // kernel points per wave (at most)
  auto has = [&](int t) { return t < KPW - 1 || wave + 4 * t < KKT; };   // uniform
  float dy[KPW], dx[KPW], mk[KPW];
#pragma unroll
  for (int t = 0; t < KPW; ++t) {
    dy[t] = dx[t] = 0.f;
    mk[t] = 1.f;
    if (!has(t)) continue;
    const int k = wave + 4 * t;
    const uint32_t ob = (static_cast<uint32_t>(b) * 2 * KKT + 2 * k) * a.HoWo + rem;
    dy[t] = ldb<BF16>(ro, ob);
    dx[t] = ldb<BF16>(ro, ob + a.HoWo);
    mk[t] = a.mask ? ldb<BF16>(rm, (static_cast<uint32_t>(b) * KKT + k) * a.HoWo + rem) : 1.f;
  }
#pragma unroll
  for (int t = 0; t < NW; ++t) {
    const int e = tid + t * 256;
    if (e < 64 * RP) wsm[e - (e / RP) * RP][e / RP] = wv[t];
  }
  float xv[KPW][CMAX][4], wq[KPW][4];
#pragma unroll
  for (int t = 0; t < KPW; ++t) {
    if (!has(t)) continue;
    const int k = wave + 4 * t;
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
    if (!has(t)) continue;
    const int k = wave + 4 * t;
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
      // channels past Cin (and a padding row) are zero
      colbuf[c * KKT + k][lane] = c < a.Cin ? wq[t][0] * xv[t][c][0] + wq[t][1] * xv[t][c][1] +
                                                  wq[t][2] * xv[t][c][2] + wq[t][3] * xv[t][c][3]
                                            : 0.f;
    }
  }
  if constexpr (RP > RMAX) {
    if (tid < 64) colbuf[RMAX][tid] = 0.f;
  }
  __syncthreads();

  // ---- contraction on the matrix cores: wave w multiplies the 32 x 32 block of output
  // channels o0 + 32*(w/2) .. +31 and pixels 32*(w%2) .. +31.  MFMA 32x32x2 f32 operands:
  // lane l holds row (A) / column (B) l % 32 at reduction index 2*step + l / 32.
  const int l32 = lane & 31, lh = lane >> 5;
  const int om = 32 * (wave >> 1), pn = 32 * (wave & 1);
  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int st = 0; st < RP / 2; ++st) {
    const float av = wsm[2 * st + lh][om + l32];
    const float bv = colbuf[2 * st + lh][pn + l32];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
  }
  // accumulator element r: output channel o0 + om + 8*(r/4) + 4*lh + r%4, pixel pn + l32.
  // The bias values are loaded first, all of them (past Cout the buffer reads zero): a
  // load under the per-element branch would make each store wait for the ones before.
  float bias[16];
  if (a.bias != nullptr) {   // uniform
    const auto rbias = rsrc(a.bias, a.Cout * ES);
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = ldb<BF16>(rbias, o0 + om + 8 * (r >> 2) + 4 * lh + (r & 3));
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = 0.f;
  }
  // Stores go through a buffer resource: the lane's offset of its first element, and per
  // accumulator element a uniform offset of whole output-channel planes (no per-element
  // address arithmetic).  A pixel past N or an output channel past Cout gets an offset
  // past the buffer, and the store is dropped.  The stores are nontemporal (nothing here
  // reads the output again, so it does not displace the inputs from L2).
  const int np = blockIdx.x * 64 + pn + l32;
  const auto rout = rsrc(a.out, static_cast<uint32_t>(a.B) * a.Cout * a.HoWo * ES);
  const int npc = np < a.N ? np : 0;
  const int bp = npc / a.HoWo, remp = npc - (npc / a.HoWo) * a.HoWo;
  const int orow = o0 + om + 4 * lh;   // output channel of accumulator element 0
  const uint32_t vo = ((static_cast<uint32_t>(bp) * a.Cout + orow) * static_cast<uint32_t>(a.HoWo) + remp) * ES;
  const uint32_t plane = static_cast<uint32_t>(a.HoWo) * ES;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int dr = 8 * (r >> 2) + (r & 3);
    const bool ok = np < a.N && orow + dr < o1;
    const float v = acc[r] + bias[r];
    const uint32_t off = ok ? vo : kOutside;
    if constexpr (BF16) __builtin_amdgcn_raw_buffer_store_b16(to_bf16(v), rout, off, dr * plane, kNonTemporal);
    else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rout, off, dr * plane, kNonTemporal);
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
