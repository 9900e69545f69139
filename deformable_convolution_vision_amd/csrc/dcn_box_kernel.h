// dcn_box_kernel.h -- the gfx950 fused deformable-convolution kernel for bf16 with an
// LDS input box (the kernel template; dcn_box.hip holds its launcher, and the
// dcn_box_inst_*.hip files instantiate it, a few tile shapes per file so they compile
// in parallel).
//
// One workgroup computes an MT x (TH x TW) tile: MT output channels by a rectangular
// TH x TW block of output pixels of one image.  It runs eight wave64, two per SIMD:
//
//  * four producer waves build the column matrix of the deformable im2col, one
//    (32-channel chunk, kernel point) step at a time, into a double-buffered LDS
//    tile.  The sampling positions, bilinear corner weights times the mask and the
//    corner offsets are computed once per (pixel, kernel point) in the prologue and
//    kept in an LDS table.  For each 32-channel chunk the producers copy the
//    rectangle of the channels-last input that the tile's samples touch (the "box":
//    its extent comes from the tile's own offsets, clipped to one pixel around the
//    image) into LDS with direct global->LDS loads, one chunk ahead, so each input
//    vector crosses the vector-memory pipe once per chunk instead of once per
//    (sample, corner).  A sample is interpolated from the box in fp32 (the bf16
//    corners widened exactly, four fp32 weights, fused multiply-adds), rounded to bf16
//    once; samples whose corners lie outside the box are read from the channels-last
//    copy in global memory instead;
//  * four consumer waves multiply the previous step's column tile with MFMA
//    32x32x16 bf16 (two per 32-channel step and 32x32 output block) against their
//    rows of the repacked weight, which they stream from L2 straight into registers
//    through a prefetch ring, and accumulate in fp32.  The 32x32 shape keeps the
//    matrix core at full rate next to the producers' VALU work and takes fewer VALU
//    issue cycles away from them than the 16x16 shape does.
//
// On each SIMD the producer's VALU work overlaps the consumer's matrix work.  The
// two box buffers are separate LDS arrays (and the producer loop is instantiated
// once per buffer parity) so the compiler can tell the copy into one from the reads
// of the other and does not make reads wait for the copy.
//
// The computation follows the deformable-convolution equation (csdn.net tags page
// "可变形卷积：Deformable ConvNets", part "Deformable Convolutional Networks",
// section on deformable convolution), with the DCNv2 modulation scalar (same page,
// section 3.2) and bilinear interpolation from the four integer neighbours (same
// page, bilinear-interpolation equation); neighbours outside the image contribute 0.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dcn_internal.h"

namespace dcn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 512;    // 4 consumer + 4 producer waves (8 producer waves: 768)
constexpr int kCK = 32;          // channels per reduction chunk (one MFMA k-step)
constexpr int kPXB = 64;         // bytes per box pixel (32 bf16 channels)
constexpr int kCOLB = 80;        // bytes per column-tile row (64 + 16 pad)

// Corner-table entry of one (kernel point, pixel), 16 bytes.  The bilinear weights
// keep fp32 precision (rounded to bf16 they would leave an error that scales with the
// corner magnitudes instead of with the sample: corners of alternating sign at
// fractions near 1/2 nearly cancel).  The four weights times the mask are
// (a*(1-lx), a*lx, b*(1-lx), b*lx) with a = (1-ly)*m, b = ly*m.
struct CEnt {
  int off;      // >= 0: byte offset of corner (y0, x0) in a box buffer; -2: every corner outside
                // the image (weights 0); <= -3: corners outside the box, read from global memory
                // at (y0, x0) = ((-off - 3) >> 16) - 1, ((-off - 3) & 0xffff) - 1
  float a, b, lx;
};
constexpr int kCEntBytes = 16;
// a table entry as the producers use it: the offset code and the four weights
struct CW { float w0, w1, w2, w3; };
struct CEw {
  int off;
  CW w;
};
__device__ __forceinline__ bool ce_global(const CEw& c) { return c.off <= -3; }

constexpr int kColBufs = 3;      // column-tile ring: produced at step s, read at s+1, multiplied at s+2
constexpr int kZeroB = 128;      // zero bytes after each box buffer: the source of samples that read nothing

// GRP: offset groups (one corner table per group, two tables in LDS: the consumers
// fill the next group's table while the current group's chunks run)
template <int FN, bool GRP = false>
struct BoxCfg {
  static constexpr int NT = 16 * FN;
  static constexpr int COL_BYTES = kColBufs * NT * kCOLB;
  static constexpr int CTAB_BYTES = (GRP ? 2 : 1) * kBoxMaxKK * NT * kCEntBytes;
  // what is left of the LDS, split into two box buffers, in whole 64-pixel groups
  // (each of the four producer waves copies 16-pixel blocks, every block of a group)
  static constexpr int BOX_PX = ((kLdsBudget - COL_BYTES - CTAB_BYTES - 2 * kZeroB - 64) / (2 * kPXB)) / 64 * 64;
};

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}


// Bilinear sample of two channels packed in one dword per corner (bf16 pairs; row 0:
// a0, a1, row 1: b0, b1) with fp32 weights: the corners are widened exactly to fp32,
// multiplied and summed in fp32, and the two results rounded to bf16 (RNE).
__device__ __forceinline__ CEw expand(const CEnt& ce) {
  const float hx = 1.f - ce.lx;
  return CEw{ce.off, CW{ce.a * hx, ce.a * ce.lx, ce.b * hx, ce.b * ce.lx}};
}
__device__ __forceinline__ uint32_t interp2(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, const CW& w) {
  const float lo = __builtin_fmaf(w.w3, __uint_as_float(b1 << 16),
                   __builtin_fmaf(w.w2, __uint_as_float(b0 << 16),
                   __builtin_fmaf(w.w1, __uint_as_float(a1 << 16), w.w0 * __uint_as_float(a0 << 16))));
  const float hi = __builtin_fmaf(w.w3, __uint_as_float(b1 & 0xffff0000u),
                   __builtin_fmaf(w.w2, __uint_as_float(b0 & 0xffff0000u),
                   __builtin_fmaf(w.w1, __uint_as_float(a1 & 0xffff0000u), w.w0 * __uint_as_float(a0 & 0xffff0000u))));
  return pk_bf16(lo, hi);
}

// 8 channels of one sample from the four corner vectors (row 0: q00, q01; row 1:
// q10, q11)
__device__ __forceinline__ uint4 interp8(uint4 q00, uint4 q01, uint4 q10, uint4 q11, const CW& ce) {
  return make_uint4(interp2(q00.x, q01.x, q10.x, q11.x, ce), interp2(q00.y, q01.y, q10.y, q11.y, ce),
                    interp2(q00.z, q01.z, q10.z, q11.z, ce), interp2(q00.w, q01.w, q10.w, q11.w, ce));
}

// the same for 4 channels (8-byte corner vectors)
__device__ __forceinline__ uint2 interp8(uint2 q00, uint2 q01, uint2 q10, uint2 q11, const CW& ce) {
  return make_uint2(interp2(q00.x, q01.x, q10.x, q11.x, ce), interp2(q00.y, q01.y, q10.y, q11.y, ce));
}

// component-wise select (a select of whole structs can become a select of their
// addresses, which keeps them out of registers)
__device__ __forceinline__ uint4 sel4(bool c, uint4 a, uint4 b) {
  return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}
__device__ __forceinline__ uint2 sel4(bool c, uint2 a, uint2 b) { return make_uint2(c ? a.x : b.x, c ? a.y : b.y); }

// f(integral_constant<int, I>) for I = B .. E-1, each call inlined with I known at compile time
template <int I, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>());
    static_for<I + 1, E>(f);
  }
}

__device__ __forceinline__ int xcd_tile(int g, int T) {
  const int xcd = g & 7, idx = g >> 3;
  const int q = T >> 3, r = T & 7;
  return xcd * q + min(xcd, r) + idx;
}

__device__ __forceinline__ float ld_bf16(const void* p, int idx) {
  const uint16_t v = reinterpret_cast<const uint16_t*>(p)[idx];
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Raw buffer resource over the `bytes` bytes at `p`: loads at offsets past the end
// return zeros (and move no data).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const unsigned char* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(p), 0, static_cast<int>(bytes), 0x00020000);
}
// a byte offset past the end of every buffer here (the host keeps them under 4 GiB - 64)
constexpr uint32_t kOOB = 0xfffffff0u;
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// the same with a wave-uniform byte offset added (the instruction's scalar offset)
__device__ __forceinline__ uint4 buffer_load16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// the corner vector type's load: 16 or 8 bytes
__device__ __forceinline__ void buffer_load_q(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint4& out) {
  out = buffer_load16(r, voff);
}
__device__ __forceinline__ void buffer_load_q(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint2& out) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
  out = make_uint2(v[0], v[1]);
}
// Direct buffer->LDS load: 16 bytes per lane from byte offset `voff`, lane l's bytes
// at dst + 16*l.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, unsigned char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, 0, 0, 0);
}

// Workgroup barriers that order LDS traffic only; outstanding global loads stay in
// flight across them.
//  * lds_barrier: release/acquire fences limited to the local address space around
//    the barrier.  The compiler knows what they order, so its wait counts for the
//    global loads before and after stay exact.  Used by waves that have no direct
//    global->LDS loads in flight (the fence would have to wait for those: they write LDS).
//  * lds_barrier_dma: the same barrier as an opaque instruction sequence, for the
//    waves whose box copies must stay in flight across it.  The "memory" clobber keeps
//    the compiler from moving memory accesses across it; its wait counts around it
//    are conservative.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);   // keep the instruction scheduler from moving work across
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void lds_barrier_dma() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// The same with the last N LDS operations of this wave still in flight: reads whose
// data nobody changes across the barrier.  LDS operations complete in order, so the
// operations before them (the column stores the barrier publishes) are complete.
template <int N>
__device__ __forceinline__ void lds_barrier_keep() {
  asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace

template <int FM, int FN, int KKT, bool GRP, int PW = 4>
__global__ __launch_bounds__(256 + 64 * PW) void dcn_box_kernel(BoxArgs ba) {
  using Cfg = BoxCfg<FN, GRP>;
  const FusedArgs& a = ba.f;
  static_assert(!GRP || KKT == 9, "offset groups: 3x3 only");
  // PW producer waves: 4 (16-byte column units, 8 channels per thread and sample) or 8
  // (8-byte units, 4 channels; two producer waves share each SIMD)
  static_assert(PW == 4 || PW == 8, "four or eight producer waves");
  static_assert(PW == 4 || (KKT == 9 && !GRP), "eight producer waves: 3x3, one offset group");
  constexpr int NTH = 256 + 64 * PW;   // threads per workgroup
  constexpr int PTH = 64 * PW;         // producer threads
  constexpr int UB = PW == 8 ? 8 : 16; // bytes per column unit
  constexpr int UPS = kPXB / UB;       // units per 32-channel sample
  constexpr int UPS_SH = PW == 8 ? 3 : 2;   // log2(UPS): thread indexes are non-negative, shifts suffice
  using QV = typename std::conditional<PW == 8, uint2, uint4>::type;
  static_assert(FM % 2 == 0 && FN % 2 == 0, "whole 32x32 MFMA blocks per wave");
  constexpr int TM = FM / 2, TN = FN / 2;   // 32x32 output blocks per consumer wave
  constexpr int WM = 16 * FM;         // rows per consumer wave
  constexpr int MT = 4 * WM;          // rows per workgroup
  constexpr int NT = Cfg::NT;         // pixel slots per workgroup
  constexpr int GUNITS = NT * UPS;    // column units per chunk
  constexpr int GU = (GUNITS + PTH - 1) / PTH;
  constexpr int BOXB = Cfg::BOX_PX * kPXB;

  // The column ring is read every step by the consumers: the largest alignment puts it
  // at the start of LDS, so its reads address it with immediate offsets.
  __shared__ __attribute__((aligned(1024))) unsigned char col[Cfg::COL_BYTES];
  // corner table (with offset groups two tables, the second from entry kBoxMaxKK * NT)
  __shared__ __attribute__((aligned(16))) CEnt ctab[(GRP ? 2 : 1) * kBoxMaxKK * NT];
  __shared__ __attribute__((aligned(16))) unsigned char box0[BOXB + kZeroB];
  __shared__ __attribute__((aligned(16))) unsigned char box1[BOXB + kZeroB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Waves w and w+4 of a workgroup run on the same SIMD.  Roles: by default waves
  // 0-3 consume and 4-7 produce, so every SIMD runs one of each; with split_roles
  // waves 0, 1, 4, 5 consume (two SIMDs) and 2, 3, 6, 7 produce (the other two).
  // wv is the wave's index within its role, rtid the thread's.
  const int wraw = __builtin_amdgcn_readfirstlane(wave);
  const bool consumer = ba.split_roles ? (wraw & 2) == 0 : wraw < 4;
  // (& 7: the index is known non-negative, so index divisions stay unsigned)
  const int wv = ba.split_roles ? (wraw & 1) | ((wraw >> 2) << 1) : ((consumer ? wraw : wraw - 4) & 7);
  const int rtid = wv * 64 + lane;
  // MFMA 32x32x16 operand lanes: row (A) or column (B) lane & 31, and a 16-byte
  // channel group: lane half lh holds channels 16*lh + 8*h .. +7 of k-half h, so a
  // lane's two halves are one contiguous 32-byte run
  const int l32 = lane & 31, lh = lane >> 5;
  const int KK = a.KK, Cp = a.Cp, K = a.K;
  const int T = a.m_tiles * ba.tiles_per_img * a.B;
  const int t = xcd_tile(blockIdx.x, T);
  const int mt = t % a.m_tiles;
  const int pt = t / a.m_tiles;
  const int b = pt / ba.tiles_per_img;
  const int rt = pt - b * ba.tiles_per_img;
  const int ty = rt / ba.tiles_x, tx = rt - (rt / ba.tiles_x) * ba.tiles_x;
  const int oy0 = ty * ba.TH, ox0 = tx * ba.TW;
  const int m0 = mt * MT;
  const int nCC = Cp / kCK;
  const int S = nCC * KK;
  // offset groups (GRP): NG groups of cpg chunks each; group g's corner table is
  // table g % 2
  const int NG = GRP ? a.G : 1;
  const int cpg = GRP ? a.Cg / kCK : nCC;
  // first entry of the table of chunk cc
  auto table_of_chunk = [&](int cc) __attribute__((always_inline)) -> int {
    if constexpr (GRP) return ((cc / cpg) & 1) * (kBoxMaxKK * NT);
    else return 0;
  };
  auto get_ce = [&](int e) __attribute__((always_inline)) -> CEnt {
    return __builtin_bit_cast(CEnt, reinterpret_cast<const uint4*>(ctab)[e]);
  };

  const unsigned char* xs = reinterpret_cast<const unsigned char*>(a.xs);
  const unsigned char* wp = reinterpret_cast<const unsigned char*>(a.wp);

  // ---- consumer state: weight fragments
  // The repacked weight is step-major, [step][Mp][32 channels], so the 32 rows x 64
  // bytes of one 32-row block are one contiguous 2 KB.  Raw buffer loads: one per-lane
  // byte offset (the lane's row of the wave's first block; the host keeps the repacked
  // weight under 4 GiB) in a vector register, and the step's base plus the block and
  // half offsets as the wave-uniform scalar offset, so the loop holds one address
  // register and forms no 64-bit address per lane.
  struct AFrag { uint4 v[TM][2]; };
  const uint32_t step_bytes = static_cast<uint32_t>(a.m_tiles * MT) * 64u;
  const uint32_t aoff = static_cast<uint32_t>(m0 + wv * WM + l32) * 64u + static_cast<uint32_t>(lh * 32);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(wp, static_cast<uint32_t>(S) * step_bytes);
  auto load_a = [&](int s) __attribute__((always_inline)) -> AFrag {
    AFrag r;
    const uint32_t sb = static_cast<uint32_t>(s) * step_bytes;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      r.v[tm][0] = buffer_load16s(wrs, aoff, sb + static_cast<uint32_t>(tm * 32 * 64));
      r.v[tm][1] = buffer_load16s(wrs, aoff, sb + static_cast<uint32_t>(tm * 32 * 64 + 16));
    }
    return r;
  };
  // Weight fragments in two sets of G slots: chunks G*g .. G*g+G-1 live in set pa
  // for even g and in set qa for odd g.  With four producer waves G = 4 for the smaller
  // tiles and G = 2 where 2*G*FM fragments would not fit next to the accumulators and
  // column fragments, and with offset groups, whose table work adds to the consumers'
  // registers.  With eight producer waves (three waves per SIMD) G = 2 for tiles up to
  // 256 x 64 (loads two steps ahead: c4 fused 31.6 -> 30.9 us) and G = 1 for wider ones.
  constexpr int G = PW == 8 ? (FM * FN <= 16 ? 2 : 1) : (FM * FN <= 16 && !GRP) ? 4 : 2;
  // consumers keep one column buffer in registers instead of two (eight producer waves
  // with tiles wider than 256 x 64)
  constexpr bool kSingleB = PW == 8 && FM * FN > 16;
  AFrag pa[G], qa[G];
  // weights for chunks c0 .. c0+G-1 (past the end a valid chunk is re-read, so every
  // group issues the same loads)
  auto load_group = [&](int c0, AFrag (&x)[G]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < G; ++i) x[i] = load_a(min(c0 + i, S - 1));
  };

  // The prologue has one barrier, and it orders LDS traffic only (lds_barrier): it
  // does not wait for the consumers' weight prefetch.

  // ---- box geometry (uniform, from the tile alone): the window the tile's samples
  // use with zero offsets, widened evenly by the largest margin the LDS budget allows,
  // within [-1, H] x [-1, W] (the host checks the offset-free window fits).  Samples
  // whose corners leave it take the global path.  Known before any offset arrives, so
  // the first chunk's copy overlaps the offset loads.
  int by0, bx0, BH, BW;
  {
    const int bh0 = (ba.TH - 1) * a.stride + (K - 1) * a.dil + 2;
    const int bw0 = (ba.TW - 1) * a.stride + (K - 1) * a.dil + 2;
    int mg = 0;
    while ((bh0 + 2 * (mg + 1)) * (bw0 + 2 * (mg + 1)) <= min(ba.box_px, Cfg::BOX_PX)) ++mg;
    by0 = max(oy0 * a.stride - a.pad - mg, -1);
    bx0 = max(ox0 * a.stride - a.pad - mg, -1);
    BH = max(min(bh0 + 2 * mg, a.H + 1 - by0), 1);
    BW = max(min(bw0 + 2 * mg, a.W + 1 - bx0), 1);
  }
  const int npx = BH * BW;
  if (tid < kZeroB / 16) {
    *reinterpret_cast<uint4*>(box0 + BOXB + tid * 16) = make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(box1 + BOXB + tid * 16) = make_uint4(0u, 0u, 0u, 0u);
  }

  // ---- the consumer waves build the corner table while the producer waves copy the
  // first box chunk (a wave waiting for its offsets would otherwise also wait for its
  // older box loads).  The consumers issue the offset and mask loads of every (tap,
  // pixel) entry, all independent, then do the table math.
  const int ntile = ba.TH * ba.TW;
  constexpr int kPE = (kBoxMaxKK * NT + 255) / 256;
  // raw bf16 bits; every address first, then every load
  uint32_t ldy[kPE], ldx[kPE], lm[kPE];
  // offsets and mask of group g (field g*KK + k of each kernel point k)
  auto load_offsets = [&](int g) __attribute__((always_inline)) {
    int ob[kPE], mb[kPE];
#pragma unroll
    for (int j = 0; j < kPE; ++j) {
      const int e = rtid + j * 256;
      const int k = e / NT, p = e - (e / NT) * NT;
      const int py = p / ba.TW, px = p - (p / ba.TW) * ba.TW;
      const int oy = oy0 + py, ox = ox0 + px;
      const bool ok = e < KK * NT && p < ntile && oy < a.Ho && ox < a.Wo;
      const int rem = ok ? oy * a.Wo + ox : 0;
      const int gk = g * KK + (ok ? k : 0);
      ob[j] = (b * 2 * KK * NG + 2 * gk) * a.HoWo + rem;
      // always a load (from the offsets when there is no mask, ignored below), so no
      // branch joins on a value still in flight
      mb[j] = a.mask ? (b * KK * NG + gk) * a.HoWo + rem : ob[j];
    }
    const uint16_t* offs = reinterpret_cast<const uint16_t*>(a.offset);
    const uint16_t* msk = reinterpret_cast<const uint16_t*>(a.mask ? a.mask : a.offset);
#pragma unroll
    for (int j = 0; j < kPE; ++j) {
      ldy[j] = offs[ob[j]];
      ldx[j] = offs[ob[j] + a.HoWo];
      lm[j] = msk[mb[j]];
    }
  };
  if (consumer) load_offsets(0);

  // ---- the producers' box-copy plan (with the box pixels outside the image zeroed),
  // then chunk 0 of the box
  const int pw = wv;                        // producer wave 0..PW-1 (unused by consumers)
  // Box copy, one wave instruction per 16 pixels: lane -> pixel blk*16 + lane/4,
  // 16-byte quarter lane%4.  Pixels advance by 16*PW between a wave's blocks; the
  // row/column step is precomputed so no division is needed per block.
  const int nblk = (npx + 15) >> 4;
  const int step_r = (16 * PW) / BW, step_c = 16 * PW - ((16 * PW) / BW) * BW;
  const int px_first = pw * 16 + (lane >> 2);
  const int ry_first = px_first / BW, rx_first = px_first - (px_first / BW) * BW;
  // per-lane byte offsets (32-bit: the host keeps the staged copy under 4 GiB)
  // relative to a wave-uniform base for the chunk
  const uint32_t img_off = static_cast<uint32_t>(b * a.H) * static_cast<uint32_t>(a.W * Cp) * 2u +
                           static_cast<uint32_t>((lane & 3) * 16);
  const uint32_t row_bytes = static_cast<uint32_t>(a.W * Cp) * 2u, px_bytes = static_cast<uint32_t>(Cp) * 2u;
  // The per-lane byte offsets of the wave's blocks are the same for every chunk (only
  // the chunk's channel base moves), so they are computed once; each copy is then
  // one direct global->LDS load per block.  A lane with no pixel to copy (past the
  // box, or outside the image: those box pixels are zero) loads from past the end
  // of the buffer, which moves no data, so every block is issued unconditionally
  // and the number of vector-memory operations of each step is a compile-time
  // constant (exact wait counts for the prefetched global-path corners below).
  // blocks per wave, rounded up: PW * MAXB blocks cover the whole buffer (with eight
  // producer waves a buffer of 960 or 832 pixels is not a whole number of 128-pixel rounds)
  constexpr int MAXB = (Cfg::BOX_PX + 16 * PW - 1) / (16 * PW);
  const uint32_t xs_bytes = static_cast<uint32_t>(a.B * a.H) * static_cast<uint32_t>(a.W * Cp) * 2u;
  uint32_t boff[MAXB];
  if (!consumer) {
    int px = px_first, ry = ry_first, rx = rx_first;
    static_for<0, MAXB>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      const int gy = by0 + ry, gx = bx0 + rx;
      const bool inside = gy >= 0 && gy < a.H && gx >= 0 && gx < a.W;
      const bool ok = pw + PW * j < nblk && px < npx && inside;
      boff[j] = ok ? img_off + static_cast<uint32_t>(gy) * row_bytes + static_cast<uint32_t>(gx) * px_bytes
                   : kOOB;
      // box pixels outside the image stay zero in both buffers
      if (pw + PW * j < nblk && px < npx && !inside) {
        *reinterpret_cast<uint4*>(box0 + px * kPXB + (lane & 3) * 16) = make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(box1 + px * kPXB + (lane & 3) * 16) = make_uint4(0u, 0u, 0u, 0u);
      }
      px += 16 * PW;
      ry += step_r;
      rx += step_c;
      if (rx >= BW) { rx -= BW; ++ry; }
    });
  }
  // chunk cc's view of the staged copy; past the last chunk an empty range, so the
  // steady-state schedule can issue its copies and loads there too (they move no data)
  auto chunk_rsrc = [&](int cc) __attribute__((always_inline)) {
    return make_rsrc(xs + cc * kCK * 2, cc < nCC ? xs_bytes - static_cast<uint32_t>(cc * kCK * 2) : 0u);
  };
  // blocks J0 .. J1-1 of the wave for chunk cc into `dst` (raw buffer loads into LDS:
  // a scalar resource per chunk plus a 32-bit vector offset, so no per-block 64-bit
  // address arithmetic)
  auto copy_blocks = [&](int cc, unsigned char* dst, auto j0c, auto j1c) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rsrc = chunk_rsrc(cc);
    static_for<decltype(j0c)::value, decltype(j1c)::value>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      if constexpr (PW * MAXB * 16 > Cfg::BOX_PX) {
        // the rounded-up last round: only blocks inside the buffer are issued (an
        // out-of-range load still has an LDS destination)
        if (pw + PW * j < Cfg::BOX_PX / 16) buffer_to_lds16(rsrc, dst + (pw + PW * j) * 1024, boff[j]);
      } else {
        buffer_to_lds16(rsrc, dst + (pw + PW * j) * 1024, boff[j]);
      }
    });
  };
  auto copy_box = [&](int cc, unsigned char* dst) __attribute__((always_inline)) {
    copy_blocks(cc, dst, std::integral_constant<int, 0>(), std::integral_constant<int, MAXB>());
  };
  // the share of the copy issued in step k < 4 of a chunk
  auto copy_part4 = [&](int cc, unsigned char* dst, auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    copy_blocks(cc, dst, std::integral_constant<int, k * MAXB / 4>(),
                std::integral_constant<int, (k + 1) * MAXB / 4>());
  };
  // chunk 0: direct buffer->LDS loads by the four producer waves
  if (!consumer) copy_box(0, box0);

  // ---- corner table (consumer waves): sampling positions, bilinear weights times
  // the mask, and the byte offset of corner (y0, x0) in a box buffer, from the
  // offsets load_offsets left in ldy/ldx/lm
  auto build_table = [&](int tb) __attribute__((always_inline)) {
#pragma unroll
  for (int jj = 0; jj < kPE; ++jj) {
    const int e = rtid + jj * 256;
    if (e >= KK * NT) continue;
    const int k = e / NT, p = e - (e / NT) * NT;
    CEnt ce;
    ce.off = -2;
    ce.a = ce.b = ce.lx = 0.f;
    const int py = p / ba.TW, px = p - (p / ba.TW) * ba.TW;
    const int oy = oy0 + py, ox = ox0 + px;
    if (p < ntile && oy < a.Ho && ox < a.Wo) {
      const int i = k / K, j = k - (k / K) * K;
      const float dy = __uint_as_float(ldy[jj] << 16), dx = __uint_as_float(ldx[jj] << 16);
      const float m = a.mask ? __uint_as_float(lm[jj] << 16) : 1.f;
      // integer and fractional parts of the offset are exact in fp32
      const float fy = floorf(dy), fx = floorf(dx);
      const float ly = dy - fy, lx = dx - fx;
      const float y0 = static_cast<float>(oy * a.stride - a.pad + i * a.dil) + fy;
      const float x0 = static_cast<float>(ox * a.stride - a.pad + j * a.dil) + fx;
      // at least one corner inside the image (float tests first: NaN fails them all)
      if (y0 >= -1.f && y0 <= static_cast<float>(a.H - 1) && x0 >= -1.f && x0 <= static_cast<float>(a.W - 1)) {
        const int iy = static_cast<int>(y0), ix = static_cast<int>(x0);
        const float hy = 1.f - ly;
        const int ry = iy - by0, rx = ix - bx0;
        // (iy + 1 < 2^15 and ix + 1 < 2^16: the host keeps H and W under 32000)
        ce.off = (ry >= 0 && ry + 1 < BH && rx >= 0 && rx + 1 < BW) ? (ry * BW + rx) * kPXB
                                                                    : -(((iy + 1) << 16) | (ix + 1)) - 3;
        ce.a = hy * m;
        ce.b = ly * m;
        ce.lx = lx;
      }
    }
    ctab[tb + e] = ce;
  }
  };
  if (consumer) build_table(0);
  // Drain: the producers' chunk-0 copy and the consumers' offset loads (the padded
  // entries' loads are never read, and a register they left pending would later make
  // a wait cover the weight loads too).
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0) only
  lds_barrier();

  if (consumer) {
    // ================= consumers: MFMA on the previous step's column tile =================
    // The first 2G weight steps are loaded here rather than in the shared prologue:
    // the two role branches are laid out one after the other in the compiled code, so
    // registers the consumers load before the branch would stay allocated through the
    // producers' code.  Steps 0 and 1 have no multiply, which hides most of the latency.
    load_group(0, pa);
    load_group(G, qa);
    floatx16 acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;

    // B fragments of one column tile (read one step before they are multiplied)
    struct BFrag { bf16x8 v[TN][2]; };
    auto read_b = [&](int c) __attribute__((always_inline)) -> BFrag {
      BFrag r;
      const unsigned char* csrc = col + (c % kColBufs) * NT * kCOLB + l32 * kCOLB + lh * 32;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        r.v[tn][0] = *reinterpret_cast<const bf16x8*>(csrc + tn * 32 * kCOLB);
        r.v[tn][1] = *reinterpret_cast<const bf16x8*>(csrc + tn * 32 * kCOLB + 16);
      }
      return r;
    };
    // k-half outer, so two MFMAs into one accumulator are TM*TN instructions apart
    auto mma = [&](const AFrag& af, const BFrag& bf) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const bf16x8 av = __builtin_bit_cast(bf16x8, af.v[tm][h]);
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bf.v[tn][h], acc[tm][tn], 0, 0, 0);
        }
    };
    // Chunk c is multiplied during step c+2, between barriers c+1 and c+2: read
    // chunk c+1's columns (produced in step c+1), multiply chunk c (columns read
    // during step c+1), then barrier c+2.  Steps 0 and 1 have no multiply and the
    // last two chunks no barrier after them, so the consumers pass exactly S barriers,
    // like the producers.  `step` is the steady state (all three parts present);
    // `step_tail` tests each part.
    // Each step reloads the weight slot it has just multiplied with the chunk 2G
    // steps later, so the weight loads are spread evenly and arrive 2G-1 steps early.
    // Offset groups: during the first chunk cc0 of group g the consumers fill group
    // g+1's table (the other table, last read by group g-1's steps): its offset loads
    // in step 9*cc0 (between barriers 9*cc0+1 and +2), its entries in step 9*cc0+2
    // (barriers +3 to +4).  The producers first read it at step 7 of group g's last
    // chunk, three barriers or more later.
    auto table_work = [&](int c, auto phase) __attribute__((always_inline)) {
      if constexpr (GRP) {
        constexpr int ph = decltype(phase)::value;
        const int cc = c / 9, kk = c - cc * 9;
        if (kk != (ph == 0 ? 0 : 2)) return;
        const int g = cc / cpg;
        if (g * cpg != cc || g + 1 >= NG) return;
        if constexpr (ph == 0) load_offsets(g + 1);
        else build_table(((g + 1) & 1) * (kBoxMaxKK * NT));
      }
    };
    auto step = [&](int c, AFrag& af, const BFrag& bc, BFrag& bn) __attribute__((always_inline)) {
      table_work(c, std::integral_constant<int, 0>());
      bn = read_b(c + 1);
      // the column reads go out before the multiplies, so their latency hides behind them
      // (scheduled after, the barrier below would wait for the whole LDS round trip)
      __builtin_amdgcn_sched_barrier(0);
      mma(af, bc);
      af = load_a(min(c + 2 * G, S - 1));
      table_work(c, std::integral_constant<int, 1>());
      lds_barrier();
    };
    auto step_tail = [&](int c, AFrag& af, const BFrag& bc, BFrag& bn) __attribute__((always_inline)) {
      if (c >= S) return;
      table_work(c, std::integral_constant<int, 0>());
      if (c + 1 < S) bn = read_b(c + 1);
      __builtin_amdgcn_sched_barrier(0);
      mma(af, bc);
      if (c + 2 * G < S) af = load_a(c + 2 * G);
      table_work(c, std::integral_constant<int, 1>());
      if (c + 2 < S) lds_barrier();
    };
    if constexpr (!kSingleB) {
      BFrag b0{}, b1{};
      lds_barrier();                 // barrier 0: chunk 0 is produced
      b0 = read_b(0);
      if (S > 1) lds_barrier();      // barrier 1: chunk 1 is produced
      // 2G chunks per iteration (slots p0.. then q0..).  The loop runs while every step
      // of the iteration has all three parts, so its body has no branches.
      // step c + i of an iteration (c even): column fragments b0 -> b1 for even i
      auto run = [&](auto tail, int c, auto ic, AFrag& af) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if constexpr (decltype(tail)::value) {
          if constexpr ((i & 1) == 0) step_tail(c + i, af, b0, b1);
          else step_tail(c + i, af, b1, b0);
        } else {
          if constexpr ((i & 1) == 0) step(c + i, af, b0, b1);
          else step(c + i, af, b1, b0);
        }
      };
      int c = 0;
      for (; c + 2 * G + 2 <= S; c += 2 * G) {
        static_for<0, G>([&](auto ic) __attribute__((always_inline)) {
          run(std::false_type(), c, ic, pa[decltype(ic)::value]);
        });
        static_for<0, G>([&](auto ic) __attribute__((always_inline)) {
          run(std::false_type(), c, std::integral_constant<int, G + decltype(ic)::value>(), qa[decltype(ic)::value]);
        });
      }
      // at most 2G+1 chunks remain; the slots hold chunks c .. c+2G-1 and step c
      // reloads pa[0] with chunk c+2G
      static_for<0, G>([&](auto ic) __attribute__((always_inline)) {
        run(std::true_type(), c, ic, pa[decltype(ic)::value]);
      });
      static_for<0, G>([&](auto ic) __attribute__((always_inline)) {
        run(std::true_type(), c, std::integral_constant<int, G + decltype(ic)::value>(), qa[decltype(ic)::value]);
      });
      run(std::true_type(), c, std::integral_constant<int, 2 * G>(), pa[0]);
    } else {
      // One column buffer in registers (eight producer waves with the wider tiles,
      // where two would not fit in 168 registers): chunk c is read after barrier c,
      // when it is complete, and multiplied at once; the producers meanwhile write
      // chunk c+2 into another buffer of the ring.
      auto step1 = [&](int c, AFrag& af) __attribute__((always_inline)) {
        const BFrag bf = read_b(c);
        mma(af, bf);
        af = load_a(min(c + 2 * G, S - 1));
        if (c + 1 < S) lds_barrier();
      };
      lds_barrier();                 // barrier 0: chunk 0 is produced
      int c = 0;
      for (; c + 2 * G <= S; c += 2 * G) {
        static_for<0, G>([&](auto ic) __attribute__((always_inline)) { step1(c + decltype(ic)::value, pa[decltype(ic)::value]); });
        static_for<0, G>([&](auto ic) __attribute__((always_inline)) { step1(c + G + decltype(ic)::value, qa[decltype(ic)::value]); });
      }
      static_for<0, G>([&](auto ic) __attribute__((always_inline)) {
        if (c + decltype(ic)::value < S) step1(c + decltype(ic)::value, pa[decltype(ic)::value]);
      });
      static_for<0, G>([&](auto ic) __attribute__((always_inline)) {
        if (c + G + decltype(ic)::value < S) step1(c + G + decltype(ic)::value, qa[decltype(ic)::value]);
      });
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0) only; see the end of the producer branch

    // ---- epilogue, part 1: bias and bf16 rounding into an LDS copy of the output
    // tile, [pixel][row] with a pixel stride of MT+2 elements (an odd number of
    // dwords, so neighbouring pixels start in neighbouring banks), in the first box
    // buffer.  A lane's four consecutive rows of a pixel are one 8-byte write.  The producers read no box after barrier S-1, and the consumers pass
    // that barrier only after every producer's reads are complete.  The bias values
    // are loaded first; rows past Cout read the last bias value and are not stored.
    // Accumulator element r of a 32x32 block: row 8*(r/4) + 4*lh + r%4, column l32.
    float bv[TM][16] = {};
    if (a.bias) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          bv[tm][r] = ld_bf16(a.bias, min(m0 + wv * WM + tm * 32 + 8 * (r >> 2) + 4 * lh + (r & 3), a.Cout - 1));
    }
    uint32_t* stage = reinterpret_cast<uint32_t*>(box0);
    {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int row = wv * WM + tm * 32 + 8 * g + 4 * lh;   // even
            uint32_t* d = stage + ((tn * 32 + l32) * (MT + 2) + row) / 2;
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[tm][tn][4 * g + i] + bv[tm][4 * g + i];
            d[0] = pk_bf16(v[0], v[1]);
            d[1] = pk_bf16(v[2], v[3]);
          }
    }
  } else {
    // ================= producers: box copies and column tiles =================
    const int ptid = rtid;                  // producer thread 0..PTH-1
    // the global-path corners: this thread's unit within a pixel
    const uint32_t g_img_off =
        PW == 4 ? img_off   // the copy plan's lane offset is the same 16-byte quarter
                : static_cast<uint32_t>(b * a.H) * static_cast<uint32_t>(a.W * Cp) * 2u +
                      static_cast<uint32_t>((ptid & (UPS - 1)) * UB);

    // Producer state of one step: the corner-table entries and the four corner vectors
    // of this thread's samples.  A sample with nothing in the box reads the zero bytes
    // after the buffer with a row stride of 0.
    struct PSet { CEw ce[GU]; QV q[GU][4]; };
    // Samples whose corners lie outside the box (ce_global) take their corners from
    // the channels-last copy in global memory.  When a wave has any such sample in a
    // step (gfl, wave-uniform), its lanes load the four corner vectors straight into
    // registers (gq) one step ahead, right after the previous step's interpolation,
    // so the loads are in flight across a barrier; lanes without such a sample, and
    // corners outside the image, load zeros.  One step's vectors are live at a time.
    QV gq[GU][4];
    bool gfl[GU];
    // With one sample per thread and 3x3 taps the thread's nine table entries stay in
    // registers for the whole tile (the steps index them with compile-time taps), which
    // takes the table reads off every step.
    constexpr bool kCeRegs = GU == 1 && KKT == 9;
    constexpr int kCeN = kCeRegs ? 9 : 1;
    CEnt ce_r[kCeN];
    if constexpr (kCeRegs) {
#pragma unroll
      for (int k = 0; k < 9; ++k) ce_r[k] = get_ce(k * NT + (ptid >> UPS_SH));
    }
    // the entries of the nine taps from table tb into registers (offset groups: at
    // step 7 of a group's last chunk, when every entry of the current group is used)
    auto load_ce_regs = [&](int tb) __attribute__((always_inline)) {
      if constexpr (kCeRegs) {
#pragma unroll
        for (int k = 0; k < 9; ++k) ce_r[k] = get_ce(tb + k * NT + (ptid >> UPS_SH));
      }
    };
    auto read_ce = [&](int k, PSet& f, int tb) __attribute__((always_inline)) {
      if constexpr (kCeRegs) {
        // the weights are formed at each use (five instructions per step): formed once
        // for all nine taps they would hold 36 more registers for the whole tile
        CEnt e = ce_r[k];
        asm volatile("" : "+v"(e.a), "+v"(e.b), "+v"(e.lx));
        f.ce[0] = expand(e);
      } else {
#pragma unroll
        for (int g = 0; g < GU; ++g)
          if (GUNITS % PTH == 0 || pw * 64 + g * PTH < GUNITS)
            f.ce[g] = expand(get_ce(tb + k * NT + ((ptid + g * PTH) >> UPS_SH)));
      }
    };
    auto read_q = [&](const unsigned char* src, PSet& f) __attribute__((always_inline)) {
#pragma unroll
      for (int g = 0; g < GU; ++g) {
        if (GUNITS % PTH == 0 || pw * 64 + g * PTH < GUNITS) {
          const CEw& ce = f.ce[g];
          const bool in_box = ce.off >= 0;
          const unsigned char* q = src + (in_box ? ce.off : BOXB) + (ptid & (UPS - 1)) * UB;
          const int rs = in_box ? BW * kPXB : 0;
          f.q[g][0] = *reinterpret_cast<const QV*>(q);
          f.q[g][1] = *reinterpret_cast<const QV*>(q + kPXB);
          f.q[g][2] = *reinterpret_cast<const QV*>(q + rs);
          f.q[g][3] = *reinterpret_cast<const QV*>(q + rs + kPXB);
        }
      }
    };
    // the global-path corner vectors of the step (chunk cc, tap k) whose table entries are in f
    // (glob false: the wave has no global-path sample in any tap, and nothing is loaded)
    auto load_g = [&](int cc, int k, const PSet& f, int tb, auto glob) __attribute__((always_inline)) {
      if constexpr (!decltype(glob)::value) return;
#pragma unroll
      for (int g = 0; g < GU; ++g) {
        if (GUNITS % PTH == 0 || pw * 64 + g * PTH < GUNITS) {
          const CEw& ce = f.ce[g];
          gfl[g] = __ballot(ce_global(ce)) != 0;
          if (gfl[g]) {
            const __amdgpu_buffer_rsrc_t rsrc = chunk_rsrc(cc);
            const int yx = -ce.off - 3;
            const int y0 = (yx >> 16) - 1, x0 = (yx & 0xffff) - 1;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int yy = y0 + (qq >> 1), xx = x0 + (qq & 1);
              const bool ok = ce_global(ce) & (yy >= 0) & (yy < a.H) & (xx >= 0) & (xx < a.W);
              const uint32_t voff =
                  ok ? g_img_off + static_cast<uint32_t>(yy) * row_bytes + static_cast<uint32_t>(xx) * px_bytes : kOOB;
              buffer_load_q(rsrc, voff, gq[g][qq]);
            }
          }
        }
      }
    };
    // interpolate and store into column buffer s % 3
    auto finish = [&](int s, const PSet& f, auto glob) __attribute__((always_inline)) {
      unsigned char* cdst = col + (s % kColBufs) * NT * kCOLB;
#pragma unroll
      for (int g = 0; g < GU; ++g) {
        if (GUNITS % PTH == 0 || pw * 64 + g * PTH < GUNITS) {
          const int u = ptid + g * PTH;
          const int p = u >> UPS_SH, sub = u & (UPS - 1);
          const CEw& ce = f.ce[g];
          QV c0 = f.q[g][0], c1 = f.q[g][1], c2 = f.q[g][2], c3 = f.q[g][3];
          if constexpr (decltype(glob)::value) {
            if (gfl[g]) {   // wave-uniform: some lane's sample takes the global-path corners
              const bool o = ce_global(ce);
              c0 = sel4(o, gq[g][0], c0);
              c1 = sel4(o, gq[g][1], c1);
              c2 = sel4(o, gq[g][2], c2);
              c3 = sel4(o, gq[g][3], c3);
            }
          }
          const QV r = interp8(c0, c1, c2, c3, ce.w);
          *reinterpret_cast<QV*>(cdst + p * kCOLB + sub * UB) = r;
        }
      }
    };

    // Chunks alternate between the two box buffers.  The buffer of each chunk is a
    // compile-time choice (the two parities are laid out one after the other, never
    // behind a runtime pointer select), so every LDS access names its array and only
    // waits for copies into that array.  Each chunk starts copying the next chunk's
    // box into the other buffer and waits for that copy before its last barrier.
    PSet X, Y;
    if constexpr (KKT == 9) {
      // Three kernel points: the nine steps of a chunk are unrolled and software
      // pipelined over register sets.  The next chunk's box is copied during steps 0-3;
      // each wave waits for its part before barrier 6, after which the whole box is in
      // LDS and steps 7 and 8 read the corners of the next chunk's steps 0 and 1 from it.
      constexpr int kRd = 4;                             // corner reads per sample
      constexpr int kKeep = GU * (kRd + 1) < 15 ? GU * (kRd + 1) : 15;   // LDS reads issued after the column stores
      // One sample per thread: each step interpolates the NEXT step's column, so its
      // column store stays in flight across the barrier (the consumers read it only
      // after the next one) and no store latency is on a step's critical path.  Two
      // register sets, step j's data in set j % 2 (the parity flips with each
      // nine-step chunk).  Step k of chunk cc (global step s):
      //   1. reads the corners of step s+2 into set s % 2, whose step s was
      //      interpolated during step k-1 (box of the next chunk from step 7 on,
      //      after barrier 6);
      //   2. issues its share of the next chunk's box copy (k < 4);
      //   3. interpolates step s+1 from corners read a step earlier and stores it;
      //   4. loads the global-path corners of step s+2.
      // The corner-table entries of all nine taps are in registers.
      auto chunk9w = [&](int cc, auto parity, auto glob) __attribute__((always_inline)) {
        constexpr bool odd = decltype(parity)::value;
        const unsigned char* src = odd ? box1 : box0;
        unsigned char* dst = odd ? box0 : box1;
        const int t_cur = table_of_chunk(cc);
        const int t_nxt = table_of_chunk(cc + 1);
        static_for<0, 9>([&](auto kc) __attribute__((always_inline)) {
          constexpr int k = decltype(kc)::value;
          PSet& s0 = ((k + (odd ? 1 : 0)) & 1) == 0 ? X : Y;   // set of steps s and s+2
          PSet& s1 = ((k + (odd ? 1 : 0)) & 1) == 0 ? Y : X;   // set of step s+1
          if constexpr (GRP && k == 7) {
            if (cc + 1 < nCC && t_nxt != t_cur) load_ce_regs(t_nxt);
          }
          read_ce((k + 2) % 9, s0, t_cur);
          if constexpr (k + 2 < 9) {
            read_q(src, s0);
          } else {
            // the next chunk's steps 0 and 1 (a dummy re-read of this box after the last chunk)
            if (cc + 1 < nCC) read_q(dst, s0);
            else read_q(src, s0);
          }
          if constexpr (k < 4) copy_part4(cc + 1, dst, kc);
          const bool last = k == 8 && cc + 1 == nCC;   // no step s+1
          if (!last) finish(cc * 9 + k + 1, s1, glob);
          load_g(k < 7 ? cc : cc + 1, (k + 2) % 9, s0, k < 7 ? t_cur : t_nxt, glob);
          if constexpr (k == 6) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          // keep the corner reads and the column store in flight; the previous step's
          // store (older) is complete
          if (!last) lds_barrier_keep<kRd + 1>();
          else lds_barrier_keep<kRd>();
        });
      };
      // With more than one sample per thread three sets would not fit in registers:
      // two sets, step k using set (k + chunk parity) % 2, corners read one step ahead.
      auto chunk9_two = [&](int cc, auto parity) __attribute__((always_inline)) {
        constexpr bool odd = decltype(parity)::value;
        const unsigned char* src = odd ? box1 : box0;
        unsigned char* dst = odd ? box0 : box1;
        const int t_cur = table_of_chunk(cc);
        const int t_nxt = table_of_chunk(cc + 1);
        static_for<0, 9>([&](auto kc) __attribute__((always_inline)) {
          constexpr int k = decltype(kc)::value;
          PSet& cur = ((k + (odd ? 1 : 0)) & 1) == 0 ? X : Y;
          PSet& oth = ((k + (odd ? 1 : 0)) & 1) == 0 ? Y : X;
          if constexpr (k < 4) copy_part4(cc + 1, dst, kc);
          finish(cc * 9 + k, cur, std::true_type());
          if constexpr (k < 8) load_g(cc, k + 1, oth, t_cur, std::true_type());
          asm volatile("" ::: "memory");
          if constexpr (k + 1 < 9) read_q(src, oth);
          read_ce((k + 2) % 9, cur, k + 2 < 9 ? t_cur : t_nxt);
          if constexpr (k == 8) {
            __builtin_amdgcn_s_waitcnt(0);
            lds_barrier_dma();
            if (cc + 1 < nCC) {
              read_q(dst, oth);
              load_g(cc + 1, 0, oth, t_nxt, std::true_type());
            }
          } else {
            lds_barrier_keep<kKeep>();
          }
        });
      };
      if constexpr (GU == 1) {
        auto run = [&](auto glob) __attribute__((always_inline)) {
          read_ce(0, X, 0);
          read_q(box0, X);
          read_ce(1, Y, 0);
          read_q(box0, Y);
          load_g(0, 0, X, 0, glob);
          finish(0, X, glob);          // column 0, before the loop
          load_g(0, 1, Y, 0, glob);
          for (int cc = 0; cc < nCC; cc += 2) {
            chunk9w(cc, std::false_type(), glob);
            if (cc + 1 < nCC) chunk9w(cc + 1, std::true_type(), glob);
          }
        };
        // A wave none of whose samples (all nine taps, one offset group) leaves the box
        // runs the loop without the global path: no ballot, branch or select per step.
        // Both versions pass the same barriers.
        bool anyg = false;
#pragma unroll
        for (int k = 0; k < 9; ++k) anyg |= ce_r[k].off <= -3;
        if (!GRP && __ballot(anyg) == 0) run(std::false_type());
        else run(std::true_type());
      } else {
        read_ce(0, X, 0);
        read_ce(1, Y, 0);
        read_q(box0, X);
        load_g(0, 0, X, 0, std::true_type());
        for (int cc = 0; cc < nCC; cc += 2) {
          chunk9_two(cc, std::false_type());
          if (cc + 1 < nCC) chunk9_two(cc + 1, std::true_type());
        }
      }
    } else {
      // any other kernel size: one step at a time, the entries and corners of each
      // step read at its start
      auto chunk = [&](int cc, auto parity) __attribute__((always_inline)) {
        constexpr bool odd = decltype(parity)::value;
        const unsigned char* src = odd ? box1 : box0;
        unsigned char* dst = odd ? box0 : box1;
        if (cc + 1 < nCC) copy_box(cc + 1, dst);
        for (int k = 0; k < KK; ++k) {
          read_ce(k, X, 0);
          read_q(src, X);
          load_g(cc, k, X, 0, std::true_type());
          finish(cc * KK + k, X, std::true_type());
          if (k == KK - 1 && cc + 1 < nCC) __builtin_amdgcn_s_waitcnt(0);
          lds_barrier_dma();
        }
      };
      for (int cc = 0; cc < nCC; cc += 2) {
        chunk(cc, std::false_type());
        if (cc + 1 < nCC) chunk(cc + 1, std::true_type());
      }
    }
    // S barriers here match the consumers' S barriers.  The role branches are laid out
    // one after the other in the compiled code, so loads still counted at the end of
    // one look pending to the other; drain them here (nothing useful is in flight).
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0) only
  }

  // ---- epilogue, part 2 (all waves): NCHW stores of the tile, along its rows, two
  // pixels per 4-byte store where the element index is even
  static_assert(NT * (MT + 2) * 2 <= BOXB, "output tile must fit in a box buffer");
  __syncthreads();
  {
    // Thread -> (column pair of a tile row, first row).  Pairs are aligned to even
    // output columns, so with even Wo and Ho*Wo a pair with both columns in the tile
    // is one aligned 4-byte store.  Rows advance by a fixed stride with the (row,
    // channel) split kept incrementally; LDS reads are unconditional (clamped index)
    // so the loop has no divisions and no branch around a read.
    const uint16_t* stage = reinterpret_cast<const uint16_t*>(box0);
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
    const int TH = ba.TH, TW = ba.TW;
    const int xs0 = ox0 & ~1;
    const int slots = (ox0 - xs0 + TW + 1) >> 1;
    const int rows = MT * TH, rstep = NTH / slots;
    const int slot = tid % slots, r0 = tid / slots;
    const int c0 = xs0 + slot * 2, xend = min(ox0 + TW, a.Wo);
    const bool in0 = c0 >= ox0 && c0 < xend, in1 = c0 + 1 >= ox0 && c0 + 1 < xend;
    const int q0 = max(c0 - ox0, 0), q1 = min(c0 + 1 - ox0, TW - 1);
    const bool pair = in0 && in1 && (a.Wo & 1) == 0 && (a.HoWo & 1) == 0;
    if (r0 < rstep && (in0 || in1)) {
      const int dol = rstep / TH, dpy = rstep - (rstep / TH) * TH;
      int ol = r0 / TH, py = r0 - (r0 / TH) * TH;
#pragma unroll 4
      for (int r = r0; r < rows; r += rstep) {
        const int o = m0 + ol, oy = oy0 + py;
        const uint16_t* src = stage + (py * TW) * (MT + 2) + ol;
        const uint32_t v0 = src[q0 * (MT + 2)], v1 = src[q1 * (MT + 2)];
        if (o < a.Cout && oy < a.Ho) {
          uint16_t* dst = out;
          const int e = (b * a.Cout + o) * a.HoWo + oy * a.Wo + c0;
          if (pair) {
            *reinterpret_cast<uint32_t*>(dst + e) = v0 | (v1 << 16);
          } else {
            if (in0) dst[e] = static_cast<uint16_t>(v0);
            if (in1) dst[e + 1] = static_cast<uint16_t>(v1);
          }
        }
        ol += dol;
        py += dpy;
        if (py >= TH) {
          py -= TH;
          ++ol;
        }
      }
    }
  }
}

constexpr bool box_groups_built(int fm, int fn) { return fn <= 8 && !(fm == 4 && fn == 6); }
constexpr bool box_pw8_built(int fm, int fn) { return (fm == 4 && fn <= 6) || (fm == 2 && fn >= 8); }


// optional instances per tile shape (must agree with box_pw8_built / box_groups_built)
#define DCN_BOX_IF_2_4(KW) KW __global__ void dcn_box_kernel<2, 4, 9, true, 4>(BoxArgs);
#define DCN_BOX_IF_2_6(KW) KW __global__ void dcn_box_kernel<2, 6, 9, true, 4>(BoxArgs);
#define DCN_BOX_IF_2_8(KW) KW __global__ void dcn_box_kernel<2, 8, 9, false, 8>(BoxArgs); KW __global__ void dcn_box_kernel<2, 8, 9, true, 4>(BoxArgs);
#define DCN_BOX_IF_2_10(KW) KW __global__ void dcn_box_kernel<2, 10, 9, false, 8>(BoxArgs);
#define DCN_BOX_IF_4_4(KW) KW __global__ void dcn_box_kernel<4, 4, 9, false, 8>(BoxArgs); KW __global__ void dcn_box_kernel<4, 4, 9, true, 4>(BoxArgs);
#define DCN_BOX_IF_4_6(KW) KW __global__ void dcn_box_kernel<4, 6, 9, false, 8>(BoxArgs);

// The instances built for one (FM, FN): eight producer waves where built, any K*K <= 9, offset groups where built, and the 3x3 schedule.
// DCN_BOX_INSTANCES(template, ...) instantiates them; with "extern template" it declares
// them for the launcher.
#define DCN_BOX_INSTANCES(KW, FM, FN)                                                          \
  KW __global__ void dcn_box_kernel<FM, FN, 0, false, 4>(BoxArgs);                     \
  KW __global__ void dcn_box_kernel<FM, FN, 9, false, 4>(BoxArgs);                     \
  DCN_BOX_IF_##FM##_##FN(KW)

}  // namespace dcn
