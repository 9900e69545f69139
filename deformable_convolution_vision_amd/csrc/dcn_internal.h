// dcn_internal.h -- launch interface between the host API (dcn_api.hip) and the
// gfx950 kernels (dcn_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct dcn_desc;

namespace dcn {

// Descriptor checks shared by every entry point: geometry, dtype, the output size
// (Ho, Wo >= 1) and float-exact base positions.  DCN_OK or a negative dcn_status.
int check_desc(const dcn_desc* d, int64_t* Ho, int64_t* Wo);

// Everything the fused kernel needs; all sizes fit int32 (checked on the host).
struct FusedArgs {
  const void* xs;      // staged x, channels last: [B][H][W][Cp]
  const void* wp;      // repacked weight: [Mp][K*K][Cp], zero rows/channels beyond Cout/Cin
  const void* x;       // x as given, [B][Cin][H][W] (direct variants only)
  const void* w;       // weight as given, [Cout][Cin][K][K] (direct variants only)
  const void* offset;  // [B][2G K^2][Ho][Wo]
  const void* mask;    // [B][G K^2][Ho][Wo] or null
  const void* bias;    // [Cout] or null
  void* out;           // [B][Cout][Ho][Wo]
  int B, Cin, H, W, Cp, Cout, K, KK, stride, pad, dil, Ho, Wo, HoWo, N;
  int m_tiles, n_tiles;
  int G, Cg;           // offset groups and channels per group (1 and Cin for one group)
  // The offset/mask branch (tile kernels): offset == null samples at zero offsets (a
  // regular convolution); with om_split > 0 the output channels o < om_split go to out
  // as [B][om_split][Ho][Wo] and the others, through a sigmoid, to out2 as
  // [B][Cout - om_split][Ho][Wo].
  void* out2;
  int om_split;
};

struct StageArgs {
  const void* x;   // [B][Cin][H][W]
  const void* w;   // [Cout][Cin][K][K]
  void* xs;        // [B][H*W][Cp]
  void* wp;        // wlayout 0: [Mp][KK][Cp]; wlayout 1: [Cp/32 * KK][Mp][32] (step-major);
                   // wlayout 2: [KK * Cp/16][Mp][16] (tap-major 16-channel steps)
  int B, Cin, HW, Cp, Cout, Mp, KK;
  int wlayout;
  // an optional second weight of the same input (w2 null: none), repacked by the same
  // launch: [Cout2][Cin][K][K] -> wp2 in wlayout2 with Mp2 rows
  const void* w2;
  void* wp2;
  int Cout2, Mp2, wlayout2;
  int nw2;         // workgroups repacking the second weight (set by launch_stage)
};

// The offset/mask branch as a regular convolution on the staged channels-last input:
// M = 3*G*K*K outputs, the first `split` (2*G*K*K) written to offset, the sigmoid of the
// rest to mask, both [B][channels][Ho][Wo], bf16.
struct OmArgs {
  const void* xs;      // [B][H][W][Cp] bf16
  const void* wp;      // [KK * Cp/16][Mp][16] bf16 (wlayout 2)
  const void* bias;    // [M] bf16 or null
  void* offset;        // [B][split][Ho][Wo]
  void* mask;          // [B][M - split][Ho][Wo]
  int B, H, W, Cp, M, Mp, K, KK, stride, pad, dil, Ho, Wo, HoWo, N, split;
};

// Box kernel (bf16): FusedArgs plus the output-tile geometry and the LDS budget.
struct BoxArgs {
  FusedArgs f;
  int TH, TW;            // output tile: TH rows x TW columns of one image
  int tiles_x;           // tiles per output row of tiles
  int tiles_per_img;
  int box_px;            // capacity of one LDS box buffer, in pixels
  int KK_NT;             // corner-table entries: K*K * 16*FN
  int lds_bytes;         // dynamic LDS per workgroup
  int split_roles;       // 0: each SIMD runs one consumer and one producer wave;
                         // 1: the consumers share two SIMDs, the producers the other two
  int pw;                // producer waves: 4 (512 threads) or 8 (768 threads)
};

enum Variant : int {
  V_TILE_F32_M64_N64 = 0,
  V_TILE_F32_M128_N64,
  V_TILE_BF16_M64_N64,
  V_TILE_BF16_M128_N64,
  V_TILE_BF16_M128_N32,
  V_TILE_BF16_M256_N64,
  V_BOX_BF16_M128,
  V_BOX_BF16_M256,
  V_DIRECT_F32,
  V_DIRECT_BF16,
  V_OM_BF16,       // the offset/mask branch's regular convolution (dcn_om.hip)
  V_COUNT
};

struct VariantInfo {
  const char* name;
  int is_bf16;
  int mt, nt;      // tile of the fused kernel: MT output channels x NT output pixels
  int ck;          // channels per reduction chunk (Cp is a multiple of it)
  int staged;      // 1: needs dcn_stage's workspace
};

const VariantInfo& variant_info(int v);

hipError_t launch_stage(int variant, const StageArgs& a, hipStream_t stream);
hipError_t launch_fused(int variant, const FusedArgs& a, hipStream_t stream);

// box kernel: fm = MT/64 (2: fn 4, 6, 8, 10; 4: fn 4, 6), fn = NT/16; offset groups
// (f.G > 1) with K = 3 and 32-channel multiples per group.
// box_capacity_px: pixels one LDS box buffer holds for a given fn, with one corner
// table or (groups) two (0 if not built).
hipError_t launch_box(int fm, int fn, const BoxArgs& a, hipStream_t stream);
int box_capacity_px(int fn, bool groups);
bool box_groups_supported(int fm, int fn);   // an offset-group kernel is built for (fm, fn)
bool box_pw8_supported(int fm, int fn);      // an eight-producer-wave kernel is built for (fm, fn)

// the offset/mask branch's convolution (bf16, staged input, weight in wlayout 2)
hipError_t launch_om(const OmArgs& a, hipStream_t stream);

// direct kernel (no staging): Cin <= 4 and K*K in {1, 4, 9}
bool direct_supported(int cin, int kk);
hipError_t launch_direct(bool bf16, const FusedArgs& a, hipStream_t stream);
constexpr int kLdsBudget = 160 * 1024;   // LDS per workgroup on gfx950
constexpr int kBoxMaxKK = 9;             // the box kernel handles K*K <= 9

}  // namespace dcn
