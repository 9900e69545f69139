// dcn_box.hip -- launcher of the box kernel (dcn_box_kernel.h): instance choice per
// tile shape and schedule, LDS capacity queries for the planner.  The instances are
// compiled in dcn_box_inst_*.hip.

#include "dcn_box_kernel.h"

namespace dcn {

DCN_BOX_INSTANCES(extern template, 2, 4)
DCN_BOX_INSTANCES(extern template, 2, 6)
DCN_BOX_INSTANCES(extern template, 2, 8)
DCN_BOX_INSTANCES(extern template, 2, 10)
DCN_BOX_INSTANCES(extern template, 4, 4)
DCN_BOX_INSTANCES(extern template, 4, 6)

template <int FM, int FN>
static hipError_t launch_box_t(const BoxArgs& ba, hipStream_t stream) {
  void* args[] = {const_cast<BoxArgs*>(&ba)};
  const dim3 grid(ba.f.m_tiles * ba.tiles_per_img * ba.f.B);
  const void* fn = nullptr;
  if (ba.f.om_split > 0) return hipErrorInvalidValue;   // the offset/mask branch has its own kernel
  if (ba.pw == 8) {   // eight producer waves: 3x3, one offset group, paired roles
    if constexpr (box_pw8_built(FM, FN)) {
      if (ba.f.KK != 9 || ba.f.G > 1 || ba.split_roles) return hipErrorInvalidValue;
      return hipLaunchKernel(reinterpret_cast<const void*>(&dcn_box_kernel<FM, FN, 9, false, 8>), grid,
                             dim3(256 + 64 * 8), args, 0, stream);
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (ba.f.KK != 9) {
    fn = reinterpret_cast<const void*>(&dcn_box_kernel<FM, FN, 0, false>);
  } else if (ba.f.G > 1) {
    // two corner tables leave too little LDS for the output staging of 160 slots, and
    // 256 x 96 tiles too few registers for the consumers' table work
    if constexpr (box_groups_built(FM, FN)) fn = reinterpret_cast<const void*>(&dcn_box_kernel<FM, FN, 9, true>);
    else return hipErrorInvalidValue;
  } else {
    fn = reinterpret_cast<const void*>(&dcn_box_kernel<FM, FN, 9, false>);
  }
  return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, stream);
}

hipError_t launch_box(int fm, int fn, const BoxArgs& ba, hipStream_t stream) {
#define DCN_BOX_CASE(FMv, FNv) \
  if (fm == FMv && fn == FNv) return launch_box_t<FMv, FNv>(ba, stream);
  DCN_BOX_CASE(2, 4) DCN_BOX_CASE(2, 6) DCN_BOX_CASE(2, 8) DCN_BOX_CASE(2, 10)
  DCN_BOX_CASE(4, 4) DCN_BOX_CASE(4, 6)
#undef DCN_BOX_CASE
  return hipErrorInvalidValue;
}

bool box_groups_supported(int fm, int fn) { return box_groups_built(fm, fn); }
bool box_pw8_supported(int fm, int fn) { return box_pw8_built(fm, fn); }

int box_capacity_px(int fn, bool groups) {
  switch (fn) {
    case 4: return groups ? BoxCfg<4, true>::BOX_PX : BoxCfg<4>::BOX_PX;
    case 6: return groups ? BoxCfg<6, true>::BOX_PX : BoxCfg<6>::BOX_PX;
    case 8: return groups ? BoxCfg<8, true>::BOX_PX : BoxCfg<8>::BOX_PX;
    case 10: return groups ? 0 : BoxCfg<10>::BOX_PX;   // no offset-group kernel for 160 slots
    default: return 0;
  }
}

}  // namespace dcn
