// dcn_box_inst_d.hip -- instances of the box kernel (dcn_box_kernel.h) for the
// tile shapes 256 x 64, 256 x 96 (output channels x pixel slots).

#include "dcn_box_kernel.h"

namespace dcn {

DCN_BOX_INSTANCES(template, 4, 4)
DCN_BOX_INSTANCES(template, 4, 6)

}  // namespace dcn
