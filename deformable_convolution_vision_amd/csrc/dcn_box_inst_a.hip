// dcn_box_inst_a.hip -- instances of the box kernel (dcn_box_kernel.h) for the
// tile shapes 128 x 64, 128 x 96 (output channels x pixel slots).

#include "dcn_box_kernel.h"

namespace dcn {

DCN_BOX_INSTANCES(template, 2, 4)
DCN_BOX_INSTANCES(template, 2, 6)

}  // namespace dcn
