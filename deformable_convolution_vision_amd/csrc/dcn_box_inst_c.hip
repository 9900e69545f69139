// dcn_box_inst_c.hip -- instances of the box kernel (dcn_box_kernel.h) for the
// tile shapes 128 x 160 (output channels x pixel slots).

#include "dcn_box_kernel.h"

namespace dcn {

DCN_BOX_INSTANCES(template, 2, 10)

}  // namespace dcn
