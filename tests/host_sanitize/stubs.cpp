// Launch stubs for the host-only build of the library's host layer: every
// launch record the validation accepts arrives here and is counted instead
// of launched, so the argument checks and the planner run without a GPU.
#include "cam_internal.h"

namespace cam {
long g_launches = 0;
cam_status launch_dense_relayout(const DenseRelayout&, void*) { ++g_launches; return CAM_OK; }
cam_status launch_varlen_relayout(const VarlenRelayout&, void*) { ++g_launches; return CAM_OK; }
cam_status launch_pack(const Pack&, void*) { ++g_launches; return CAM_OK; }
cam_status launch_combine(const Combine&, void*) { ++g_launches; return CAM_OK; }
cam_status launch_copy(const Copy&, void*) { ++g_launches; return CAM_OK; }
cam_status launch_dense_lds(const DenseLds&, void*) { ++g_launches; return CAM_OK; }
cam_status launch_merge(const Merge&, void*) { ++g_launches; return CAM_OK; }
cam_status launch_combine_bwd(const CombineBwd&, void*) { ++g_launches; return CAM_OK; }
cam_status launch_proj(const Proj&, void*) { ++g_launches; return CAM_OK; }
}  // namespace cam
