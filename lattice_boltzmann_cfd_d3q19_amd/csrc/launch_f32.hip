// launch_f32.hip -- fp32 instantiation of the step and state-transfer launchers.
#include "launch_impl.hpp"

namespace lbm {
template hipError_t launch_step<float>(int, int, float*, float*, const LaunchGeom&, const LaunchPhys&, float*, float*,
                                       hipStream_t);
template hipError_t launch_io<float>(int, int, int, float*, float*, const LaunchGeom&, const LaunchPhys&,
                                     float*, float*, const float*, const float*, hipStream_t);
template hipError_t launch_step_compact<float>(int, float*, float*, const LaunchGeom&, const CompactTables&,
                                               const LaunchPhys&, float*, float*, hipStream_t);
template hipError_t launch_io_compact<float>(int, int, float*, const LaunchGeom&, const CompactTables&,
                                             const LaunchPhys&, float*, float*, const float*, const float*, hipStream_t);
template hipError_t launch_face_rules<float>(int, int, float*, const LaunchGeom&, const CompactTables*, const LaunchPhys&,
                                            hipStream_t);
template hipError_t launch_momentum_exchange<float>(int, int, float*, const LaunchGeom&, const CompactTables*,
                                                    const LaunchPhys&, double*, double*, hipStream_t);
template hipError_t launch_step_mex<float>(int, int, float*, float*, const LaunchGeom&, const CompactTables*,
                                          const LaunchPhys&, double*, double*, hipStream_t);

// workgroups of the momentum-exchange pass (precision-independent)
size_t mex_partial_rows(const LaunchGeom& g) { return make_shape(g).grid.x; }
}  // namespace lbm
