// launch_f64.hip -- fp64 instantiation of the step and state-transfer launchers.
#include "launch_impl.hpp"

namespace lbm {
template hipError_t launch_step<double>(int, int, double*, double*, const LaunchGeom&, const LaunchPhys&, double*, double*,
                                        hipStream_t);
template hipError_t launch_io<double>(int, int, int, double*, double*, const LaunchGeom&, const LaunchPhys&,
                                      double*, double*, const double*, const double*, hipStream_t);
template hipError_t launch_step_compact<double>(int, double*, double*, const LaunchGeom&, const CompactTables&,
                                               const LaunchPhys&, double*, double*, hipStream_t);
template hipError_t launch_io_compact<double>(int, int, double*, const LaunchGeom&, const CompactTables&,
                                             const LaunchPhys&, double*, double*, const double*, const double*, hipStream_t);
template hipError_t launch_face_rules<double>(int, int, double*, const LaunchGeom&, const CompactTables*, const LaunchPhys&,
                                            hipStream_t);
template hipError_t launch_momentum_exchange<double>(int, int, double*, const LaunchGeom&, const CompactTables*,
                                                    const LaunchPhys&, double*, double*, hipStream_t);
template hipError_t launch_step_mex<double>(int, int, double*, double*, const LaunchGeom&, const CompactTables*,
                                          const LaunchPhys&, double*, double*, hipStream_t);
}  // namespace lbm
