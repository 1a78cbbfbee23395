// eot_rows_67.hip -- explicit instantiations of the general entropic-OT kernels for
// n = 6, 7 rows (all column counts); see eot_launch.hpp.
#include "eot_launch.hpp"

namespace birk {
namespace eot {
template int by_m<6, FwdArgs>(int, const FwdArgs&);
template int by_m<6, BwdArgs>(int, const BwdArgs&);
template int by_m<7, FwdArgs>(int, const FwdArgs&);
template int by_m<7, BwdArgs>(int, const BwdArgs&);
}  // namespace eot
}  // namespace birk
