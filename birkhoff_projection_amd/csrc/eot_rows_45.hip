// eot_rows_45.hip -- explicit instantiations of the general entropic-OT kernels for
// n = 4, 5 rows (all column counts); see eot_launch.hpp.
#include "eot_launch.hpp"

namespace birk {
namespace eot {
template int by_m<4, FwdArgs>(int, const FwdArgs&);
template int by_m<4, BwdArgs>(int, const BwdArgs&);
template int by_m<5, FwdArgs>(int, const FwdArgs&);
template int by_m<5, BwdArgs>(int, const BwdArgs&);
}  // namespace eot
}  // namespace birk
