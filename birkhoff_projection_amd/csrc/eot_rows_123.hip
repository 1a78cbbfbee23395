// eot_rows_123.hip -- explicit instantiations of the general entropic-OT kernels for
// n = 1, 2, 3 rows (all column counts); see eot_launch.hpp.
#include "eot_launch.hpp"

namespace birk {
namespace eot {
template int by_m<1, FwdArgs>(int, const FwdArgs&);
template int by_m<1, BwdArgs>(int, const BwdArgs&);
template int by_m<2, FwdArgs>(int, const FwdArgs&);
template int by_m<2, BwdArgs>(int, const BwdArgs&);
template int by_m<3, FwdArgs>(int, const FwdArgs&);
template int by_m<3, BwdArgs>(int, const BwdArgs&);
}  // namespace eot
}  // namespace birk
