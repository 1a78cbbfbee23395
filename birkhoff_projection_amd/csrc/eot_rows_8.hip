// eot_rows_8.hip -- explicit instantiations of the general entropic-OT kernels for
// n = 8 rows (all column counts); see eot_launch.hpp.
#include "eot_launch.hpp"

namespace birk {
namespace eot {
template int by_m<8, FwdArgs>(int, const FwdArgs&);
template int by_m<8, BwdArgs>(int, const BwdArgs&);
}  // namespace eot
}  // namespace birk
