// Instantiations of the LDS-staged decode contraction for 1 token tile(s).
#include "decode_lds.h"

namespace qerl {
namespace dlds {

Kernel pick_mt1(int nt) { return pick_nt<1>(nt); }

}  // namespace dlds
}  // namespace qerl
