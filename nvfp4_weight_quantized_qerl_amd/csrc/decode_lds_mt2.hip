// Instantiations of the LDS-staged decode contraction for 2 token tile(s).
#include "decode_lds.h"

namespace qerl {
namespace dlds {

Kernel pick_mt2(int nt) { return pick_nt<2>(nt); }

}  // namespace dlds
}  // namespace qerl
