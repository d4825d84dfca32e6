// Instantiations of the LDS-staged decode contraction for 2 token tile(s).
#include "decode_lds.h"

namespace qerl {
namespace dlds {

Kernel pick_mt2(int nt, bool p2) { return p2 ? pick_nt<2, true>(nt) : pick_nt<2>(nt); }

}  // namespace dlds
}  // namespace qerl
