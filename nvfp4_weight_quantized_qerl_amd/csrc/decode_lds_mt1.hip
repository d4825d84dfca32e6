// Instantiations of the LDS-staged decode contraction for 1 token tile(s).
#include "decode_lds.h"

namespace qerl {
namespace dlds {

Kernel pick_mt1(int nt, bool p2) { return p2 ? pick_nt<1, true>(nt) : pick_nt<1>(nt); }

}  // namespace dlds
}  // namespace qerl
