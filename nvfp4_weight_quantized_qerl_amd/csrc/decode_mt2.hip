// Instantiations of the decode contraction for 2 token tile(s) of 32.
#include "decode_kernel.h"

namespace qerl {
namespace decode {

DecodeKernel pick_mt2(int nt) { return pick_mt<2>(nt); }

}  // namespace decode
}  // namespace qerl
