// Instantiations of the decode contraction for 1 token tile(s) of 32.
#include "decode_kernel.h"

namespace qerl {
namespace decode {

DecodeKernel pick_mt1(int nt) { return pick_mt<1>(nt); }

}  // namespace decode
}  // namespace qerl
