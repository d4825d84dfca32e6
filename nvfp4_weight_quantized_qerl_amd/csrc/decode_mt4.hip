// Instantiations of the decode contraction for 4 token tile(s) of 32.
#include "decode_kernel.h"

namespace qerl {
namespace decode {

DecodeKernel pick_mt4(int nt) { return pick_mt<4>(nt); }

}  // namespace decode
}  // namespace qerl
