// Batched (many-token) expert FFN.  Placeholder: runs the decode kernels for every token until
// the grouped MFMA path lands.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

size_t grouped_workspace_extra(int T, int K, int E, int d) {
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  return al((size_t)E * 4) + al((size_t)(E + 1) * 4) + al((size_t)T * K * 4) + al((size_t)T * K * d * 4);
}

hipError_t launch_expert_grouped(hipStream_t s, const GroupedArgs& a) { return launch_expert_decode(s, a.base); }

}  // namespace moe
