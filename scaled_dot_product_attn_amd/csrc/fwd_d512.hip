#include "kernels.h"
namespace attn {
hipError_t launch_fused_d512(const FwdArgs&) { return hipErrorNotSupported; }
}
