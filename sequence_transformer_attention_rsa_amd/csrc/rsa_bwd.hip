// rsa_bwd.hip -- Ring Self-Attention backward for gfx950 (in progress).

#include "rsa_device.h"
#include "rsa_internal.h"

namespace rsa {

size_t backward_workspace_bytes(int B, int H, int L, int d) {
    (void)d;
    return (size_t)B * H * L * sizeof(float);
}

hipError_t launch_backward(const BackwardCall& c, hipStream_t stream) {
    (void)c;
    (void)stream;
    return hipErrorNotSupported;
}

}  // namespace rsa
