#include "av_device.hpp"
#include "av_kernels.hpp"
namespace av {
size_t evo_workspace_bytes(int Ns, int Nr, int H, int dh) { return (size_t)4 * Ns * Nr * H * dh * 2; }
hipError_t launch_evoformer(const EvoArgs&, hipStream_t) { return hipErrorNotSupported; }
}
