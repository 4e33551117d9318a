// Stand-ins for the kernel launchers, linked only into the sanitizer build of
// the host ABI code (libdiffattn_san.so) that the CPU tests load: those tests
// exercise argument validation, which returns before any launch, so reaching
// one of these is itself an error.
#include "../differential_attention_forward_amd/csrc/kernels.h"

namespace diffattn {
hipError_t launch_fwd(const FwdArgs&, int, int, bool, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode(const DecodeArgs&, int, int, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode_v2(const DecodeArgs&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attention(const FwdArgs&, int, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_v2(const FwdArgs&, int, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t decode_scratch(void**) { return hipErrorNotSupported; }
hipError_t launch_bwd(const BwdArgs&, int, bool, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_lambda(const float*, const float*, const float*, const float*, int, int, float, float*,
                         hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace diffattn
