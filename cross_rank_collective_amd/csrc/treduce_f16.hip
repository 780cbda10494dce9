// treduce_f16.hip -- launchers for f16 elements: the copy and push-with-add
// kernel instances, and the per-operator selection of the reduction and ring
// instances (treduce_op.hip).
#include "treduce_launch.hpp"

namespace ptored {

int launch_f16(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_dtype<PTORED_F16, 2>(p, a, cu_count, stream);
}

int launch_ring_f16(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_ring<PTORED_F16>(p, a, cu_count, stream);
}

}  // namespace ptored
