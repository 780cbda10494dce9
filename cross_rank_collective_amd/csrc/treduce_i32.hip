// treduce_i32.hip -- launchers for i32 elements: the copy and push-with-add
// kernel instances, and the per-operator selection of the reduction and ring
// instances (treduce_op.hip).
#include "treduce_launch.hpp"

namespace ptored {

int launch_i32(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_dtype<PTORED_I32, 4>(p, a, cu_count, stream);
}

int launch_ring_i32(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_ring<PTORED_I32>(p, a, cu_count, stream);
}

}  // namespace ptored
