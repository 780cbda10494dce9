// treduce_i32.hip -- kernel instances and launcher for i32 elements.
#include "treduce_launch.cuh"

namespace ptored {

int launch_i32(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_dtype<PTORED_I32, 4>(p, a, cu_count, stream);
}

int launch_ring_i32(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_ring<PTORED_I32, 4>(p, a, cu_count, stream);
}

}  // namespace ptored
