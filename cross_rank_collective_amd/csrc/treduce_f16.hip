// treduce_f16.hip -- kernel instances and launcher for f16 elements.
#include "treduce_launch.cuh"

namespace ptored {

int launch_f16(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_dtype<PTORED_F16, 2>(p, a, cu_count, stream);
}

int launch_ring_f16(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_ring<PTORED_F16, 2>(p, a, cu_count, stream);
}

}  // namespace ptored
