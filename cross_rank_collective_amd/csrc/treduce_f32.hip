// treduce_f32.hip -- kernel instances and launcher for f32 elements.
#include "treduce_launch.cuh"

namespace ptored {

int launch_f32(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_dtype<PTORED_F32, 4>(p, a, cu_count, stream);
}

int launch_ring_f32(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_ring<PTORED_F32, 4>(p, a, cu_count, stream);
}

}  // namespace ptored
