// treduce_bf16.hip -- kernel instances and launcher for bf16 elements.
#include "treduce_launch.cuh"

namespace ptored {

int launch_bf16(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_dtype<PTORED_BF16, 2>(p, a, cu_count, stream);
}

int launch_ring_bf16(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_ring<PTORED_BF16, 2>(p, a, cu_count, stream);
}

}  // namespace ptored
