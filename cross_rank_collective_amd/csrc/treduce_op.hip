// treduce_op.hip -- reduction and ring kernel instances of one (element type,
// operator) pair.  The build compiles this file once per pair, with
// -DPTORED_INST_DT=<a ptored_dtype name> -DPTORED_INST_OP=<a ptored_op name>.
#include "treduce_launch.hpp"

#if !defined(PTORED_INST_DT) || !defined(PTORED_INST_OP)
#error "treduce_op.hip needs -DPTORED_INST_DT=<ptored_dtype> -DPTORED_INST_OP=<ptored_op>"
#endif

namespace ptored {

constexpr int kInstEs = (PTORED_INST_DT == PTORED_BF16 || PTORED_INST_DT == PTORED_F16) ? 2 : 4;

template <int DT, int OP>
int launch_op(const Plan& p, const KArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_op<DT, OP, kInstEs>(p, a, cu_count, stream);
}

template <int DT, int OP>
int launch_ring_op(const Plan& p, const RingArgs& a, int cu_count, hipStream_t stream) {
    return dispatch_ring_n<DT, OP, kInstEs>(p, a, cu_count, stream);
}

template int launch_op<PTORED_INST_DT, PTORED_INST_OP>(const Plan&, const KArgs&, int,
                                                       hipStream_t);
template int launch_ring_op<PTORED_INST_DT, PTORED_INST_OP>(const Plan&, const RingArgs&, int,
                                                            hipStream_t);

}  // namespace ptored
