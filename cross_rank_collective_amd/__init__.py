"""MI355X-native N-way cross-rank reduction (TREDUCE) on one GPU.

``libptored.so`` (HIP, gfx950) computes dst = src_0 (+) ... (+) src_{N-1}
over a valid rectangle of N equally shaped buffers; ``binding`` exposes its
C ABI to Python and ``workloads`` draws seeded synthetic inputs.
"""

from .binding import (  # noqa: F401
    DTYPES,
    OPS,
    PtoredError,
    accumulate_add,
    allreduce,
    load,
    ptored_abi_version,
    ptored_accumulate_add,
    ptored_allreduce,
    ptored_max_ranks,
    ptored_reduce_scatter_ring,
    ptored_ring_bounds,
    ptored_status_string,
    ptored_treduce,
    ptored_treduce_ex,
    ptored_treduce_plan,
    reduce_scatter_ring,
    ring_bounds,
    treduce,
    tuning,
)
