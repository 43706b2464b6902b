#include "fa_internal.h"
namespace fa {
hipError_t launch_bwd_pre(const Problem&, const BwdPtrs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_main(const Problem&, const BwdPtrs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_dq(const Problem&, const BwdPtrs&, hipStream_t) { return hipErrorNotSupported; }
}
