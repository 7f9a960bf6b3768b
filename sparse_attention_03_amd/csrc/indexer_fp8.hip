// Lightning indexer on FP8 MFMA (FP8 queries x FP8 keys): the compute-bound
// prefill shape.  Not built yet: the entry point reports DSA_ERR_UNSUPPORTED.
#include "common.h"
#include "kernels.h"

namespace dsa {

dsa_status launch_indexer_fp8(const IndexerParams&, hipStream_t) { return DSA_ERR_UNSUPPORTED; }

}  // namespace dsa
