// Many-row block scorer (prefill chunk): placeholder until the MFMA kernel lands.
#include "common.h"
#include "kernels.h"

namespace pred {

bool prefill_supported(const ScoreArgs&) { return false; }

hipError_t launch_score_prefill(const ScoreArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pred
