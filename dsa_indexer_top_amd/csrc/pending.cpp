// Entry points whose kernels are not written yet: they reject every call.
#include "common.hpp"
using namespace echo;
extern "C" {
int echo_index_scores_prefill(const uint8_t *, const float *, const uint8_t *, int32_t, int32_t, int32_t, float *, int64_t, void *) { return fail(ECHO_EUNSUPPORTED, "not built yet"); }
}
