// Entry points whose kernels are not written yet: they reject every call.
#include "common.hpp"
using namespace echo;
extern "C" {
int echo_prefetch_threshold(const uint8_t *, const float *, const uint8_t *, const float *, const int64_t *, const int32_t *, int32_t, int32_t, float, float *, void *) { return fail(ECHO_EUNSUPPORTED, "not built yet"); }
int echo_index_scores_prefill(const uint8_t *, const float *, const uint8_t *, int32_t, int32_t, int32_t, float *, int64_t, void *) { return fail(ECHO_EUNSUPPORTED, "not built yet"); }
int echo_prefetch_begin(const echo_pool *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t, void *, size_t, void *) { return fail(ECHO_EUNSUPPORTED, "not built yet"); }
int echo_prefetch_gather(const echo_pool *, const int64_t *, const int32_t *, const int32_t *, const int32_t *, int32_t *, int32_t, int32_t, const int32_t *, int32_t, const int32_t *, const int32_t *, int32_t *, int32_t *, void *) { return fail(ECHO_EUNSUPPORTED, "not built yet"); }
size_t echo_decode_workspace_bytes(const echo_decode_args *, int32_t) { return 0; }
int echo_decode_select(const echo_decode_args *, const echo_pool *, const echo_decode_out *, void *, size_t, void *, void *) { return fail(ECHO_EUNSUPPORTED, "not built yet"); }
int echo_graph_capture_decode(const echo_decode_args *, const echo_pool *, const echo_decode_out *, void *, size_t, void *, void *, echo_graph *) { return fail(ECHO_EUNSUPPORTED, "not built yet"); }
int echo_graph_launch(echo_graph, void *) { return fail(ECHO_EUNSUPPORTED, "not built yet"); }
int echo_graph_destroy(echo_graph) { return ECHO_OK; }
}
