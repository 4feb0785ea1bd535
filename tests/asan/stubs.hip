// Host-only stand-ins for the HIP runtime queries and the kernel launchers
// that api.hip calls, so that the library's argument validation can be built
// for the CPU with AddressSanitizer and driven without a GPU.  Every pointer is
// reported as device memory of device 0; no pointer is ever dereferenced.  Each
// launcher only counts its call.  Test infrastructure: never linked into the
// library.
#include "common.h"

extern "C" {
int g_launches = 0;   // calls that reached a launcher (validation passed)

hipError_t hipGetDevice(int *d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipPointerGetAttributes(hipPointerAttribute_t *a, const void *) {
    a->type = hipMemoryTypeDevice;
    a->device = 0;
    return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char *hipGetErrorName(hipError_t) { return "stub"; }
const char *hipGetErrorString(hipError_t) { return "stub"; }
}

namespace mp {
LowerLayout lower_layout(int64_t, int64_t e, bool split_dirs) {
    LowerLayout L = {};
    L.total = 4096 + (size_t)(e > 0 ? e : 1) * (split_dirs ? 96 : 64);
    return L;
}
mp_status lower_run(const void *, const void *, mp_dtype, int64_t, int64_t, mp_graph *, void *,
                    hipStream_t, bool, int *bad, hipStream_t, hipEvent_t) {
    ++g_launches;
    *bad = 0;
    return MP_OK;
}
mp_status static_workspace(void **ptr, size_t *bytes) {
    *ptr = reinterpret_cast<void *>((uintptr_t)1 << 46);   // a fake device address
    *bytes = MP_STATIC_WORKSPACE_BYTES;
    return MP_OK;
}
mp_status lower_read_info(mp_graph *, hipStream_t, int *bad) {
    *bad = 0;
    return MP_OK;
}
mp_status spmm_run(const CsrView &, const float *, int64_t, const void *, mp_dtype, int64_t,
                   float *, hipStream_t, const NormSpec *, bool, float *) {
    ++g_launches;
    return MP_OK;
}
bool spmm_fused_supported(mp_dtype, int64_t h, int64_t, const void *, const void *,
                          const void *) {
    return h <= 256;
}
mp_status spmm_fused_run(const CsrView &, const float *, int64_t, const void *, mp_dtype, int64_t,
                         float *, const void *, float *, const float *, hipStream_t,
                         const NormSpec *, bool, float *) {
    ++g_launches;
    return MP_OK;
}
mp_status set_owner_overrides(int32_t, int32_t, int32_t) { return MP_OK; }
size_t split_workspace_bytes(const int64_t *, int64_t, int64_t h) { return 4096 * (size_t)h; }
mp_status sddmm_run(const int32_t *, const int32_t *, int64_t, const void *, const void *,
                    mp_dtype, int64_t, int64_t, float *, hipStream_t) {
    ++g_launches;
    return MP_OK;
}
mp_status edge_softmax_run(const mp_graph *, const float *, int64_t, float *, float *,
                           hipStream_t) {
    ++g_launches;
    return MP_OK;
}
mp_status edge_softmax_stats_run(const mp_graph *, const float *, float *, hipStream_t) {
    ++g_launches;
    return MP_OK;
}
mp_status edge_softmax_backward_run(const mp_graph *, const float *, const float *, int64_t,
                                    float *, float *, hipStream_t) {
    ++g_launches;
    return MP_OK;
}
mp_status attention_row_dot_run(const float *, const void *, mp_dtype, int64_t, int64_t, int64_t,
                                float *, hipStream_t) {
    ++g_launches;
    return MP_OK;
}
mp_status score_grad_apply_run(const int32_t *, const float *, const float *, int64_t, int64_t,
                               float *, hipStream_t) {
    ++g_launches;
    return MP_OK;
}
mp_status edge_normalize_run(const mp_graph *, int, const float *, float *, hipStream_t) {
    ++g_launches;
    return MP_OK;
}
}  // namespace mp
