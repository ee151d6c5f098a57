// launch_stubs.cpp -- host-only stand-ins for the device launchers of
// libsage, so that the host side of the C ABI (sage_api.cpp: argument checks,
// workspace plan, sequence tables) can be built with the host sanitizers and
// driven on a machine without a GPU.  Test infrastructure: built by
// tests/test_sanitizers.py.  Every stand-in that would launch work reports an
// error (the driver never gets that far: its calls fail their checks, or the
// device check, first); the planning queries return fixed plausible values.
#include "sage_internal.h"

namespace sage {
int stat_chunks_per_wg(int d) { return 64 / (d / 8); }   // one-wave statistics workgroups
hipError_t launch_stats(const KParams&, int, const StatJobs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_finalize(const KParams&, const FinJobs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quant(const KParams&, int, const QuantArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn(const KParams&, int, const int8_t*, const float*, const int8_t*,
                       const float*, const uint8_t*, const float*, const float*, const float*,
                       void*, float*, const int8_t*, const float*, hipStream_t) {
    return hipErrorNoDevice;
}
int attn_base_wgs(const KParams& P) { return P.hkv * (P.tab.uniform ? P.tab.n : 1); }
bool use_decode_kernel(const KParams& P) { return P.kv_tiles > 0 && !P.bqs; }
int decode_waves_per_cu(int, bool, bool, int) { return 4; }
hipError_t launch_merge(const MergeArgs&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_qk_dump(const KParams&, const int8_t*, const int8_t*, int32_t*, hipStream_t) {
    return hipErrorNoDevice;
}
hipError_t noalloc_workspace(void**) { return hipErrorNoDevice; }
hipError_t launch_e4m3_dump(uint32_t, uint32_t, uint8_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t micro_rate(int, int, double*, hipStream_t) { return hipErrorNoDevice; }
}  // namespace sage
