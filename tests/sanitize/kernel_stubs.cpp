// Host-only stand-ins for the device-side entry points of the library
// (fwt_kernels.hip, fwt_ablation.hip, fwt_ozaki.hip), so that the planner
// and validation code in fwt_api.cpp can be built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every kernel variant is
// reported as compiled, which makes the planner take every branch; nothing
// here launches anything.  A driver may set g_tile_launch_hook to see the
// tile-pass launches instead.
#include "stub_hooks.h"

namespace qse {

TileLaunchHook g_tile_launch_hook = nullptr;

bool kernel_available(const KernelKey&) { return true; }
hipError_t kernels_init_device() { return hipSuccess; }
hipError_t launch_tile_pass(const KernelKey& key, void* re, void* im, int ncomp,
                            const TileArgs& args, unsigned block, size_t lds, hipStream_t,
                            hipEvent_t, hipEvent_t)
{
    return g_tile_launch_hook ? g_tile_launch_hook(key, re, im, ncomp, args, block, lds)
                              : hipErrorNotSupported;
}
hipError_t launch_pair_f32(float*, float*, int64_t, int, float, hipStream_t, hipEvent_t, hipEvent_t)
{
    return hipErrorNotSupported;
}
hipError_t launch_stream_copy(void*, const void*, int64_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t ablation_stagewise(int, void*, void*, int64_t, int, int, double, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t ablation_popc_gemm(int, void*, void*, void*, void*, int64_t, int, int, double, hipStream_t)
{
    return hipErrorNotSupported;
}
int oz_num_moduli(int n) { return n < 5 ? 0 : 10; }
void oz_pass_plan(int n, OzPass* passes, int* npasses)
{
    passes[0] = OzPass{1, 0, n < 10 ? n : 10, 0};
    *npasses = 1;
}
size_t oz_workspace_layout(int64_t batch, int n, int comps, size_t* off_partial, size_t* off_exps)
{
    const size_t words = (size_t)batch * ((size_t)1 << n) * (size_t)comps * 3;
    *off_partial = words * 4;
    *off_exps = *off_partial + 4096;
    return *off_exps + 4096;
}
hipError_t ablation_ozaki(double*, double*, int64_t, int, double, void*, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t ablation_mfma_transpose(int, void*, void*, void*, void*, int64_t, int, int, double,
                                   hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t ablation_mfma_row(int, void*, void*, int64_t, int, int, int, double, hipStream_t)
{
    return hipErrorNotSupported;
}
hipError_t onepass_occupancy(int* blocks_per_cu)
{
    *blocks_per_cu = 2;
    return hipSuccess;
}
hipError_t launch_onepass(float*, float*, int, void*, float, hipStream_t, hipEvent_t, hipEvent_t)
{
    return hipErrorNotSupported;
}

}  // namespace qse
