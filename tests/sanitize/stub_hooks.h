// Hook through which a host-only test driver can see the tile-pass
// launches that fwt_api.cpp makes (kernel_stubs.cpp calls it when set).
#pragma once
#include "../../quantum_state_encoding_amd/csrc/fwt_internal.h"

namespace qse {
typedef hipError_t (*TileLaunchHook)(const KernelKey& key, void* re, void* im, int ncomp,
                                     const TileArgs& args, unsigned block, size_t lds);
extern TileLaunchHook g_tile_launch_hook;
}  // namespace qse
