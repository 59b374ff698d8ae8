// Host-side launchers, one per kernel family.  Each enqueues on `stream`
// and returns the hipError_t of the launch.  Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace gdn {

hipError_t launch_verify(const Args &a, hipStream_t stream);
hipError_t launch_commit_verify(const Args &a, hipStream_t stream);
hipError_t launch_accept_commit_verify(const Args &a, hipStream_t stream);
hipError_t launch_commit(const Args &a, hipStream_t stream);
hipError_t launch_accepted_path(const Args &a, hipStream_t stream);
hipError_t launch_accept_greedy(const Args &a, hipStream_t stream);
hipError_t launch_accept_commit(const Args &a, hipStream_t stream);
hipError_t launch_commit_node(const Args &a, hipStream_t stream);
hipError_t launch_commit_replay(const Args &a, hipStream_t stream);
hipError_t launch_budget_select(const Args &a, int budget, float threshold, hipStream_t stream);
hipError_t launch_ancestry(const Args &a, hipStream_t stream);
hipError_t launch_attention(const AttnArgs &a, hipStream_t stream);
// Device address of the calling device's copy of the static attention scratch
// (GDN_TREE_STATIC_SCRATCH_BYTES), looked up once per device.
hipError_t static_scratch(void **ptr);
hipError_t launch_verify_storeall(const Args &a, hipStream_t stream);
hipError_t launch_commit_storeall(const Args &a, hipStream_t stream);

}  // namespace gdn
