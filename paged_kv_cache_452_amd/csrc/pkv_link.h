// Internal declarations for block copies over the host link (not part of the ABI).
#pragma once

#include "pkv_internal.h"

namespace pkv {

constexpr int kLinkWorkgroups = 64;  // workgroups of a host-link copy launch
constexpr int kLinkUnroll = 4;       // 16-byte loads in flight per thread

// The copies of launch_block_copy (same BlockCopy meaning), from a grid of at most
// kLinkWorkgroups workgroups: for swapping between the device pool and a pinned host pool, where
// the link, not the GPU, sets the rate.
hipError_t launch_block_copy_link(const BlockCopy& c, int num_layers, int num_pairs,
                                  hipStream_t stream);

}  // namespace pkv
