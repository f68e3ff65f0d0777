// Tile shapes of the gfx950 attention kernels that the host-side sizing
// logic also needs.  Plain C++ (no HIP), shared by the kernels and by
// host_checks.cpp.
#pragma once

namespace attn {

// Prefill: 8 waves x 32 query rows per work item, 64 keys per K/V tile (the
// host counts query tiles of kFwdBr rows; the launcher halves the tile, on
// 4-wave workgroups, for fixed batches with fewer tiles than CUs).
constexpr int kFwdWaves = 8;
constexpr int kFwdBr = 32 * kFwdWaves;
constexpr int kFwdBc = 64;

// Decode: 4 waves per workgroup; one work item serves up to 32 query heads
// of one KV head.
constexpr int kDecThreads = 256;
constexpr int kDecCols = 32;

}  // namespace attn
