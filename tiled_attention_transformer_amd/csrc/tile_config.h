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

// Ragged-batch prefill on a persistent grid: each workgroup lists its items
// in LDS at start, from a cost-sorted order of every (sequence, head, query
// tile) that has rows.  Bounds of that list: sequences, query tiles of the
// longest sequence, and items per workgroup.
constexpr int kSchedSeqs = 256;
constexpr int kSchedLevels = 1024;
constexpr int kSchedItems = 1024;

// Decode: 4 waves per workgroup; one work item serves up to 32 query heads
// of one KV head.
constexpr int kDecThreads = 256;
constexpr int kDecCols = 32;

// Decode with per-sequence key counts, split by the counts themselves (the
// library's choice when the caller's workspace is large enough): the 32-key
// tiles of every (sequence, KV head, query-head block) group are laid end to
// end, and each wave of a grid of kDecListWGs four-wave workgroups takes an
// equal run of them, at least kDecListMinTiles.  Up to kDecListSeqs
// sequences.
constexpr int kDecListWGs = 256;
constexpr int kDecListMinTiles = 4;
constexpr int kDecListSeqs = 2048;

}  // namespace attn
