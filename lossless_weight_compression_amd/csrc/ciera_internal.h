// Internal descriptors shared by the host API (ciera_api.cpp) and the gfx950
// kernels (ciera_kernels.hip).  Not part of the public ABI.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace ciera {

constexpr int kThreads = 256;               // one workgroup = 4 wave64
constexpr int kEPT = 16;                    // values per thread per sub-tile
constexpr int kSub = kThreads * kEPT;       // 4096 values per sub-tile
constexpr int kDecTile = kSub;              // decode tile
constexpr uint64_t kHeader = 64;

// One encode item as the kernels see it (built on the host, uploaded per call).
struct EncItem {
  const uint8_t* x;      // shard values
  const uint8_t* cache;  // cache_full + offset of the shard
  uint8_t* stream;
  uint64_t n;
  uint64_t off;
  uint64_t capacity;
  uint32_t tile_begin;   // first tile of this item in the group's tile space
  uint32_t ntiles;       // >= 1
  uint32_t rank, world;
  uint32_t block_size;
  uint32_t compress;
  uint32_t cache_aligned;  // (cache_full + off) is 16-byte aligned
  uint32_t pad;
};

// Control block at the start of an encode group's scratch; zeroed by the
// per-call descriptor upload.  raw_list[] follows it.
struct EncCtl {
  uint32_t tile_counter;  // dynamic tile ids
  uint32_t raw_count;     // items whose COMPRESSED stream was not shorter
  uint32_t pad[62];
};

struct DecItem {
  const uint8_t* streams;
  uint64_t slot;
  uint8_t* out;
  uint8_t* cache;
  uint64_t rows, cols;
  uint32_t tile_begin;
  uint32_t tiles_per_rank;   // ceil(n0 / kDecTile), >= 1
  uint32_t world;
  uint32_t block_size;
};

hipError_t launch_encode(int dtype, int sub, const EncItem* items, const uint32_t* tile_begin,
                         uint32_t count, uint32_t total_tiles, EncCtl* ctl, uint32_t* raw_list,
                         uint64_t* status, uint32_t epoch, hipStream_t s);
hipError_t launch_encode_fixup(int dtype, const EncItem* items, const EncCtl* ctl,
                               const uint32_t* raw_list, hipStream_t s);
hipError_t launch_decode(int dtype, const DecItem* items, const uint32_t* tile_begin,
                         uint32_t count, uint32_t total_tiles, uint32_t* status, hipStream_t s);
hipError_t launch_cache_update(int dtype, const uint8_t* w, uint8_t* cache, uint64_t n,
                               hipStream_t s);

}  // namespace ciera
