// Internal descriptors shared by the host API (ciera_api.cpp) and the gfx950
// kernels (ciera_kernels.hip).  Not part of the public ABI.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace ciera {

constexpr int kThreads = 256;          // one workgroup = 4 wave64
constexpr int kEPT = 16;               // values per thread per chunk
constexpr int kSub = kThreads * kEPT;  // 4096 values per chunk row of a tile
constexpr uint64_t kHeader = 64;

// Decode workgroups: kDecThreads threads, 16 values each per chunk row; a tile
// is U chunk rows.  (512- and 1024-thread groups, which put more data behind
// each tile's chain of dependent reads, measured no faster on gfx950.)
constexpr int kDecThreads = 256;
constexpr int kDecRow = kDecThreads * kEPT;
constexpr int kRecBatch = 4;  // consecutive patch records per decode thread per round
constexpr int kRecWords = (3 + 5 * kRecBatch + 3) / 4;  // aligned words that cover them

// One encode item as the kernels see it.
struct EncItem {
  const uint8_t* x;      // shard values
  const uint8_t* cache;  // cache_full + offset of the shard
  uint8_t* stream;
  uint64_t n;
  uint64_t off;
  uint64_t capacity;
  uint32_t rank, world;
  uint32_t block_size;
  uint32_t compress;
  uint32_t cache_aligned;  // (cache_full + off) is 16-byte aligned
  uint32_t elem_bytes;     // 2 (bf16) or 4 (fp32)
  uint32_t batch_id;       // the batch that wrote this descriptor
  uint32_t pad;
};

// One decode item: a tensor and its W receive slots.
struct DecItem {
  const uint8_t* streams;
  uint64_t slot;
  uint8_t* out;
  uint8_t* cache;
  uint64_t q;              // rows / world: rows of every rank ...
  uint64_t cols;
  uint32_t world;
  uint32_t block_size;
  uint32_t batch_id;       // the batch that wrote this descriptor
  uint32_t rem;            // ... plus one for ranks below rows % world
};

// Encode scratch layout (offsets in bytes from the scratch base):
//   ctl      : u32 [batch id, any_raw, error, epoch, tag] (+ padding to 256 B);
//              epoch is the tag of the next launch and lives on the device (the
//              fallback kernel advances it), tag is the running launch's, so a
//              launch's kernel arguments never change and it can be replayed
//              from a captured graph
//   raw_flag : u32 per item -- equals the launch tag if the item must be rewritten RAW
//   ctr      : u32 per item -- dynamic tile counter, back at 0 after every launch
//   items    : EncItem per item, ordered by group
//   status   : u64 per tile, look-back words tagged with the launch tag
constexpr int kCtlAnyRaw = 1, kCtlError = 2, kCtlEpoch = 3, kCtlTag = 4;
struct EncArgs {
  const EncItem* items;
  uint32_t item0;      // first item of the group
  uint32_t tpi;        // tiles per item in the group
  uint32_t* ctr;       // per-item counters (indexed by absolute item)
  uint64_t* status;    // group's status words, (item - item0) * tpi + tile
  uint32_t* raw_flag;  // per absolute item
  uint32_t* any_raw;
};

// ctl: the control words at the start of a batch's scratch.  Every descriptor
// carries the id of the batch that wrote it; kernels exit at once when the
// descriptor they read belongs to another batch (the scratch was taken over).
hipError_t launch_encode(int dtype, int sub, uint32_t nitems, const EncArgs& a, uint32_t* ctl,
                         uint32_t batch_id, hipStream_t s);
hipError_t launch_encode_fixup(const EncItem* items, uint32_t count, uint32_t wg_per_item, const uint32_t* raw_flag,
                               uint32_t* ctl, uint32_t batch_id, hipStream_t s);
hipError_t launch_decode(int dtype, int u, const DecItem* items, uint32_t item0, uint32_t nitems,
                         uint32_t tpr, uint32_t world, uint32_t* status, const uint32_t* ctl,
                         uint32_t batch_id, hipStream_t s);
hipError_t launch_cache_update(int dtype, const uint8_t* w, uint8_t* cache, uint64_t n, hipStream_t s);

}  // namespace ciera
