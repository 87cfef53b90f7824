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
constexpr uint32_t kBlockVariant = 2;  // EncItem::compress of the block-hash variant; stream mode 2
constexpr uint32_t kCoded = 3;         // EncItem::compress of entropy-coded patches; stream mode 3
constexpr uint32_t kCodedInfo = 8;     // words after a coded tile's stash data: one per chunk row
// Size of the device array that ciera_encode_noalloc uses as its scratch.
constexpr uint64_t kStaticScratchBytes = (uint64_t)1 << 20;

// Element-patch and RAW shards of at most this many encode tiles are finished
// by their own tiles (split_tile_self, one launch, no stash); larger ones, the
// block-hash variant and coded patches by a finishing kernel.
constexpr uint32_t kSelfTiles = 256;

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
  const uint8_t* cache;  // cache_full + offset of the shard (element variant)
  uint8_t* hashes;       // the shard's hash cache, 16 bytes per block (block-hash variant)
  uint8_t* stream;
  uint64_t n;
  uint64_t off;
  uint64_t capacity;
  uint64_t tile0;          // the item's first tile in the batch's per-tile count array
  uint64_t stash;          // word offset of the item's first tile stash in the batch's stash array
  uint32_t tpi;            // tiles of the item
  uint32_t tvals;          // values per tile (a multiple of 4096)
  uint32_t cap;            // records a tile stash holds
  uint32_t rank, world;
  uint32_t block_size;
  uint32_t compress;       // 0 RAW, 1 element patches, kBlockVariant the block-hash variant, kCoded coded patches
  uint32_t cache_aligned;  // (cache_full + off) is 16-byte aligned
  uint32_t elem_bytes;     // 2 (bf16, fp16) or 4 (fp32)
  uint32_t batch_id;       // the batch that wrote this descriptor
};

// One decode item: a tensor and its W receive slots.
struct DecItem {
  const uint8_t* streams;          // rank r's stream at streams + r * slot, when ranks is null
  const uint8_t* const* ranks;     // else at ranks[r] (world pointers in the batch's scratch)
  uint64_t slot;                   // bytes readable at every rank's stream
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
//   head   : u32 batch id (+ padding to 256 B)
//   items  : EncItem per item, ordered by group
//   counts : u32 per tile -- changed values of the tile, written by the split kernel
//   stash  : u32 x cap per tile -- the tile's first cap changes in ascending order,
//            (value index in the tile) | exponent << 16; the finishing kernel moves
//            them to their places in the stream.  Coded items: per chunk row of
//            the tile a 4096-byte region (its coded or dense data), then
//            kCodedInfo words, one per row: changes | words << 13 | dense << 26;
//            the tile's count is then data bytes | changes << 16
//   sync   : u64 per tile of the groups whose tiles finish their items
//            themselves: epoch << 32 | changes of the tile (zeroed by prepare)
struct EncArgs {
  const EncItem* items;
  uint32_t item0;      // first item of the group
  uint32_t tpi;        // tiles per item in the group
  uint32_t* counts;    // the batch's per-tile counts
  uint32_t* stash;     // the batch's stash words
  uint64_t* sync;      // the batch's sync words (EncItem::tile0 indexes them too)
  uint32_t self;       // the group's tiles finish their items (compress 0/1, tpi <= kSelfTiles)
  uint32_t polls;      // self: polls of a sibling's slot before counting its changes (0: default)
};

// The per-tile finishing kernel of one group (at most kThreads tiles per
// item); the group's counts and stashes are contiguous, item by item.
struct FinArgs {
  const EncItem* items;
  const uint32_t* counts;
  const uint32_t* stash;
  const uint64_t* prefix;  // coded items of more than kThreads tiles: the scan kernel's per-tile
                           // prefixes (indexed like counts); else null
  uint64_t tile0;   // the group's first tile (index into counts)
  uint64_t stash0;  // word offset of the group's first tile stash
  uint32_t item0, tpi, cap, pad;
};

// The first 256 bytes of a batch's scratch hold its batch id.  Every descriptor
// carries the id of the batch that wrote it, and every kernel takes its batch's
// id as an argument: a descriptor of another batch (the scratch was prepared
// anew for another batch) is skipped.
hipError_t launch_encode(int dtype, int sub, uint32_t nitems, const EncArgs& a, uint32_t batch_id, hipStream_t s);
hipError_t launch_encode_finish(int dtype, const EncItem* items, uint32_t item0, uint32_t nitems, uint32_t wg_per_item,
                                const uint32_t* counts, const uint32_t* stash, uint32_t batch_id, hipStream_t s);
hipError_t launch_encode_finish_tiles(int dtype, bool coded, uint32_t nitems, const FinArgs& f, uint32_t batch_id,
                                      hipStream_t s);
hipError_t launch_coded_scan(int dtype, uint32_t nitems, const FinArgs& f, uint64_t* prefix, uint32_t batch_id,
                             hipStream_t s);
// max_wg: 0, or a bound on the workgroups of each launch (each then decodes
// tiles in turn; groups of tensors flagged coded ignore it)
hipError_t launch_decode(int dtype, int u, bool coded, const DecItem* items, uint32_t item0, uint32_t nitems,
                         uint32_t tpr, uint32_t world, uint32_t* status, uint32_t batch_id, uint32_t max_wg,
                         hipStream_t s);
// The calling thread's current device's copy of the library's static scratch
// array (kStaticScratchBytes, 256-byte aligned): its device address, looked up
// once per device.
hipError_t static_scratch(void** ptr);
// Writes n encode descriptors (host array) to dst on the device by kernel
// arguments -- no host staging buffer, no copy -- zeroes nzero 64-bit words
// at zero and stores batch_id at head.
hipError_t launch_enc_desc(const EncItem* host_items, uint32_t n, EncItem* dst, uint64_t* zero, uint64_t nzero,
                           uint32_t* head, uint32_t batch_id, hipStream_t s);
hipError_t launch_cache_update(int dtype, const uint8_t* w, uint8_t* cache, uint64_t n, hipStream_t s);
hipError_t launch_hash_seed(int dtype, const uint8_t* x, uint8_t* hashes, uint64_t n, uint32_t block_size, hipStream_t s);

}  // namespace ciera
