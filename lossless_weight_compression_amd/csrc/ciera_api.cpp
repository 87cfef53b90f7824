// Host side of the CIERA codec library: argument validation, the per-tensor
// selector, prepared batches (descriptor tables resident in the caller's
// scratch) and kernel launches.  See include/ciera.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <atomic>
#include <chrono>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "ciera.h"
#include "ciera_internal.h"

using namespace ciera;

namespace {

typedef unsigned __int128 u128;

constexpr uint64_t kMaxElems = (uint64_t)1 << 48;
constexpr uint64_t kEncMagic = 0x434945524145454eull;  // batch kinds
constexpr uint64_t kDecMagic = 0x4349455241444543ull;
constexpr int kMaxGroups = 64;

uint32_t elem_bytes(uint32_t dt) { return dt == CIERA_FP32 ? 4u : 2u; }
// Sign|mantissa bits per value: bf16 8, fp32 24, fp16 11 (an LSB-first bit
// stream); the section of n values takes ceil(n * bits / 8) bytes.
uint32_t sm_bits(uint32_t dt) { return dt == CIERA_BF16 ? 8u : dt == CIERA_FP32 ? 24u : 11u; }
bool pow2(uint32_t x) { return x && !(x & (x - 1)); }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Whether the byte ranges [a, a + alen) and [b, b + blen) share a byte.
bool overlap(const void* a, uint64_t alen, const void* b, uint64_t blen) {
  if (alen == 0 || blen == 0) return false;
  const unsigned __int128 a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + blen && b0 < a0 + alen;
}
uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
uint64_t bitmap_bytes(uint64_t n, uint32_t B) { return ((n + B - 1) / B + 7) / 8; }

// The HIP error behind the calling thread's last CIERA_ERR_DEVICE.
thread_local char g_last_error[256] = "no error";

ciera_status_t device_error(const char* what, hipError_t e) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return CIERA_ERR_DEVICE;
}

ciera_status_t check_tensor(const ciera_tensor_t* t) {
  if (!t) return CIERA_ERR_INVALID_ARG;
  if (t->dtype != CIERA_BF16 && t->dtype != CIERA_FP32 && t->dtype != CIERA_FP16) return CIERA_ERR_INVALID_ARG;
  if (!pow2(t->block_size) || t->block_size < 64 || t->block_size > 4096) return CIERA_ERR_INVALID_ARG;
  if (t->world == 0) return CIERA_ERR_INVALID_ARG;
  if (t->flags & ~CIERA_TENSOR_CODED) return CIERA_ERR_INVALID_ARG;
  if (t->rows >= kMaxElems || t->cols >= kMaxElems) return CIERA_ERR_UNSUPPORTED;
  if ((u128)t->rows * t->cols >= kMaxElems) return CIERA_ERR_UNSUPPORTED;
  // patch records carry u32 shard-local indices: the largest shard (rank 0's)
  // must hold fewer than 2^32 values
  const uint64_t rows0 = t->rows / t->world + (t->rows % t->world ? 1 : 0);
  if ((u128)rows0 * t->cols >= ((u128)1 << 32)) return CIERA_ERR_UNSUPPORTED;
  return CIERA_OK;
}

// ZeRO-style even row partition: rank r holds floor(R/W) + [r < R%W] rows.
void shard_of(const ciera_tensor_t* t, uint32_t r, uint64_t* off, uint64_t* n) {
  const uint64_t q = t->rows / t->world, rem = t->rows % t->world;
  const uint64_t rows_before = (uint64_t)r * q + std::min<uint64_t>(r, rem);
  *off = rows_before * t->cols;
  *n = (q + (r < rem ? 1 : 0)) * t->cols;
}

// ---------------------------------------------------------------- staging
// Descriptor tables travel host -> device through a small ring of pinned
// buffers per device; a slot is reused only after its previous copy completed.
constexpr int kSlots = 8;
struct Slot {
  void* buf = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};
struct Staging {
  std::mutex mu;
  Slot slot[kSlots];
  unsigned next = 0;
};
std::mutex g_staging_mu;
std::unordered_map<int, Staging*> g_staging;

Staging* staging_for(int dev) {
  std::lock_guard<std::mutex> lk(g_staging_mu);
  auto it = g_staging.find(dev);
  if (it != g_staging.end()) return it->second;
  Staging* s = new Staging();
  g_staging[dev] = s;
  return s;
}

hipError_t upload(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  Staging* st = staging_for(dev);
  std::lock_guard<std::mutex> lk(st->mu);
  Slot& sl = st->slot[st->next++ % kSlots];
  if (sl.pending) {
    if ((e = hipEventSynchronize(sl.ev)) != hipSuccess) return e;
    sl.pending = false;
  }
  if (sl.cap < bytes) {
    if (sl.buf && (e = hipHostFree(sl.buf)) != hipSuccess) return e;
    sl.buf = nullptr;
    sl.cap = 0;
    const size_t cap = std::max<size_t>(align_up(bytes, 1 << 16), 1 << 16);
    if ((e = hipHostMalloc(&sl.buf, cap, hipHostMallocDefault)) != hipSuccess) return e;
    sl.cap = cap;
  }
  if (!sl.ev && (e = hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming)) != hipSuccess) return e;
  std::memcpy(sl.buf, src, bytes);
  if ((e = hipMemcpyAsync(dst, sl.buf, bytes, hipMemcpyHostToDevice, stream)) != hipSuccess) return e;
  if ((e = hipEventRecord(sl.ev, stream)) != hipSuccess) return e;
  sl.pending = true;
  return hipSuccess;
}

// Polls of a sibling tile's count before an encode tile counts its changes
// itself (0: the kernel's default).
std::atomic<uint32_t> g_sync_polls{0};

// Batch ids: distinct per prepare, never 0.
std::atomic<uint32_t> g_ids{(uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761u};
uint32_t next_id() {
  uint32_t v;
  do v = g_ids.fetch_add(0x9E3779B9u) ^ 0x5bd1e995u; while (v == 0);
  return v;
}

// ------------------------------------------------------------------ batches
struct Group {
  uint32_t dtype, unit;  // unit: encode sub-tiles S, decode chunk rows U
  uint32_t item0, nitems;
  uint32_t tpi;          // encode: tiles per item
  uint32_t tpr, world;   // decode: tiles per rank, world
  uint32_t coded;        // items with coded patches (encode) / tensors flagged coded (decode)
  uint32_t self;         // encode: tiles that finish their items themselves (split_tile_self)
  uint64_t tile0;        // encode: the group's first tile in the batch's count array
  uint64_t stash0;       // encode: word offset of the group's first tile stash
};
struct BatchImpl {
  uint64_t magic;
  uint8_t* scratch;
  uint64_t scratch_bytes;
  uint32_t* status_dev;
  uint32_t count, ngroups;
  uint32_t batch_id, reserved0;
  uint32_t launches, any_compress;
  uint32_t fin_wg, reserved1;  // encode finishing kernel: workgroups per item
  uint64_t off_counts, off_stash, off_items, off_sync;
  Group g[kMaxGroups];
};
static_assert(sizeof(BatchImpl) <= sizeof(ciera_batch_t), "batch handle too small");

BatchImpl* impl(ciera_batch_t* b) { return reinterpret_cast<BatchImpl*>(b); }

// Encode tile: S rows of 4096 values, at least 8*B values so every tile owns
// whole bitmap bytes; two rows once the shard exceeds one row.
uint32_t enc_sub(uint32_t B, uint64_t n) {
  uint32_t s = std::max<uint32_t>(1u, B / 512u);
  if (n > (uint64_t)kSub && s < 2) s = 2;
  return s;
}
uint32_t dec_unit(uint64_t n0) { return n0 > (uint64_t)kDecRow ? 2u : 1u; }

// A tile's stash holds up to T/4 changes (25% of its values); a tile with
// more has them derived again by the finishing kernel.
constexpr uint32_t kStashDiv = 4;

// Stash words per tile: T/4; for coded patches T bytes of chunk data (a
// 4096-byte region per row) and kCodedInfo info words.
uint32_t stash_cap(uint32_t S, bool coded) {
  return (uint32_t)kSub * S / kStashDiv + (coded ? kCodedInfo : 0u);
}

struct EncPlan {
  std::vector<uint32_t> order;  // items in group order
  std::vector<Group> groups;
  std::vector<uint64_t> tile0, stash;  // per item in group order
  uint64_t off_items = 0, off_sync = 0, off_counts = 0, off_stash = 0, upload = 0, total = 0;
};

// Whether an item's own tiles finish it (element patches and RAW of at most
// kSelfTiles tiles) rather than a finishing kernel (larger items, the
// block-hash variant and coded patches).
bool self_finished(uint32_t compress, uint64_t tpi) { return compress <= 1 && tpi <= kSelfTiles; }

// An encode item's launch group: (dtype, S, tiles per item, coded, self),
// after the checks of its tensor, rank and size.
using EncKey = std::tuple<uint32_t, uint32_t, uint32_t, uint32_t, uint32_t>;
ciera_status_t enc_item_key(const ciera_encode_item_t& it, EncKey* key) {
  ciera_status_t s = check_tensor(&it.t);
  if (s) return s;
  if (it.rank >= it.t.world) return CIERA_ERR_INVALID_ARG;
  uint64_t off, n;
  shard_of(&it.t, it.rank, &off, &n);
  if (n >= ((uint64_t)1 << 32)) return CIERA_ERR_UNSUPPORTED;
  const uint32_t S = enc_sub(it.t.block_size, n);
  const uint64_t T = (uint64_t)kSub * S;
  const uint64_t tpi = std::max<uint64_t>(1, (n + T - 1) / T);
  const uint32_t coded = it.compress == kCoded ? 1u : 0u;
  // coded: the chunk table's u32 running byte counts hold the data of every
  // chunk of the shard, 4096 bytes each at most
  if (coded && n >= ((uint64_t)1 << 31)) return CIERA_ERR_UNSUPPORTED;
  *key = std::make_tuple(it.t.dtype, S, (uint32_t)tpi, coded, self_finished(it.compress, tpi) ? 1u : 0u);
  return CIERA_OK;
}

// Scratch offsets of an encode batch of `count` items, `tiles` tiles and
// `words` stash words: descriptors, sync words (uploaded as zeros), counts,
// stashes.
void enc_offsets(uint32_t count, uint64_t tiles, uint64_t words, EncPlan* pl) {
  pl->off_items = 256;
  pl->off_sync = align_up(pl->off_items + sizeof(EncItem) * (uint64_t)count, 256);
  pl->upload = pl->off_sync + 8 * tiles;
  pl->off_counts = align_up(pl->upload, 256);
  pl->off_stash = align_up(pl->off_counts + 4 * tiles, 256);
  pl->total = align_up(pl->off_stash + 4 * words, 256);
}

ciera_status_t enc_layout(const ciera_encode_item_t* items, uint32_t count, EncPlan* pl) {
  if (count && !items) return CIERA_ERR_INVALID_ARG;
  std::map<EncKey, std::vector<uint32_t>> by;
  for (uint32_t i = 0; i < count; ++i) {
    EncKey key;
    if (ciera_status_t s = enc_item_key(items[i], &key)) return s;
    by[key].push_back(i);
  }
  if (by.size() > (size_t)kMaxGroups) return CIERA_ERR_UNSUPPORTED;
  uint64_t tiles = 0, words = 0;
  for (auto& kv : by) {
    Group g{};
    g.dtype = std::get<0>(kv.first);
    g.unit = std::get<1>(kv.first);
    g.tpi = std::get<2>(kv.first);
    g.coded = std::get<3>(kv.first);
    g.self = std::get<4>(kv.first);
    g.item0 = (uint32_t)pl->order.size();
    g.nitems = (uint32_t)kv.second.size();
    if ((uint64_t)g.nitems * g.tpi >= ((uint64_t)1 << 31)) return CIERA_ERR_UNSUPPORTED;
    g.tile0 = tiles;
    g.stash0 = words;
    const uint64_t cap = g.self ? 0 : stash_cap(g.unit, g.coded != 0);
    for (uint32_t k = 0; k < g.nitems; ++k) {
      pl->tile0.push_back(tiles);
      pl->stash.push_back(words);
      tiles += g.tpi;
      words += g.tpi * cap;
    }
    pl->order.insert(pl->order.end(), kv.second.begin(), kv.second.end());
    pl->groups.push_back(g);
  }
  enc_offsets(count, tiles, words, pl);
  return CIERA_OK;
}

struct DecPlan {
  std::vector<uint32_t> order;
  std::vector<Group> groups;
  uint64_t off_items = 0, off_ranks = 0, total = 0;  // ranks: the items' rank pointers, 8 bytes each
};

ciera_status_t dec_layout(const ciera_decode_item_t* items, uint32_t count, DecPlan* pl) {
  if (count && !items) return CIERA_ERR_INVALID_ARG;
  std::map<std::tuple<uint32_t, uint32_t, uint32_t, uint32_t, uint32_t>, std::vector<uint32_t>> by;
  for (uint32_t i = 0; i < count; ++i) {
    const ciera_decode_item_t& it = items[i];
    ciera_status_t s = check_tensor(&it.t);
    if (s) return s;
    uint64_t off, n0;
    shard_of(&it.t, 0, &off, &n0);
    if (n0 >= ((uint64_t)1 << 32)) return CIERA_ERR_UNSUPPORTED;
    const uint32_t U = dec_unit(n0);
    const uint64_t T = (uint64_t)kDecRow * U;
    const uint64_t tpr = std::max<uint64_t>(1, (n0 + T - 1) / T);
    by[std::make_tuple(it.t.dtype, U, (uint32_t)tpr, it.t.world, it.t.flags & CIERA_TENSOR_CODED)].push_back(i);
  }
  if (by.size() > (size_t)kMaxGroups) return CIERA_ERR_UNSUPPORTED;
  for (auto& kv : by) {
    Group g{};
    g.dtype = std::get<0>(kv.first);
    g.unit = std::get<1>(kv.first);
    g.tpr = std::get<2>(kv.first);
    g.world = std::get<3>(kv.first);
    g.coded = std::get<4>(kv.first);
    g.item0 = (uint32_t)pl->order.size();
    g.nitems = (uint32_t)kv.second.size();
    if ((u128)g.nitems * g.tpr * g.world >= ((u128)1 << 31)) return CIERA_ERR_UNSUPPORTED;
    pl->order.insert(pl->order.end(), kv.second.begin(), kv.second.end());
    pl->groups.push_back(g);
  }
  uint64_t nptr = 0;
  for (uint32_t i = 0; i < count; ++i)
    if (items[i].rank_streams) nptr += items[i].t.world;
  pl->off_items = 256;
  pl->off_ranks = align_up(pl->off_items + sizeof(DecItem) * (uint64_t)count, 256);
  pl->total = align_up(pl->off_ranks + 8 * nptr, 256);
  return CIERA_OK;
}

}  // namespace

extern "C" {

uint32_t ciera_abi_version(void) { return CIERA_ABI_VERSION; }

const char* ciera_last_error(void) { return g_last_error; }

const char* ciera_status_str(ciera_status_t s) {
  switch (s) {
    case CIERA_OK: return "ok";
    case CIERA_ERR_INVALID_ARG: return "invalid argument";
    case CIERA_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case CIERA_ERR_UNSUPPORTED: return "unsupported size";
    case CIERA_ERR_DEVICE: return "HIP runtime error";
  }
  return "unknown status";
}

ciera_status_t ciera_shard(const ciera_tensor_t* t, uint32_t rank, uint64_t* offset, uint64_t* n) {
  ciera_status_t s = check_tensor(t);
  if (s) return s;
  if (rank >= t->world || !offset || !n) return CIERA_ERR_INVALID_ARG;
  shard_of(t, rank, offset, n);
  return CIERA_OK;
}

ciera_status_t ciera_plan(const ciera_tensor_t* t, uint32_t change_ppm, const ciera_cost_model_t* cm,
                          ciera_plan_t* out) {
  ciera_status_t s = check_tensor(t);
  if (s) return s;
  if (!out || change_ppm > 1000000u) return CIERA_ERR_INVALID_ARG;
  ciera_cost_model_t c = {8000, 5600000, 5000, 1, 0};
  if (cm) c = *cm;
  if (c.link_bytes_per_us == 0 || c.hbm_bytes_per_us == 0) return CIERA_ERR_INVALID_ARG;
  uint64_t off, n;
  shard_of(t, 0, &off, &n);
  const u128 e = elem_bytes(t->dtype), W = t->world;
  const u128 raw = kHeader + (u128)n * e;
  const u128 P = ((u128)change_ppm * n + 999999u) / 1000000u;
  const u128 comp = kHeader + ((u128)n * sm_bits(t->dtype) + 7) / 8 + (P ? bitmap_bytes(n, t->block_size) + 5 * P : 0);
  std::memset(out, 0, sizeof(*out));
  out->raw_stream_bytes = (uint64_t)raw;
  out->max_stream_bytes = (uint64_t)raw;
  out->expected_changed = (uint64_t)P;
  out->cache_bytes = t->rows * t->cols;
  if (comp >= raw) {
    out->compress = 0;
    out->expected_stream_bytes = (uint64_t)raw;
    out->gain_ns = 0;
    return CIERA_OK;
  }
  const u128 save = (raw - comp) * (W - 1) * 1000u / c.link_bytes_per_us;
  const u128 dec = c.fixed_ns + W * (comp + 2 * (u128)n + (u128)n * e) * 1000u / c.hbm_bytes_per_us;
  const u128 enc = c.overlap_encode ? 0 : c.fixed_ns + ((u128)n * e + n + comp) * 1000u / c.hbm_bytes_per_us;
  const int64_t gain = (int64_t)save - (int64_t)dec - (int64_t)enc;
  out->compress = gain > 0 ? 1u : 0u;
  out->expected_stream_bytes = (uint64_t)(gain > 0 ? comp : raw);
  out->gain_ns = gain;
  return CIERA_OK;
}

ciera_status_t ciera_plan_batch(const ciera_tensor_t* t, const uint32_t* change_ppm, uint32_t count,
                                const ciera_cost_model_t* cm, ciera_plan_t* out) {
  if (count && (!t || !change_ppm || !out)) return CIERA_ERR_INVALID_ARG;
  for (uint32_t i = 0; i < count; ++i)
    if (ciera_status_t s = ciera_plan(t + i, change_ppm[i], cm, out + i)) return s;
  return CIERA_OK;
}

ciera_status_t ciera_select(const ciera_plan_t* plans, uint32_t count, uint64_t cache_budget_bytes,
                            uint32_t* compress_out) {
  if (count && (!plans || !compress_out)) return CIERA_ERR_INVALID_ARG;
  std::vector<uint32_t> cand;
  for (uint32_t i = 0; i < count; ++i) {
    compress_out[i] = 0;
    if (plans[i].gain_ns > 0) cand.push_back(i);
  }
  // a before b when g_a / M_a > g_b / M_b, i.e. g_a * M_b > g_b * M_a (g > 0)
  std::stable_sort(cand.begin(), cand.end(), [plans](uint32_t a, uint32_t b) {
    return (u128)(uint64_t)plans[a].gain_ns * plans[b].cache_bytes >
           (u128)(uint64_t)plans[b].gain_ns * plans[a].cache_bytes;
  });
  u128 used = 0;
  for (uint32_t i : cand) {
    if (used + plans[i].cache_bytes > cache_budget_bytes) break;
    compress_out[i] = 1;
    used += plans[i].cache_bytes;
  }
  return CIERA_OK;
}

// ------------------------------------------------------------------ encode

ciera_status_t ciera_encode_scratch_bytes(const ciera_encode_item_t* items, uint32_t count, uint64_t* bytes) {
  if (!bytes) return CIERA_ERR_INVALID_ARG;
  EncPlan pl;
  ciera_status_t s = enc_layout(items, count, &pl);
  if (s) return s;
  *bytes = pl.total;
  return CIERA_OK;
}

namespace {

// Every item checked as ciera_encode checks it (the layout checked the tensors).
ciera_status_t check_encode_items(const ciera_encode_item_t* items, uint32_t count) {
  for (uint32_t i = 0; i < count; ++i) {
    const ciera_encode_item_t& it = items[i];
    uint64_t off, n;
    shard_of(&it.t, it.rank, &off, &n);
    if (it.compress > kCoded) return CIERA_ERR_INVALID_ARG;
    if (it.compress == kCoded && !(it.t.flags & CIERA_TENSOR_CODED)) return CIERA_ERR_INVALID_ARG;
    if (n && (!it.shard || !aligned(it.shard, 16) || !it.cache_full)) return CIERA_ERR_INVALID_ARG;
    if (n && it.compress == kBlockVariant && !aligned(it.cache_full, 16)) return CIERA_ERR_INVALID_ARG;
    if (!it.stream || !aligned(it.stream, 16)) return CIERA_ERR_INVALID_ARG;
    if (it.stream_capacity < kHeader + n * elem_bytes(it.t.dtype)) return CIERA_ERR_BUFFER_TOO_SMALL;
    // the stream written is disjoint from the shard and the cache slice read
    const uint64_t wlen = kHeader + n * elem_bytes(it.t.dtype);
    const uint64_t clen = it.compress == kBlockVariant ? (n + it.t.block_size - 1) / it.t.block_size * 16 : n;
    const uint8_t* cptr = it.compress == kBlockVariant ? it.cache_full : it.cache_full + off;
    if (overlap(it.stream, wlen, it.shard, n * elem_bytes(it.t.dtype)) ||
        (it.cache_full && overlap(it.stream, wlen, cptr, clen)))
      return CIERA_ERR_INVALID_ARG;
  }
  return CIERA_OK;
}

// The batch's descriptors di[0..count) in group order; *any: some item may be
// compressed; *max_bytes: the largest shard a finishing kernel may rewrite RAW.
void fill_enc_item(const ciera_encode_item_t& it, uint64_t tile0, uint64_t stash, uint32_t batch_id, EncItem& d,
                   uint32_t* any, uint64_t* max_bytes) {
  {
    uint64_t off, n;
    shard_of(&it.t, it.rank, &off, &n);
    d.x = static_cast<const uint8_t*>(it.shard);
    const bool blocks = it.compress == kBlockVariant;
    // the block-hash variant reads and updates the shard's hash cache instead
    d.cache = blocks ? nullptr : it.cache_full + off;
    d.hashes = blocks ? const_cast<uint8_t*>(it.cache_full) : nullptr;
    d.stream = it.stream;
    d.n = n;
    d.off = off;
    d.capacity = it.stream_capacity;
    const uint32_t S = enc_sub(it.t.block_size, n);
    d.tile0 = tile0;
    d.stash = stash;
    d.tvals = (uint32_t)kSub * S;
    d.tpi = (uint32_t)std::max<uint64_t>(1, (n + d.tvals - 1) / d.tvals);
    const bool self = self_finished(it.compress, d.tpi);
    d.cap = self ? 0u : stash_cap(S, it.compress == kCoded);
    d.rank = it.rank;
    d.world = it.t.world;
    d.block_size = it.t.block_size;
    d.compress = it.compress;
    d.cache_aligned = !blocks && aligned(d.cache, 16) ? 1u : 0u;
    d.elem_bytes = elem_bytes(it.t.dtype);
    d.batch_id = batch_id;
    *any |= d.compress != 0;
    if (d.compress && !self) *max_bytes = std::max<uint64_t>(*max_bytes, n * d.elem_bytes);
  }
}
void fill_enc_items(const ciera_encode_item_t* items, uint32_t count, const EncPlan& pl, uint32_t batch_id,
                    EncItem* di, uint32_t* any, uint64_t* max_bytes) {
  *any = 0;
  *max_bytes = 0;
  for (uint32_t j = 0; j < count; ++j)
    fill_enc_item(items[pl.order[j]], pl.tile0[j], pl.stash[j], batch_id, di[j], any, max_bytes);
}

void set_enc_batch(BatchImpl* b, const EncPlan& pl, const Group* groups, uint32_t ngroups, void* scratch,
                   uint64_t scratch_bytes, uint32_t count, uint32_t any, uint64_t max_bytes) {
  b->magic = kEncMagic;
  b->scratch = static_cast<uint8_t*>(scratch);
  b->scratch_bytes = scratch_bytes;
  b->count = count;
  b->ngroups = ngroups;
  b->any_compress = any;
  b->fin_wg = (uint32_t)std::min<uint64_t>(64, std::max<uint64_t>(1, (max_bytes + 65535) / 65536));
  b->off_counts = pl.off_counts;
  b->off_stash = pl.off_stash;
  b->off_items = pl.off_items;
  b->off_sync = pl.off_sync;
  for (uint32_t g = 0; g < ngroups; ++g) b->g[g] = groups[g];
}

}  // namespace

ciera_status_t ciera_encode_prepare(const ciera_encode_item_t* items, uint32_t count, void* scratch,
                                    uint64_t scratch_bytes, ciera_batch_t* batch, void* stream) {
  if (!batch) return CIERA_ERR_INVALID_ARG;
  std::memset(batch, 0, sizeof(*batch));
  EncPlan pl;
  ciera_status_t s = enc_layout(items, count, &pl);
  if (s) return s;
  if (!scratch || !aligned(scratch, 256)) return CIERA_ERR_INVALID_ARG;
  if (scratch_bytes < pl.total) return CIERA_ERR_BUFFER_TOO_SMALL;
  if ((s = check_encode_items(items, count))) return s;
  BatchImpl* b = impl(batch);
  b->batch_id = next_id();
  std::vector<uint8_t> blob(pl.upload, 0);  // descriptors; the sync words go up as zeros
  reinterpret_cast<uint32_t*>(blob.data())[0] = b->batch_id;
  uint32_t any;
  uint64_t max_bytes;
  fill_enc_items(items, count, pl, b->batch_id, reinterpret_cast<EncItem*>(blob.data() + pl.off_items), &any,
                 &max_bytes);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipError_t e = upload(scratch, blob.data(), blob.size(), st)) return device_error("descriptor upload", e);
  set_enc_batch(b, pl, pl.groups.data(), (uint32_t)pl.groups.size(), scratch, scratch_bytes, count, any, max_bytes);
  return CIERA_OK;
}

ciera_status_t ciera_encode_launch(ciera_batch_t* batch, void* stream) {
  if (!batch) return CIERA_ERR_INVALID_ARG;
  BatchImpl* b = impl(batch);
  if (b->magic != kEncMagic) return CIERA_ERR_INVALID_ARG;
  if (b->count == 0) return CIERA_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const EncItem* items = reinterpret_cast<const EncItem*>(b->scratch + b->off_items);
  uint32_t* counts = reinterpret_cast<uint32_t*>(b->scratch + b->off_counts);
  uint32_t* stash = reinterpret_cast<uint32_t*>(b->scratch + b->off_stash);
  for (uint32_t gi = 0; gi < b->ngroups; ++gi) {
    const Group& g = b->g[gi];
    EncArgs a;
    a.items = items;
    a.item0 = g.item0;
    a.tpi = g.tpi;
    a.counts = counts;
    a.stash = stash;
    a.sync = reinterpret_cast<uint64_t*>(b->scratch + b->off_sync);
    a.self = g.self;
    a.polls = g_sync_polls.load(std::memory_order_relaxed);
    if (hipError_t e = launch_encode(g.dtype, g.unit, g.nitems, a, b->batch_id, st))
      return device_error("encode launch", e);
  }
  // finishing kernels: one workgroup per tile for groups of at most kThreads
  // tiles per item (overflowing tiles are then derived again in parallel);
  // per item, over windows of tiles, for larger items
  for (uint32_t gi = 0; gi < b->ngroups; ++gi) {
    const Group& g = b->g[gi];
    if (g.self) continue;  // finished by its own tiles
    hipError_t e;
    if (g.tpi <= (uint32_t)kThreads || g.coded) {
      FinArgs f{};
      f.items = items;
      f.counts = counts;
      f.stash = stash;
      f.tile0 = g.tile0;
      f.stash0 = g.stash0;
      f.item0 = g.item0;
      f.tpi = g.tpi;
      f.cap = stash_cap(g.unit, g.coded != 0);
      if (g.tpi > (uint32_t)kThreads) {  // coded items of many tiles: prefixes first, in the sync words
        uint64_t* prefix = reinterpret_cast<uint64_t*>(b->scratch + b->off_sync);
        f.prefix = prefix;
        if ((e = launch_coded_scan(g.dtype, g.nitems, f, prefix, b->batch_id, st))) return device_error("encode scan launch", e);
      }
      e = launch_encode_finish_tiles(g.dtype, g.coded != 0, g.nitems, f, b->batch_id, st);
    } else {
      e = launch_encode_finish(g.dtype, items, g.item0, g.nitems, b->fin_wg, counts, stash, b->batch_id, st);
    }
    if (e) return device_error("encode finish launch", e);
  }
  b->launches += 1;
  return CIERA_OK;
}

void ciera_set_sync_polls(uint32_t polls) { g_sync_polls.store(polls, std::memory_order_relaxed); }

static_assert(kStaticScratchBytes == CIERA_NOALLOC_SCRATCH_BYTES, "static scratch size");

ciera_status_t ciera_encode_noalloc(const ciera_encode_item_t* items, uint32_t count, void* stream) {
  if (count == 0) return CIERA_OK;
  if (!items) return CIERA_ERR_INVALID_ARG;
  // The groups and the descriptors are laid out as ciera_encode lays them out
  // (same checks in the same order, groups in ascending key order), without
  // heap memory: the keys in a fixed array, each group's descriptors found by
  // a pass over the items, sent a kernel argument pack at a time.
  EncKey keys[kMaxGroups];
  uint32_t nkeys = 0;
  bool too_many = false;
  for (uint32_t i = 0; i < count; ++i) {
    EncKey key;
    if (ciera_status_t s = enc_item_key(items[i], &key)) return s;
    const EncKey* hit = std::find(keys, keys + nkeys, key);
    if (hit == keys + nkeys) {
      if (nkeys == (uint32_t)kMaxGroups) too_many = true;
      else keys[nkeys++] = key;
    }
  }
  if (too_many) return CIERA_ERR_UNSUPPORTED;
  std::sort(keys, keys + nkeys);
  Group groups[kMaxGroups];
  uint64_t tiles = 0;
  uint32_t item0 = 0;
  bool all_self = true;
  for (uint32_t k = 0; k < nkeys; ++k) {
    Group& g = groups[k];
    g = Group{};
    g.dtype = std::get<0>(keys[k]);
    g.unit = std::get<1>(keys[k]);
    g.tpi = std::get<2>(keys[k]);
    g.coded = std::get<3>(keys[k]);
    g.self = std::get<4>(keys[k]);
    g.item0 = item0;
    for (uint32_t i = 0; i < count; ++i) {
      EncKey key;
      (void)enc_item_key(items[i], &key);  // checked above
      if (key == keys[k]) ++g.nitems;
    }
    if ((uint64_t)g.nitems * g.tpi >= ((uint64_t)1 << 31)) return CIERA_ERR_UNSUPPORTED;
    g.tile0 = tiles;
    g.stash0 = 0;
    tiles += (uint64_t)g.nitems * g.tpi;
    item0 += g.nitems;
    all_self = all_self && g.self;
  }
  EncPlan pl;  // offsets only
  enc_offsets(count, tiles, 0, &pl);
  if (ciera_status_t s = check_encode_items(items, count)) return s;
  if (!all_self) return CIERA_ERR_UNSUPPORTED;  // a finishing kernel would need a stash
  if (pl.total > kStaticScratchBytes) return CIERA_ERR_BUFFER_TOO_SMALL;
  void* base = nullptr;
  if (hipError_t e = static_scratch(&base)) return device_error("static scratch lookup", e);
  ciera_batch_t batch;
  std::memset(&batch, 0, sizeof(batch));
  BatchImpl* b = impl(&batch);
  b->batch_id = next_id();
  uint8_t* const sb = static_cast<uint8_t*>(base);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  EncItem* const dst = reinterpret_cast<EncItem*>(sb + pl.off_items);
  constexpr uint32_t kPack = 30;  // descriptors per launch_enc_desc call (it cuts larger counts itself)
  EncItem pack[kPack];
  uint32_t np = 0, sent = 0, any = 0;
  uint64_t max_bytes = 0;
  // descriptors by kernel arguments; the first launch also zeroes the sync
  // words the tiles publish in and writes the batch id
  auto flush = [&]() -> hipError_t {
    hipError_t e = launch_enc_desc(pack, np, dst + sent, sent == 0 ? reinterpret_cast<uint64_t*>(sb + pl.off_sync)
                                                                   : nullptr,
                                   sent == 0 ? (pl.upload - pl.off_sync) / 8 : 0,
                                   sent == 0 ? reinterpret_cast<uint32_t*>(sb) : nullptr, b->batch_id, st);
    sent += np;
    np = 0;
    return e;
  };
  for (uint32_t k = 0; k < nkeys; ++k) {
    uint64_t tile = groups[k].tile0;
    for (uint32_t i = 0; i < count; ++i) {
      EncKey key;
      (void)enc_item_key(items[i], &key);
      if (key != keys[k]) continue;
      fill_enc_item(items[i], tile, 0, b->batch_id, pack[np++], &any, &max_bytes);
      tile += groups[k].tpi;
      if (np == kPack)
        if (hipError_t e = flush()) return device_error("descriptor launch", e);
    }
  }
  if (np)
    if (hipError_t e = flush()) return device_error("descriptor launch", e);
  set_enc_batch(b, pl, groups, nkeys, base, kStaticScratchBytes, count, any, max_bytes);
  return ciera_encode_launch(&batch, stream);
}

ciera_status_t ciera_encode(const ciera_encode_item_t* items, uint32_t count, void* scratch,
                            uint64_t scratch_bytes, void* stream) {
  if (count == 0) return CIERA_OK;
  ciera_batch_t b;
  ciera_status_t s = ciera_encode_prepare(items, count, scratch, scratch_bytes, &b, stream);
  if (s) return s;
  return ciera_encode_launch(&b, stream);
}

// ------------------------------------------------------------------ decode

ciera_status_t ciera_decode_scratch_bytes(const ciera_decode_item_t* items, uint32_t count, uint64_t* bytes) {
  if (!bytes) return CIERA_ERR_INVALID_ARG;
  DecPlan pl;
  ciera_status_t s = dec_layout(items, count, &pl);
  if (s) return s;
  *bytes = pl.total;
  return CIERA_OK;
}

ciera_status_t ciera_decode_prepare(const ciera_decode_item_t* items, uint32_t count, uint32_t* status_dev,
                                    void* scratch, uint64_t scratch_bytes, ciera_batch_t* batch, void* stream) {
  if (!batch) return CIERA_ERR_INVALID_ARG;
  std::memset(batch, 0, sizeof(*batch));
  DecPlan pl;
  ciera_status_t s = dec_layout(items, count, &pl);
  if (s) return s;
  if (!scratch || !aligned(scratch, 256) || !status_dev || !aligned(status_dev, 4)) return CIERA_ERR_INVALID_ARG;
  if (scratch_bytes < pl.total) return CIERA_ERR_BUFFER_TOO_SMALL;
  for (uint32_t i = 0; i < count; ++i) {
    const ciera_decode_item_t& it = items[i];
    uint64_t off, n0;
    shard_of(&it.t, 0, &off, &n0);
    if ((it.streams != nullptr) == (it.rank_streams != nullptr)) return CIERA_ERR_INVALID_ARG;
    if (it.streams && !aligned(it.streams, 16)) return CIERA_ERR_INVALID_ARG;
    if (it.slot_bytes % 16 != 0) return CIERA_ERR_INVALID_ARG;
    if (it.slot_bytes < kHeader + n0 * elem_bytes(it.t.dtype)) return CIERA_ERR_BUFFER_TOO_SMALL;
    if (it.t.rows * it.t.cols && (!it.out_full || !aligned(it.out_full, 16) || !it.cache_full))
      return CIERA_ERR_INVALID_ARG;
    // the rebuilt values, the cache and the streams are disjoint
    const uint64_t N = it.t.rows * it.t.cols, obytes = N * elem_bytes(it.t.dtype);
    if (overlap(it.out_full, obytes, it.cache_full, N)) return CIERA_ERR_INVALID_ARG;
    if (it.streams) {
      const unsigned __int128 sb = (unsigned __int128)it.slot_bytes * it.t.world;
      const uint64_t slen = sb > (unsigned __int128)UINT64_MAX ? UINT64_MAX : (uint64_t)sb;
      if (overlap(it.out_full, obytes, it.streams, slen) || overlap(it.cache_full, N, it.streams, slen))
        return CIERA_ERR_INVALID_ARG;
    } else {
      for (uint32_t r = 0; r < it.t.world; ++r) {
        const uint8_t* p = it.rank_streams[r];
        if (!p || !aligned(p, 16)) return CIERA_ERR_INVALID_ARG;
        if (overlap(it.out_full, obytes, p, it.slot_bytes) || overlap(it.cache_full, N, p, it.slot_bytes))
          return CIERA_ERR_INVALID_ARG;
      }
    }
  }
  BatchImpl* b = impl(batch);
  b->batch_id = next_id();
  std::vector<uint8_t> blob(pl.total, 0);
  reinterpret_cast<uint32_t*>(blob.data())[0] = b->batch_id;
  DecItem* di = reinterpret_cast<DecItem*>(blob.data() + pl.off_items);
  uint64_t nptr = 0;  // rank pointers placed so far
  for (uint32_t j = 0; j < count; ++j) {
    const ciera_decode_item_t& it = items[pl.order[j]];
    DecItem& d = di[j];
    d.streams = it.streams;
    d.ranks = nullptr;
    if (it.rank_streams) {
      const uint64_t at = pl.off_ranks + 8 * nptr;
      std::memcpy(blob.data() + at, it.rank_streams, 8 * (size_t)it.t.world);
      d.ranks = reinterpret_cast<const uint8_t* const*>(static_cast<uint8_t*>(scratch) + at);
      nptr += it.t.world;
    }
    d.slot = it.slot_bytes;
    d.out = static_cast<uint8_t*>(it.out_full);
    d.cache = it.cache_full;
    d.q = it.t.rows / it.t.world;
    d.rem = (uint32_t)(it.t.rows % it.t.world);
    d.cols = it.t.cols;
    d.world = it.t.world;
    d.block_size = it.t.block_size;
    d.batch_id = b->batch_id;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipError_t e = upload(scratch, blob.data(), blob.size(), st)) return device_error("descriptor upload", e);
  b->magic = kDecMagic;
  b->scratch = static_cast<uint8_t*>(scratch);
  b->scratch_bytes = scratch_bytes;
  b->status_dev = status_dev;
  b->count = count;
  b->ngroups = (uint32_t)pl.groups.size();
  b->off_items = pl.off_items;
  for (size_t g = 0; g < pl.groups.size(); ++g) b->g[g] = pl.groups[g];
  return CIERA_OK;
}

ciera_status_t ciera_decode_launch(ciera_batch_t* batch, void* stream) {
  return ciera_decode_launch_bounded(batch, 0, stream);
}

ciera_status_t ciera_decode_launch_bounded(ciera_batch_t* batch, uint32_t max_workgroups, void* stream) {
  if (!batch) return CIERA_ERR_INVALID_ARG;
  BatchImpl* b = impl(batch);
  if (b->magic != kDecMagic) return CIERA_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const DecItem* items = reinterpret_cast<const DecItem*>(b->scratch + b->off_items);
  for (uint32_t gi = 0; gi < b->ngroups; ++gi) {
    const Group& g = b->g[gi];
    if (hipError_t e = launch_decode(g.dtype, g.unit, g.coded != 0, items, g.item0, g.nitems, g.tpr, g.world, b->status_dev,
                                     b->batch_id, max_workgroups, st))
      return device_error("decode launch", e);
  }
  b->launches += 1;
  return CIERA_OK;
}

ciera_status_t ciera_decode(const ciera_decode_item_t* items, uint32_t count, uint32_t* status_dev, void* scratch,
                            uint64_t scratch_bytes, void* stream) {
  if (count == 0) return CIERA_OK;
  ciera_batch_t b;
  ciera_status_t s = ciera_decode_prepare(items, count, status_dev, scratch, scratch_bytes, &b, stream);
  if (s) return s;
  return ciera_decode_launch(&b, stream);
}

ciera_status_t ciera_hash_update(const ciera_tensor_t* t, uint32_t rank, const void* shard, uint8_t* hash_cache,
                                 void* stream) {
  ciera_status_t s = check_tensor(t);
  if (s) return s;
  if (rank >= t->world) return CIERA_ERR_INVALID_ARG;
  uint64_t off, n;
  shard_of(t, rank, &off, &n);
  if (n == 0) return CIERA_OK;
  if (!shard || !aligned(shard, 16) || !hash_cache || !aligned(hash_cache, 16)) return CIERA_ERR_INVALID_ARG;
  if (hipError_t e = launch_hash_seed(t->dtype, static_cast<const uint8_t*>(shard), hash_cache, n, t->block_size,
                                      reinterpret_cast<hipStream_t>(stream)))
    return device_error("hash update launch", e);
  return CIERA_OK;
}

ciera_status_t ciera_cache_update(const ciera_tensor_t* t, const void* weights_full, uint8_t* cache_full,
                                  void* stream) {
  ciera_status_t s = check_tensor(t);
  if (s) return s;
  const uint64_t N = t->rows * t->cols;
  if (N == 0) return CIERA_OK;
  if (!weights_full || !aligned(weights_full, 16) || !cache_full) return CIERA_ERR_INVALID_ARG;
  if (hipError_t e = launch_cache_update(t->dtype, static_cast<const uint8_t*>(weights_full), cache_full, N,
                                         reinterpret_cast<hipStream_t>(stream)))
    return device_error("cache update launch", e);
  return CIERA_OK;
}

}  // extern "C"
