// Host side of the CIERA codec library: argument validation, the per-tensor
// selector, descriptor tables and kernel launches.  See include/ciera.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstring>
#include <map>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "ciera.h"
#include "ciera_internal.h"

using namespace ciera;

namespace {

typedef unsigned __int128 u128;

constexpr uint64_t kMaxElems = (uint64_t)1 << 48;

uint32_t elem_bytes(uint32_t dt) { return dt == CIERA_BF16 ? 2u : 4u; }
uint32_t sm_bytes(uint32_t dt) { return dt == CIERA_BF16 ? 1u : 3u; }

bool pow2(uint32_t x) { return x && !(x & (x - 1)); }

ciera_status_t check_tensor(const ciera_tensor_t* t) {
  if (!t) return CIERA_ERR_INVALID_ARG;
  if (t->dtype != CIERA_BF16 && t->dtype != CIERA_FP32) return CIERA_ERR_INVALID_ARG;
  if (!pow2(t->block_size) || t->block_size < 64 || t->block_size > 4096) return CIERA_ERR_INVALID_ARG;
  if (t->world == 0) return CIERA_ERR_INVALID_ARG;
  if (t->rows >= kMaxElems || t->cols >= kMaxElems) return CIERA_ERR_UNSUPPORTED;
  if ((u128)t->rows * t->cols >= kMaxElems) return CIERA_ERR_UNSUPPORTED;
  return CIERA_OK;
}

// ZeRO-style even row partition: rank r holds floor(R/W) + [r < R%W] rows.
void shard_of(const ciera_tensor_t* t, uint32_t r, uint64_t* off, uint64_t* n) {
  const uint64_t q = t->rows / t->world, rem = t->rows % t->world;
  const uint64_t rows_before = (uint64_t)r * q + std::min<uint64_t>(r, rem);
  const uint64_t my_rows = q + (r < rem ? 1 : 0);
  *off = rows_before * t->cols;
  *n = my_rows * t->cols;
}

uint64_t bitmap_bytes(uint64_t n, uint32_t B) { return ((n + B - 1) / B + 7) / 8; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

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

// Per-call epoch of the encode look-back words; starts from a clock-derived
// value so that words left by an earlier process do not match.
std::atomic<uint32_t> g_epoch{(uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761u};

// ------------------------------------------------------------ encode plan
struct EncGroup {
  uint32_t dtype, sub;
  std::vector<uint32_t> idx;  // item indices
  uint32_t tiles = 0;
  uint64_t off_ctl = 0, off_raw = 0, off_tb = 0, off_items = 0, up_end = 0, off_status = 0;
};

uint32_t sub_for(uint32_t B) { return std::max<uint32_t>(1u, B / 512u); }

ciera_status_t enc_layout(const ciera_encode_item_t* items, uint32_t count,
                          std::vector<EncGroup>* groups, uint64_t* upload_bytes, uint64_t* total) {
  if (count && !items) return CIERA_ERR_INVALID_ARG;
  std::map<std::pair<uint32_t, uint32_t>, size_t> gi;
  for (uint32_t i = 0; i < count; ++i) {
    const ciera_encode_item_t& it = items[i];
    ciera_status_t s = check_tensor(&it.t);
    if (s) return s;
    if (it.rank >= it.t.world) return CIERA_ERR_INVALID_ARG;
    uint64_t off, n;
    shard_of(&it.t, it.rank, &off, &n);
    if (n >= ((uint64_t)1 << 32)) return CIERA_ERR_UNSUPPORTED;
    const auto key = std::make_pair(it.t.dtype, sub_for(it.t.block_size));
    auto f = gi.find(key);
    if (f == gi.end()) {
      gi[key] = groups->size();
      groups->push_back(EncGroup{key.first, key.second, {}});
      f = gi.find(key);
    }
    EncGroup& g = (*groups)[f->second];
    const uint64_t T = (uint64_t)kSub * g.sub;
    const uint64_t nt = std::max<uint64_t>(1, (n + T - 1) / T);
    if ((uint64_t)g.tiles + nt >= ((uint64_t)1 << 31)) return CIERA_ERR_UNSUPPORTED;
    g.tiles += (uint32_t)nt;
    g.idx.push_back(i);
  }
  uint64_t cur = 0;
  for (EncGroup& g : *groups) {
    const uint64_t c = g.idx.size();
    g.off_ctl = align_up(cur, 256);
    g.off_raw = g.off_ctl + sizeof(EncCtl);
    g.off_tb = align_up(g.off_raw + 4 * c, 64);
    g.off_items = align_up(g.off_tb + 4 * c, 64);
    g.up_end = g.off_items + sizeof(EncItem) * c;
    cur = g.up_end;
  }
  *upload_bytes = cur;
  for (EncGroup& g : *groups) {
    g.off_status = align_up(cur, 256);
    cur = g.off_status + 8ull * g.tiles;
  }
  *total = align_up(cur, 256);
  return CIERA_OK;
}

struct DecGroup {
  uint32_t dtype;
  std::vector<uint32_t> idx;
  uint32_t tiles = 0;
  uint64_t off_tb = 0, off_items = 0;
};

ciera_status_t dec_layout(const ciera_decode_item_t* items, uint32_t count,
                          std::vector<DecGroup>* groups, uint64_t* total) {
  if (count && !items) return CIERA_ERR_INVALID_ARG;
  for (uint32_t i = 0; i < count; ++i) {
    const ciera_decode_item_t& it = items[i];
    ciera_status_t s = check_tensor(&it.t);
    if (s) return s;
    uint64_t off, n0;
    shard_of(&it.t, 0, &off, &n0);
    if (n0 >= ((uint64_t)1 << 32)) return CIERA_ERR_UNSUPPORTED;
    DecGroup* g = nullptr;
    for (DecGroup& x : *groups)
      if (x.dtype == it.t.dtype) g = &x;
    if (!g) {
      groups->push_back(DecGroup{it.t.dtype, {}});
      g = &groups->back();
    }
    const uint64_t tpr = std::max<uint64_t>(1, (n0 + kDecTile - 1) / kDecTile);
    const uint64_t nt = tpr * it.t.world;
    if ((uint64_t)g->tiles + nt >= ((uint64_t)1 << 31)) return CIERA_ERR_UNSUPPORTED;
    g->tiles += (uint32_t)nt;
    g->idx.push_back(i);
  }
  uint64_t cur = 0;
  for (DecGroup& g : *groups) {
    g.off_tb = align_up(cur, 256);
    g.off_items = align_up(g.off_tb + 4 * g.idx.size(), 64);
    cur = g.off_items + sizeof(DecItem) * g.idx.size();
  }
  *total = align_up(cur, 256);
  return CIERA_OK;
}

}  // namespace

extern "C" {

uint32_t ciera_abi_version(void) { return CIERA_ABI_VERSION; }

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
  const u128 e = elem_bytes(t->dtype), k = sm_bytes(t->dtype), W = t->world;
  const u128 raw = kHeader + (u128)n * e;
  const u128 P = ((u128)change_ppm * n + 999999u) / 1000000u;
  const u128 comp = kHeader + (u128)n * k + (P ? bitmap_bytes(n, t->block_size) + 5 * P : 0);
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

ciera_status_t ciera_encode_scratch_bytes(const ciera_encode_item_t* items, uint32_t count,
                                          uint64_t* bytes) {
  if (!bytes) return CIERA_ERR_INVALID_ARG;
  std::vector<EncGroup> groups;
  uint64_t up = 0, total = 0;
  ciera_status_t s = enc_layout(items, count, &groups, &up, &total);
  if (s) return s;
  *bytes = total;
  return CIERA_OK;
}

ciera_status_t ciera_encode(const ciera_encode_item_t* items, uint32_t count, void* scratch,
                            uint64_t scratch_bytes, void* stream) {
  if (count == 0) return CIERA_OK;
  std::vector<EncGroup> groups;
  uint64_t up = 0, total = 0;
  ciera_status_t s = enc_layout(items, count, &groups, &up, &total);
  if (s) return s;
  if (!scratch || !aligned(scratch, 256)) return CIERA_ERR_INVALID_ARG;
  if (scratch_bytes < total) return CIERA_ERR_BUFFER_TOO_SMALL;
  for (uint32_t i = 0; i < count; ++i) {
    const ciera_encode_item_t& it = items[i];
    uint64_t off, n;
    shard_of(&it.t, it.rank, &off, &n);
    if (n && (!it.shard || !aligned(it.shard, 16) || !it.cache_full)) return CIERA_ERR_INVALID_ARG;
    if (!it.stream || !aligned(it.stream, 16)) return CIERA_ERR_INVALID_ARG;
    if (it.stream_capacity < kHeader + n * elem_bytes(it.t.dtype)) return CIERA_ERR_BUFFER_TOO_SMALL;
  }
  std::vector<uint8_t> blob(up, 0);  // zeroed control blocks included
  for (EncGroup& g : groups) {
    uint32_t* tb = reinterpret_cast<uint32_t*>(blob.data() + g.off_tb);
    EncItem* di = reinterpret_cast<EncItem*>(blob.data() + g.off_items);
    const uint64_t T = (uint64_t)kSub * g.sub;
    uint32_t tile = 0;
    for (size_t j = 0; j < g.idx.size(); ++j) {
      const ciera_encode_item_t& it = items[g.idx[j]];
      uint64_t off, n;
      shard_of(&it.t, it.rank, &off, &n);
      EncItem& d = di[j];
      d.x = static_cast<const uint8_t*>(it.shard);
      d.cache = it.cache_full + off;
      d.stream = it.stream;
      d.n = n;
      d.off = off;
      d.capacity = it.stream_capacity;
      d.tile_begin = tile;
      d.ntiles = (uint32_t)std::max<uint64_t>(1, (n + T - 1) / T);
      d.rank = it.rank;
      d.world = it.t.world;
      d.block_size = it.t.block_size;
      d.compress = it.compress ? 1u : 0u;
      d.cache_aligned = aligned(d.cache, 16) ? 1u : 0u;
      d.pad = 0;
      tb[j] = tile;
      tile += d.ntiles;
    }
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(scratch);
  if (upload(base, blob.data(), up, st) != hipSuccess) return CIERA_ERR_DEVICE;
  const uint32_t epoch = g_epoch.fetch_add(1u);
  for (EncGroup& g : groups) {
    const EncItem* di = reinterpret_cast<const EncItem*>(base + g.off_items);
    EncCtl* ctl = reinterpret_cast<EncCtl*>(base + g.off_ctl);
    uint32_t* raw = reinterpret_cast<uint32_t*>(base + g.off_raw);
    if (launch_encode(g.dtype, g.sub, di, reinterpret_cast<const uint32_t*>(base + g.off_tb),
                      (uint32_t)g.idx.size(), g.tiles, ctl, raw,
                      reinterpret_cast<uint64_t*>(base + g.off_status), epoch, st) != hipSuccess)
      return CIERA_ERR_DEVICE;
    if (launch_encode_fixup(g.dtype, di, ctl, raw, st) != hipSuccess) return CIERA_ERR_DEVICE;
  }
  return CIERA_OK;
}

ciera_status_t ciera_decode_scratch_bytes(const ciera_decode_item_t* items, uint32_t count,
                                          uint64_t* bytes) {
  if (!bytes) return CIERA_ERR_INVALID_ARG;
  std::vector<DecGroup> groups;
  uint64_t total = 0;
  ciera_status_t s = dec_layout(items, count, &groups, &total);
  if (s) return s;
  *bytes = total;
  return CIERA_OK;
}

ciera_status_t ciera_decode(const ciera_decode_item_t* items, uint32_t count, uint32_t* status_dev,
                            void* scratch, uint64_t scratch_bytes, void* stream) {
  if (count == 0) return CIERA_OK;
  std::vector<DecGroup> groups;
  uint64_t total = 0;
  ciera_status_t s = dec_layout(items, count, &groups, &total);
  if (s) return s;
  if (!scratch || !aligned(scratch, 256) || !status_dev || !aligned(status_dev, 4))
    return CIERA_ERR_INVALID_ARG;
  if (scratch_bytes < total) return CIERA_ERR_BUFFER_TOO_SMALL;
  for (uint32_t i = 0; i < count; ++i) {
    const ciera_decode_item_t& it = items[i];
    if (!it.streams || !aligned(it.streams, 16)) return CIERA_ERR_INVALID_ARG;
    if (it.slot_bytes % 16 != 0) return CIERA_ERR_INVALID_ARG;
    if (it.slot_bytes < kHeader) return CIERA_ERR_BUFFER_TOO_SMALL;
    if (it.t.rows * it.t.cols && (!it.out_full || !aligned(it.out_full, 16) || !it.cache_full))
      return CIERA_ERR_INVALID_ARG;
  }
  std::vector<uint8_t> blob(total, 0);
  for (DecGroup& g : groups) {
    uint32_t* tb = reinterpret_cast<uint32_t*>(blob.data() + g.off_tb);
    DecItem* di = reinterpret_cast<DecItem*>(blob.data() + g.off_items);
    uint32_t tile = 0;
    for (size_t j = 0; j < g.idx.size(); ++j) {
      const ciera_decode_item_t& it = items[g.idx[j]];
      uint64_t off, n0;
      shard_of(&it.t, 0, &off, &n0);
      DecItem& d = di[j];
      d.streams = it.streams;
      d.slot = it.slot_bytes;
      d.out = static_cast<uint8_t*>(it.out_full);
      d.cache = it.cache_full;
      d.rows = it.t.rows;
      d.cols = it.t.cols;
      d.tile_begin = tile;
      d.tiles_per_rank = (uint32_t)std::max<uint64_t>(1, (n0 + kDecTile - 1) / kDecTile);
      d.world = it.t.world;
      d.block_size = it.t.block_size;
      tb[j] = tile;
      tile += d.tiles_per_rank * d.world;
    }
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* base = static_cast<uint8_t*>(scratch);
  if (upload(base, blob.data(), total, st) != hipSuccess) return CIERA_ERR_DEVICE;
  for (DecGroup& g : groups) {
    if (launch_decode(g.dtype, reinterpret_cast<const DecItem*>(base + g.off_items),
                      reinterpret_cast<const uint32_t*>(base + g.off_tb), (uint32_t)g.idx.size(),
                      g.tiles, status_dev, st) != hipSuccess)
      return CIERA_ERR_DEVICE;
  }
  return CIERA_OK;
}

ciera_status_t ciera_cache_update(const ciera_tensor_t* t, const void* weights_full,
                                  uint8_t* cache_full, void* stream) {
  ciera_status_t s = check_tensor(t);
  if (s) return s;
  const uint64_t N = t->rows * t->cols;
  if (N == 0) return CIERA_OK;
  if (!weights_full || !aligned(weights_full, 16) || !cache_full) return CIERA_ERR_INVALID_ARG;
  if (launch_cache_update(t->dtype, static_cast<const uint8_t*>(weights_full), cache_full, N,
                          reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return CIERA_ERR_DEVICE;
  return CIERA_OK;
}

}  // extern "C"
