/*
 * ciera.h -- C ABI of the CIERA exponent-reuse codec for MI355X (gfx950).
 *
 * Method: "CIERA: Cross-Iteration Exponent Reuse for Lossless Allgather in
 * Sharded MoE Training" (arXiv 2609.04609v1), cited as [CIERA].  Every value of
 * a rank's weight shard is split into exponent and sign|mantissa bits; the
 * exponents of the previous iteration are cached on every rank; a rank sends
 * the sign|mantissa bits of all its values plus only the exponents that
 * changed, and every receiver rebuilds the full tensor bit-exactly from its
 * cache [CIERA section 3.1; Appendix A, Algorithm 1].  A per-tensor selector
 * keeps compression only where it saves time [CIERA section 3.2].
 *
 * Stream format (one stream per (tensor, rank); all integers little-endian):
 *   header, 64 bytes:
 *     [0,4) "CIER"  [4,6) version=1  [6] dtype  [7] mode (0 RAW, 1 COMPRESSED, 2 BLOCK, 3 CODED)
 *     [8,12) block size B  [12,16) 0  [16,24) n  [24,32) n_changed
 *     [32,40) total_len  [40,48) element offset of the shard in the tensor
 *     [48,52) rank  [52,56) world  [56,64) 0
 *   COMPRESSED body: n sign|mantissa records (bf16: 1 byte, sign in bit 7 and
 *     the 7 mantissa bits below; fp32: 3 bytes of sign<<23|mantissa; fp16:
 *     the 11-bit values sign<<10|mantissa back to back in one bit stream,
 *     least significant bit first, ceil(11n/8) bytes -- the exponent of an
 *     fp16 value is its 5-bit field, cached in a byte), then --
 *     only if n_changed > 0 -- a bitmap of ceil(ceil(n/B)/8) bytes (bit b =
 *     byte b/8, bit b%8: block b of B values holds a changed exponent), then
 *     n_changed records of 5 bytes (u32 shard-local index, u8 exponent) in
 *     strictly ascending index order.
 *   BLOCK body (the block-hash variant, the pages' own change detection): the
 *     n sign|mantissa records as above, then -- only if n_changed > 0, which
 *     here counts changed blocks -- the bitmap (bit b: block b's exponents
 *     changed) and the exponent bytes of every changed block, B bytes each in
 *     block order, the last block zero-padded to B.
 *   CODED body (entropy-coded patches [CIERA 3.1: changed exponents ANS-coded]):
 *     the n sign|mantissa records, then -- only if n_changed > 0 -- the bitmap,
 *     zero bytes up to a multiple of 4 from the stream start, a chunk table and
 *     the chunks' data.  The shard is cut into chunks of 4096 values from value
 *     0; the table holds two u32 per chunk: the changed values and the data
 *     bytes of this and all earlier chunks.  A chunk's data is dense -- its
 *     exponent bytes, zero-padded to a multiple of 4 -- when that is what its
 *     byte count says, else range-ANS data: L = min(64, ceil(c/4)) final coder
 *     states (u32), 16-bit words, a zero word when their number is odd.  Change
 *     j of the chunk (index order) belongs to state j mod L and is four
 *     symbols: its gap bucket b = bit length of (gap + 1), gap = index -
 *     previous index - 1 (previous -1 at the chunk start), coded with the
 *     frequencies (sum 4096) of a geometric gap model with p = c / chunk
 *     length in 32-bit fixed point; the b - 1 bits of gap + 1 below its
 *     leading one; its exponent class (+1, -1, +2, -2, ..., +7, -7 modulo 256,
 *     else escape; frequencies 2032, 2032, twelve of 2, 8); for an escape the
 *     new exponent as 8 bits.  States stay in [2^16, 2^32); decoding takes the
 *     changes L at a time and their four symbols as four sub-steps, after each
 *     of which every state below 2^16, in state order, reads the next word.
 *     The encoder sends a chunk dense when it has more than 1024 changes or
 *     when the coded data would not be shorter.
 *   RAW body: the n values as stored (2 or 4 bytes each).
 *   fp16 extends the pages' bf16/fp32 scope the same way; its layout is this
 *   library's reading, not a format of the pages.
 *   A stream is COMPRESSED (BLOCK, CODED) only if the caller asked for it and
 *   it is strictly shorter than the RAW stream (64 + n*element bytes).
 *
 * Sharding: a tensor of rows x cols (row-major; a 1-D vector is rows=len,
 * cols=1) is split over W ranks by rows; rank r holds floor(R/W) + [r < R%W]
 * consecutive rows (ZeRO-style even partition).  Patch indices are u32, so a
 * shard holds fewer than 2^32 values (larger shards: CIERA_ERR_UNSUPPORTED).
 *
 * Conventions for every device call:
 *   - all pointers are device pointers of the current HIP device unless noted;
 *     the caller owns every buffer; nothing is retained after the call returns
 *     except what the call's kernels still read until they complete;
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream);
 *     calls are asynchronous on it and never synchronize the host with it;
 *   - argument errors are returned synchronously, before anything is enqueued;
 *     CIERA_ERR_DEVICE reports a failed HIP call (copy or launch);
 *   - a call may be issued concurrently with other calls on other streams only
 *     with scratch buffers of its own.
 */
#ifndef CIERA_H
#define CIERA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CIERA_ABI_VERSION 4u
#define CIERA_HEADER_BYTES 64u

typedef enum { CIERA_BF16 = 1, CIERA_FP32 = 2, CIERA_FP16 = 3 } ciera_dtype_t;

typedef enum {
  CIERA_OK = 0,
  CIERA_ERR_INVALID_ARG = 1,      /* null / misaligned pointer, bad dtype, B, world, rank */
  CIERA_ERR_BUFFER_TOO_SMALL = 2, /* stream capacity, slot or scratch too small */
  CIERA_ERR_UNSUPPORTED = 3,      /* a shard of >= 2^32 values, sizes beyond 2^48, or a CODED
                                     shard of 2^31 values or more */
  CIERA_ERR_DEVICE = 4            /* a HIP runtime call failed */
} ciera_status_t;

/* Bits OR-ed into *status_dev by ciera_decode (the caller zeroes it first).
 * They are format validation, not an integrity check: they flag a stream that
 * does not parse as a stream of its shard (so that its decode never reaches
 * outside its buffers), not every edit of a well-formed one.  Edits that decode
 * with status 0 and a different output include: any sign|mantissa byte; any
 * byte of a RAW body; a patch record's exponent byte; a record's index moved
 * within its block without passing a neighbour; BLOCK payload bytes; and in
 * CODED data, bits of a coder state that the raw-bit symbols of a gap absorb
 * (the low bits of a state at a change's first step pass through to its gap's
 * raw bits and leave the state as before: every later change of the chunk
 * moves by the same amount, and only a move across a block boundary or past
 * the chunk is flagged).  Integrity in transit is the transport's; the pages'
 * payload carries no checksum either. */
#define CIERA_ST_MAGIC 1u  /* bad magic or version */
#define CIERA_ST_FIELD 2u  /* dtype, B, n, offset, rank, world or mode mismatch */
#define CIERA_ST_LENGTH 4u /* total_len / n_changed inconsistent or beyond the slot; CODED: a
                              chunk table entry out of order or range (that chunk is skipped) */
#define CIERA_ST_PATCH 8u  /* a patch index >= n, or indices not strictly ascending; CODED: a
                              change past its chunk, an exponent wider than the field, words
                              missing or left over, a final state other than 2^16, or dense
                              data whose differences from the cache number other than the
                              chunk's count */
#define CIERA_ST_BITMAP 16u /* bitmap disagrees with the patches (unspecified with ST_PATCH, and
                               for CODED with ST_LENGTH); BLOCK: set bits other than n_changed,
                               or a set bit past the last block */

/* One logical tensor and how it is sharded.  block_size is B, a power of two in
 * [64, 4096] (the pages sweep 256..4096 and default to 512 [CIERA 4.1, 4.5]).
 * flags: 0, or CIERA_TENSOR_CODED when the tensor's streams may be CODED --
 * required to encode with compress = 3 and to decode CODED streams (the
 * decode of such tensors runs a kernel with the rANS decoder; without the
 * flag a CODED stream is a mode mismatch, CIERA_ST_FIELD). */
#define CIERA_TENSOR_CODED 1u
typedef struct {
  uint64_t rows, cols;
  uint32_t dtype;      /* ciera_dtype_t */
  uint32_t block_size; /* B */
  uint32_t world;      /* W >= 1 */
  uint32_t flags;      /* 0 or CIERA_TENSOR_CODED */
} ciera_tensor_t;

/* Cost model of the selector: bytes per microsecond of the Allgather bus and of
 * HBM, a fixed per-kernel cost, and whether encode is overlapped with other work
 * (then it costs nothing on the critical path [CIERA 3.2, 3.3]). */
typedef struct {
  uint64_t link_bytes_per_us; /* default 8000: ~8 GB/s cross-node AllGather bus [CIERA 4.1] */
  uint64_t hbm_bytes_per_us;  /* default 5,600,000: 70% of 8 TB/s */
  uint64_t fixed_ns;          /* default 5000 */
  uint32_t overlap_encode;    /* default 1 */
  uint32_t reserved;
} ciera_cost_model_t;

typedef struct {
  uint32_t compress;              /* 1: encode COMPRESSED (subject to the length rule) */
  uint32_t reserved;
  uint64_t raw_stream_bytes;      /* 64 + n0*e for the largest shard n0 (rank 0) */
  uint64_t max_stream_bytes;      /* capacity every stream / receive slot needs */
  uint64_t expected_stream_bytes; /* model payload of rank 0 at the given change rate */
  uint64_t expected_changed;      /* ceil(change_ppm * n0 / 1e6) */
  uint64_t cache_bytes;           /* exponent cache per rank: one byte per tensor value */
  int64_t gain_ns;                /* modelled saving per Allgather; 0 when comp >= raw */
} ciera_plan_t;

/* ciera_plan -- per-tensor selector [CIERA 3.2]:
 *   g = Comm(S) - [Comm(S') + T_enc + T_dec], compress iff g > 0.
 * With n0 = rank 0's shard, P = ceil(change_ppm*n0/1e6), comp/raw the stream
 * lengths above (all integer, divisions floor in this order):
 *   save = (raw-comp)*(W-1)*1000 / link;  dec = fixed + W*(comp+2*n0+n0*e)*1000 / hbm;
 *   enc  = overlap ? 0 : fixed + (n0*e+n0+comp)*1000 / hbm;  gain = save-dec-enc.
 * If comp >= raw the answer is RAW with gain 0.  Host only, pure; cm may be NULL
 * for the defaults.  Errors: INVALID_ARG for a bad tensor or null t/out. */
ciera_status_t ciera_plan(const ciera_tensor_t* t, uint32_t change_ppm,
                          const ciera_cost_model_t* cm, ciera_plan_t* out);

/* ciera_plan_batch -- ciera_plan for `count` tensors in one call (one plan per
 * iteration of a whole layer without a call per tensor): out[i] is exactly
 * ciera_plan(&t[i], change_ppm[i], cm, &out[i]).  t, change_ppm and out are host
 * arrays of `count` entries.  Errors: INVALID_ARG for null arrays (count > 0);
 * otherwise the status of the first tensor ciera_plan rejects (out[i] for that
 * i and after it are then unspecified). */
ciera_status_t ciera_plan_batch(const ciera_tensor_t* t, const uint32_t* change_ppm, uint32_t count,
                                const ciera_cost_model_t* cm, ciera_plan_t* out);

/* ciera_select -- benefit-driven selection under a cache budget [CIERA 3.2]:
 * among the tensors whose plan has a positive gain (plans[i].gain_ns > 0), rank
 * them by gain per byte of exponent cache, gain_ns / cache_bytes, descending
 * (exact integer cross-multiplication; equal ratios keep the input order; a
 * tensor with no cache ranks first), then take them in that order while the
 * running total of cache_bytes stays <= cache_budget_bytes, stopping at the
 * first one that does not fit.  compress_out[i] = 1 for the selected tensors,
 * 0 for all others.  plans: count host plans from ciera_plan; compress_out:
 * count host words, caller-owned.  Host only, pure.  Errors: INVALID_ARG when
 * count > 0 and plans or compress_out is NULL. */
ciera_status_t ciera_select(const ciera_plan_t* plans, uint32_t count, uint64_t cache_budget_bytes,
                            uint32_t* compress_out);

/* ciera_shard -- element offset and count of rank's row shard.  Host only. */
ciera_status_t ciera_shard(const ciera_tensor_t* t, uint32_t rank, uint64_t* offset,
                           uint64_t* n);

/* One rank's shard of one tensor to encode. */
typedef struct {
  ciera_tensor_t t;
  uint32_t rank;              /* < t.world */
  uint32_t compress;          /* 0 always RAW; 1 COMPRESSED (the plan's decision); 2 the
                                 block-hash variant (BLOCK); 3 CODED (t.flags must hold
                                 CIERA_TENSOR_CODED; shards of fewer than 2^31 values,
                                 so that the chunk table's u32 byte counts hold
                                 their data); each subject to the
                                 length rule */
  const void* shard;          /* n_r values of t.dtype; 16-byte aligned */
  const uint8_t* cache_full;  /* compress 0/1/3: N = rows*cols cached exponents; [off_r, off_r+n_r)
                                 is read.  compress 2: the shard's hash cache instead --
                                 16 bytes per block of B values (two little-endian u64),
                                 16-byte aligned -- read and updated in place */
  uint8_t* stream;            /* output; 16-byte aligned */
  uint64_t stream_capacity;   /* >= 64 + n_r*e (the RAW length) */
} ciera_encode_item_t;

/* A prepared batch: host-side handle of a batch whose descriptor tables already
 * sit in the caller's device scratch, so that each launch enqueues kernels only
 * (no host-to-device traffic).  Caller-owned plain bytes; not shareable between
 * threads during a call.  The scratch belongs to the batch until it is prepared
 * anew: preparing another batch in the same scratch invalidates this one (its
 * kernels then detect the foreign contents and write nothing). */
#define CIERA_BATCH_BYTES 4096u
typedef struct {
  uint64_t opaque[CIERA_BATCH_BYTES / 8];
} ciera_batch_t;

/* ciera_encode_scratch_bytes -- device scratch ciera_encode needs for this batch. */
ciera_status_t ciera_encode_scratch_bytes(const ciera_encode_item_t* items, uint32_t count,
                                          uint64_t* bytes);

/* ciera_encode -- sender side of one Allgather for `count` shards in one batch
 * [CIERA 3.1; Algorithm 1 sender]: split every value, compare its exponent with
 * the cached one, write the sign|mantissa bytes, the per-block bitmap and the
 * ascending (index, exponent) patch list, or a RAW stream when the plan says so
 * or when the compressed stream would not be shorter.  Each stream's header
 * (total_len, n_changed, mode) is written on the device; the host is never
 * synchronized.  Bytes of a stream past its total_len are unspecified.  A
 * stream's first 64 + n*e bytes must not overlap its shard or its cache slice
 * (the hash cache for compress = 2): INVALID_ARG.  `items` is a host array.  Scratch: a device buffer of at least
 * ciera_encode_scratch_bytes, 256-byte aligned, used only until the call's
 * kernels complete.  Encode cannot fail on data: every bit pattern is valid. */
ciera_status_t ciera_encode(const ciera_encode_item_t* items, uint32_t count, void* scratch,
                            uint64_t scratch_bytes, void* stream);

/* ciera_encode_prepare -- validate `items` (host array) exactly as ciera_encode
 * does, write the batch's tables into `scratch` (one host-to-device copy on
 * `stream`) and fill *batch.  The items' buffers are bound to the batch: every
 * launch encodes whatever they hold at that point of the stream.
 * ciera_encode_launch -- one encode of a prepared batch on `stream` (the one it
 * was prepared on, or a stream ordered after it).  ciera_encode is prepare +
 * launch.  Launches of one batch must not overlap in time. */
ciera_status_t ciera_encode_prepare(const ciera_encode_item_t* items, uint32_t count, void* scratch,
                                    uint64_t scratch_bytes, ciera_batch_t* batch, void* stream);
ciera_status_t ciera_encode_launch(ciera_batch_t* batch, void* stream);

/* ciera_set_sync_polls -- the tiles of an element-patch or RAW shard of at
 * most 256 encode tiles finish the stream themselves: each publishes its change
 * count and reads its siblings' (the item's total decides the mode, the counts
 * before it place its records).  A tile polls a sibling's count at most `polls`
 * times (0: the default, about a millisecond) and otherwise counts that
 * sibling's changes itself from the shard and the cache, so the streams are the
 * same either way; a small value exercises that path.  Process-wide; takes
 * effect at the next launch.  Host only. */
void ciera_set_sync_polls(uint32_t polls);

/* ciera_encode_noalloc -- ciera_encode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same streams, byte for byte, with the library's own
 * device array of CIERA_NOALLOC_SCRATCH_BYTES (one per device, held until the
 * process ends) in place of a caller's scratch.  It allocates no memory,
 * device or host: no hipMalloc or other allocating HIP or library routine, no
 * heap -- the batch's launch groups and descriptors are laid out in fixed-size
 * arrays, and the descriptors reach the device as kernel arguments of a small
 * kernel, which also clears the count words the tiles publish.  Limits:
 * element patches and RAW (compress 0 or 1) of shards of at most 256 encode
 * tiles (2^21 values at B <= 1024), else CIERA_ERR_UNSUPPORTED; a batch whose
 * scratch (ciera_encode_scratch_bytes) exceeds CIERA_NOALLOC_SCRATCH_BYTES
 * (about 7,000 items of 16 tiles), CIERA_ERR_BUFFER_TOO_SMALL.  Every call on
 * a device uses that device's one array and leaves its contents behind: calls
 * that overlap in time on one device (other streams, other threads) race and
 * must not be issued.  Argument checks as for ciera_encode. */
#define CIERA_NOALLOC_SCRATCH_BYTES 1048576u
ciera_status_t ciera_encode_noalloc(const ciera_encode_item_t* items, uint32_t count, void* stream);

/* The W received streams of one tensor, in one of two layouts: W slots of one
 * buffer (`streams`, what a fixed-slot Allgather delivers), or W buffers
 * anywhere (`rank_streams`, one per sending rank). */
typedef struct {
  ciera_tensor_t t;
  const uint8_t* streams; /* rank r's stream starts at streams + r*slot_bytes; 16-byte aligned.
                             NULL when rank_streams is given */
  uint64_t slot_bytes;    /* multiple of 16, >= the RAW length of rank 0's shard
                             (ciera_plan's max_stream_bytes): every slot can hold any stream.
                             With rank_streams: the bytes readable at each rank's pointer */
  void* out_full;         /* N values, rebuilt; 16-byte aligned */
  uint8_t* cache_full;    /* N bytes: exponents of the previous iteration, updated in place */
  const uint8_t* const* rank_streams; /* optional host array of t.world device pointers: rank r's
                             stream at rank_streams[r], 16-byte aligned, slot_bytes readable
                             there; none of the W ranges may overlap out_full or cache_full
                             (they may overlap each other).  The pointers are copied into the
                             decode scratch by ciera_decode / ciera_decode_prepare; the array
                             need not outlive the call.  NULL: the slot layout of `streams` */
} ciera_decode_item_t;

/* ciera_decode_scratch_bytes -- device scratch ciera_decode needs for this batch. */
ciera_status_t ciera_decode_scratch_bytes(const ciera_decode_item_t* items, uint32_t count,
                                          uint64_t* bytes);

/* ciera_decode -- receiver side [CIERA 3.1; Algorithm 1 receiver]: for every
 * rank's stream take the cached exponents of its shard, replace the changed
 * ones, merge them with the sign|mantissa bytes into out_full and leave the
 * cache equal to the exponents of the rebuilt values.  RAW streams are copied
 * and refresh the cache too.  Validation sets CIERA_ST_* bits in *status_dev
 * (a device uint32_t the caller zeroed); a shard whose header or lengths are
 * bad is left untouched (CODED: a chunk whose table entry is bad), a shard
 * with bad patches or bitmap is rebuilt in an unspecified way -- in no case is
 * memory outside the item's buffers touched.  For a CODED stream the decode
 * first writes each coded chunk's changes as 4-byte records at the start of
 * that chunk's part of out_full, then overwrites them with the values.
 * out_full, the cache and the W slots (or the W rank_streams ranges) must not
 * overlap: INVALID_ARG; so are both or neither of streams and rank_streams
 * set, and a null or misaligned rank pointer.  `items` is a host array.
 * Scratch as for encode (ciera_decode_scratch_bytes counts 8 bytes per rank
 * pointer). */
ciera_status_t ciera_decode(const ciera_decode_item_t* items, uint32_t count,
                            uint32_t* status_dev, void* scratch, uint64_t scratch_bytes,
                            void* stream);

/* ciera_decode_prepare / ciera_decode_launch -- the prepared form of
 * ciera_decode, as for encode; status_dev is bound to the batch. */
ciera_status_t ciera_decode_prepare(const ciera_decode_item_t* items, uint32_t count,
                                    uint32_t* status_dev, void* scratch, uint64_t scratch_bytes,
                                    ciera_batch_t* batch, void* stream);
ciera_status_t ciera_decode_launch(ciera_batch_t* batch, void* stream);

/* ciera_decode_launch_bounded -- ciera_decode_launch from a grid of at most
 * max_workgroups workgroups per kernel launch, each decoding tiles of 8192
 * values in turn (0: one workgroup per tile, as ciera_decode_launch).  For a
 * decode that runs beside other work on another stream [CIERA 3.3: the codec
 * overlapped with communication and compute]: the bound caps the compute units
 * the decode holds at once.  Same results; tensors flagged CIERA_TENSOR_CODED
 * are decoded as by ciera_decode_launch. */
ciera_status_t ciera_decode_launch_bounded(ciera_batch_t* batch, uint32_t max_workgroups, void* stream);

/* ciera_hash_update -- the block-hash variant's sender state [CIERA 3.1;
 * Algorithm 1 (HashCache)]: for rank's shard of t (n_r values), hash_cache
 * receives the 128-bit hash of every block's exponents, 16 bytes per block
 * (ceil(n_r/B) blocks): two 64-bit halves, each
 *   mix64((sum_j mix64(w_j ^ (seed + (j+1)*0x9E3779B97F4A7C15)) + L) mod 2^64)
 * over the block's exponent bytes as little-endian 8-byte words w_j (the last
 * zero-padded), L the block's length in bytes, mix64 the SplitMix64 output
 * function, seeds 0x243F6A8885A308D3 and 0x13198A2E03707344.  Seeds the cache
 * when reuse is switched on; encode with compress = 2 keeps it current.
 * shard and hash_cache 16-byte aligned.  Errors: INVALID_ARG for a bad tensor,
 * rank or pointer. */
ciera_status_t ciera_hash_update(const ciera_tensor_t* t, uint32_t rank, const void* shard,
                                 uint8_t* hash_cache, void* stream);

/* ciera_cache_update -- cache_full[i] = exponent of weights_full[i] for the
 * whole tensor: seeds the cache when exponent reuse is switched on after
 * warmup [CIERA 2.2, 3.1].  weights_full 16-byte aligned. */
ciera_status_t ciera_cache_update(const ciera_tensor_t* t, const void* weights_full,
                                  uint8_t* cache_full, void* stream);

const char* ciera_status_str(ciera_status_t s);
uint32_t ciera_abi_version(void);

/* ciera_last_error -- which HIP call failed, and how, behind the calling
 * thread's most recent CIERA_ERR_DEVICE (a static per-thread string). */
const char* ciera_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CIERA_H */
