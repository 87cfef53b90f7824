// gfx950 kernels of the CIERA exponent-reuse codec.
//
// [CIERA section 3.1; Appendix A, Algorithm 1]: the sender splits every value
// into exponent and sign|mantissa bits, detects which exponents differ from the
// cached ones and emits the sign|mantissa bytes, a per-block change bitmap and
// the changed exponents; the receiver merges the sign|mantissa bytes with its
// cached exponents after replacing the changed ones.
//
// Everything here is integer bit manipulation on HBM-resident buffers: no MFMA,
// no floating point on data (so NaN payloads, -0 and subnormals pass through).
// Work is cut into tiles of 4096 values per 256-thread workgroup, 16 contiguous
// values per thread, moved with 16-byte loads and stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ciera.h"
#include "ciera_internal.h"

namespace ciera {
namespace {

template <int DT>
struct Tr;
template <>
struct Tr<1> {  // bf16: 1 sign, 8 exponent, 7 mantissa bits
  static constexpr int E = 2, K = 1, SHIFT = 7;
};
template <>
struct Tr<2> {  // fp32: 1 sign, 8 exponent, 23 mantissa bits
  static constexpr int E = 4, K = 3, SHIFT = 23;
};

template <int DT>
__device__ __forceinline__ uint32_t exp_of(uint32_t v) {
  return (v >> Tr<DT>::SHIFT) & 0xFFu;
}
// sign|mantissa: bf16 -> sign<<7 | mantissa(7); fp32 -> sign<<23 | mantissa(23)
template <int DT>
__device__ __forceinline__ uint32_t sm_of(uint32_t v) {
  if constexpr (DT == 1) return ((v >> 8) & 0x80u) | (v & 0x7Fu);
  else return ((v >> 8) & 0x800000u) | (v & 0x7FFFFFu);
}
template <int DT>
__device__ __forceinline__ uint32_t join(uint32_t sm, uint32_t ex) {
  if constexpr (DT == 1) return ((sm & 0x80u) << 8) | (ex << 7) | (sm & 0x7Fu);
  else return ((sm & 0x800000u) << 8) | (ex << 23) | (sm & 0x7FFFFFu);
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// --------------------------------------------------------------- 16-value I/O

// 16 values starting at p (p = base + c0*E, 16-byte aligned when cnt == 16).
template <int DT>
__device__ __forceinline__ void load16(const uint8_t* p, int cnt, uint32_t v[16]) {
  if (cnt == 16) {
    if constexpr (DT == 1) {
      const uint4 a = reinterpret_cast<const uint4*>(p)[0];
      const uint4 b = reinterpret_cast<const uint4*>(p)[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[2 * j] = w[j] & 0xFFFFu;
        v[2 * j + 1] = w[j] >> 16;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[q];
        v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < cnt) {
        if constexpr (DT == 1) v[j] = reinterpret_cast<const uint16_t*>(p)[j];
        else v[j] = reinterpret_cast<const uint32_t*>(p)[j];
      } else {
        v[j] = 0;
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void store16(uint8_t* p, int cnt, const uint32_t v[16], bool vec = true) {
  if (cnt == 16 && vec) {
    if constexpr (DT == 1) {
      uint4 a, b;
      a.x = v[0] | (v[1] << 16); a.y = v[2] | (v[3] << 16);
      a.z = v[4] | (v[5] << 16); a.w = v[6] | (v[7] << 16);
      b.x = v[8] | (v[9] << 16); b.y = v[10] | (v[11] << 16);
      b.z = v[12] | (v[13] << 16); b.w = v[14] | (v[15] << 16);
      reinterpret_cast<uint4*>(p)[0] = a;
      reinterpret_cast<uint4*>(p)[1] = b;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 a;
        a.x = v[4 * q]; a.y = v[4 * q + 1]; a.z = v[4 * q + 2]; a.w = v[4 * q + 3];
        reinterpret_cast<uint4*>(p)[q] = a;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < cnt) {
        if constexpr (DT == 1) reinterpret_cast<uint16_t*>(p)[j] = (uint16_t)v[j];
        else reinterpret_cast<uint32_t*>(p)[j] = v[j];
      }
    }
  }
}

// 16 bytes (cache exponents) as four little-endian words.
__device__ __forceinline__ void load_bytes16(const uint8_t* p, int cnt, bool aligned, uint32_t c[4]) {
  if (cnt == 16 && aligned) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w;
  } else {
    c[0] = c[1] = c[2] = c[3] = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < cnt) c[j >> 2] |= (uint32_t)p[j] << (8 * (j & 3));
  }
}

__device__ __forceinline__ void store_bytes16(uint8_t* p, int cnt, bool aligned, const uint32_t c[4]) {
  if (cnt == 16 && aligned) {
    uint4 a;
    a.x = c[0]; a.y = c[1]; a.z = c[2]; a.w = c[3];
    *reinterpret_cast<uint4*>(p) = a;
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < cnt) p[j] = (uint8_t)(c[j >> 2] >> (8 * (j & 3)));
  }
}

__device__ __forceinline__ uint32_t byte_of(const uint32_t c[4], int j) {
  return (c[j >> 2] >> (8 * (j & 3))) & 0xFFu;
}

// sign|mantissa records of 16 values: bf16 16 bytes, fp32 48 bytes (3 per value, LE).
template <int DT>
__device__ __forceinline__ void store_sm16(uint8_t* p, int cnt, const uint32_t sm[16]) {
  if constexpr (DT == 1) {
    uint32_t c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      c[q] = sm[4 * q] | (sm[4 * q + 1] << 8) | (sm[4 * q + 2] << 16) | (sm[4 * q + 3] << 24);
    store_bytes16(p, cnt, true, c);
  } else {
    if (cnt == 16) {
      uint32_t w[12];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t a = sm[4 * q], b = sm[4 * q + 1], c = sm[4 * q + 2], d = sm[4 * q + 3];
        w[3 * q] = a | (b << 24);
        w[3 * q + 1] = (b >> 8) | (c << 16);
        w[3 * q + 2] = (c >> 16) | (d << 8);
      }
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        uint4 o;
        o.x = w[4 * q]; o.y = w[4 * q + 1]; o.z = w[4 * q + 2]; o.w = w[4 * q + 3];
        reinterpret_cast<uint4*>(p)[q] = o;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j < cnt) {
          p[3 * j] = (uint8_t)sm[j];
          p[3 * j + 1] = (uint8_t)(sm[j] >> 8);
          p[3 * j + 2] = (uint8_t)(sm[j] >> 16);
        }
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void load_sm16(const uint8_t* p, int cnt, uint32_t sm[16]) {
  if constexpr (DT == 1) {
    uint32_t c[4];
    load_bytes16(p, cnt, true, c);
#pragma unroll
    for (int j = 0; j < 16; ++j) sm[j] = byte_of(c, j);
  } else {
    if (cnt == 16) {
      uint32_t w[12];
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[q];
        w[4 * q] = a.x; w[4 * q + 1] = a.y; w[4 * q + 2] = a.z; w[4 * q + 3] = a.w;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w0 = w[3 * q], w1 = w[3 * q + 1], w2 = w[3 * q + 2];
        sm[4 * q] = w0 & 0xFFFFFFu;
        sm[4 * q + 1] = (w0 >> 24) | ((w1 & 0xFFFFu) << 8);
        sm[4 * q + 2] = (w1 >> 16) | ((w2 & 0xFFu) << 16);
        sm[4 * q + 3] = w2 >> 8;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        sm[j] = (j < cnt) ? ((uint32_t)p[3 * j] | ((uint32_t)p[3 * j + 1] << 8) |
                             ((uint32_t)p[3 * j + 2] << 16))
                          : 0u;
    }
  }
}

__device__ __forceinline__ uint32_t load_u32_le(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

// Item i with tb[i] <= tile < tb[i+1]; tb strictly ascending from 0.  Called by
// all 64 lanes of one wave; the result is wave-uniform.
__device__ uint32_t find_item(const uint32_t* tb, uint32_t count, uint32_t tile) {
  uint32_t lo = 0, hi = count;
  const uint32_t lane = lane_id();
  while (hi - lo > 1) {
    const uint32_t step = (hi - lo + 63u) / 64u;
    const uint32_t p = lo + lane * step;
    const bool pred = (p < hi) && (tb[p] <= tile);
    const uint64_t m = __ballot(pred);
    const uint32_t last = 63u - (uint32_t)__clzll(m);
    const uint32_t nlo = lo + last * step;
    hi = min(hi, nlo + step);
    lo = nlo;
  }
  return lo;
}

// ------------------------------------------------------- decoupled look-back
// One 64-bit word per tile: [63:62] flag, [61:32] epoch, [31:0] count.
// The epoch (per call) makes words of earlier calls read as "not ready", so the
// status array needs no clearing between calls.
constexpr uint64_t kFlagAgg = 1, kFlagIncl = 2;

__device__ __forceinline__ uint64_t pack_status(uint64_t flag, uint32_t epoch, uint32_t v) {
  return (flag << 62) | ((uint64_t)(epoch & 0x3FFFFFFFu) << 32) | v;
}
__device__ __forceinline__ void publish(uint64_t* w, uint64_t val) {
  __hip_atomic_store(w, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t peek(uint64_t* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix of this tile's count within its item.  Wave-wide call.
// Every predecessor read has a lower dynamic tile id, i.e. its workgroup is
// already running, so every wait ends.
__device__ uint32_t look_back(uint64_t* status, uint32_t tile, uint32_t first_tile,
                              uint32_t epoch) {
  const uint32_t lane = lane_id();
  uint32_t excl = 0;
  int64_t hi = (int64_t)tile - 1;
  while (true) {
    const int64_t j = hi - (int64_t)lane;
    const bool valid = j >= (int64_t)first_tile;
    uint64_t w;
    while (true) {
      w = valid ? peek(status + j) : pack_status(kFlagIncl, epoch, 0u);
      const bool ready = ((w >> 62) != 0) && (((uint32_t)(w >> 32) & 0x3FFFFFFFu) == (epoch & 0x3FFFFFFFu));
      if (__all(ready)) break;
      __builtin_amdgcn_s_sleep(1);
    }
    const uint64_t incl = __ballot((w >> 62) == kFlagIncl);
    uint32_t mine = (uint32_t)w;
    if (incl) {
      const uint32_t stop = (uint32_t)__ffsll((unsigned long long)incl) - 1u;  // nearest inclusive
      if (lane > stop) mine = 0;
    }
    // wave sum
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mine += __shfl_xor(mine, o);
    excl += mine;
    if (incl) break;
    hi -= 64;
  }
  return excl;
}

// --------------------------------------------------------------------- encode

template <int DT, int S>
__global__ __launch_bounds__(kThreads) void encode_kernel(const EncItem* __restrict__ items,
                                                          const uint32_t* __restrict__ tile_begin,
                                                          uint32_t count, uint32_t total_tiles,
                                                          EncCtl* ctl, uint32_t* raw_list,
                                                          uint64_t* status, uint32_t epoch) {
  constexpr int E = Tr<DT>::E, K = Tr<DT>::K;
  constexpr uint32_t T = (uint32_t)kSub * S;
  __shared__ uint32_t s_tile, s_item, s_excl;
  __shared__ uint32_t s_wtot[4 * S];
  __shared__ uint32_t s_bm[2];

  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  if (tid == 0) s_tile = atomicAdd(&ctl->tile_counter, 1u);
  if (tid < 2) s_bm[tid] = 0;
  __syncthreads();
  const uint32_t tile = s_tile;
  if (tile >= total_tiles) return;  // uniform
  if (wave == 0) {
    const uint32_t it = find_item(tile_begin, count, tile);
    if (lane == 0) s_item = it;
  }
  __syncthreads();
  const uint32_t item = s_item;
  const EncItem d = items[item];
  const uint32_t t_local = tile - d.tile_begin;
  const uint64_t base = (uint64_t)t_local * T;
  const uint64_t n = d.n;
  const uint32_t B = d.block_size;
  const bool compress = d.compress != 0;
  const bool caligned = d.cache_aligned != 0;

  uint32_t mask[S];
  uint32_t expk[S][4];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
    const int cnt = c0 < n ? (int)min<uint64_t>(16, n - c0) : 0;
    uint32_t v[16], c[4];
    mask[s] = 0;
    expk[s][0] = expk[s][1] = expk[s][2] = expk[s][3] = 0;
    if (cnt > 0) {
      load16<DT>(d.x + c0 * E, cnt, v);
      load_bytes16(d.cache + c0, cnt, caligned, c);
      uint32_t sm[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t e = exp_of<DT>(v[j]);
        expk[s][j >> 2] |= e << (8 * (j & 3));
        if (j < cnt && e != byte_of(c, j)) mask[s] |= 1u << j;
        sm[j] = sm_of<DT>(v[j]);
      }
      if (compress) {
        store_sm16<DT>(d.stream + kHeader + c0 * K, cnt, sm);
      } else {
        store16<DT>(d.stream + kHeader + c0 * E, cnt, v);
      }
      if (mask[s]) {
        const uint32_t rel = (uint32_t)(((uint64_t)s * kSub + (uint64_t)tid * kEPT) / B);
        atomicOr(&s_bm[rel >> 5], 1u << (rel & 31u));
      }
    }
  }

  // block-wide exclusive scan of the per-thread change counts, sub-tile major
  uint32_t lpre[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint32_t c = (uint32_t)__popc(mask[s]);
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {
      const uint64_t m = __ballot((c >> b) & 1u);
      pre += lanes_below(m) << b;
      tot += (uint32_t)__popcll(m) << b;
    }
    lpre[s] = pre;
    if (lane == 0) s_wtot[s * 4 + wave] = tot;
  }
  __syncthreads();
  uint32_t agg = 0;
  uint32_t before[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t t = s_wtot[s * 4 + w];
      if (w == (int)wave) before[s] = agg;
      agg += t;
    }
  }

  // global offset of this tile's first patch
  if (wave == 0) {
    uint32_t excl = 0;
    if (t_local == 0) {
      if (lane == 0) publish(status + tile, pack_status(kFlagIncl, epoch, agg));
    } else {
      if (lane == 0) publish(status + tile, pack_status(kFlagAgg, epoch, agg));
      excl = look_back(status, tile, d.tile_begin, epoch);
      if (lane == 0) publish(status + tile, pack_status(kFlagIncl, epoch, excl + agg));
    }
    if (lane == 0) s_excl = excl;
  }
  __syncthreads();
  const uint32_t excl = s_excl;

  const uint64_t nb = (n + B - 1) / B;
  const uint64_t nbm = (nb + 7) / 8;
  if (compress) {
    // bitmap bytes of this tile's blocks (the tile spans a whole number of bytes)
    const uint64_t in_tile = min<uint64_t>(T, n > base ? n - base : 0);
    const uint32_t tblocks = (uint32_t)((in_tile + B - 1) / B);
    const uint32_t tbytes = (tblocks + 7) / 8;
    if (tid < tbytes) {
      const uint32_t word = s_bm[tid >> 2];
      d.stream[kHeader + n * K + base / ((uint64_t)B * 8) + tid] = (uint8_t)(word >> (8 * (tid & 3)));
    }
    // (index, exponent) records
    const uint64_t pbase = kHeader + n * K + nbm;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      uint32_t m = mask[s];
      uint64_t g = (uint64_t)excl + before[s] + lpre[s];
      const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
      while (m) {
        const int j = __ffs(m) - 1;
        m &= m - 1;
        const uint64_t pos = pbase + 5 * g;
        if (pos + 5 <= d.capacity) {
          const uint32_t idx = (uint32_t)(c0 + j);
          uint8_t* q = d.stream + pos;
          q[0] = (uint8_t)idx; q[1] = (uint8_t)(idx >> 8);
          q[2] = (uint8_t)(idx >> 16); q[3] = (uint8_t)(idx >> 24);
          q[4] = (uint8_t)byte_of(expk[s], j);
        }
        ++g;
      }
    }
  }

  // the item's last tile knows the total and writes the header
  if (t_local == d.ntiles - 1 && tid == 0) {
    const uint64_t P = (uint64_t)excl + agg;
    const uint64_t comp = kHeader + n * K + (P ? nbm + 5 * P : 0);
    const uint64_t raw = kHeader + n * E;
    const bool cmode = compress && comp < raw;
    if (compress && !cmode) {
      const uint32_t k = atomicAdd(&ctl->raw_count, 1u);
      raw_list[k] = item;
    }
    uint32_t h[16];
    h[0] = 0x52454943u;                               // "CIER"
    h[1] = 1u | ((uint32_t)DT << 16) | ((cmode ? 1u : 0u) << 24);
    h[2] = B;
    h[3] = 0;
    h[4] = (uint32_t)n; h[5] = (uint32_t)(n >> 32);
    h[6] = (uint32_t)P; h[7] = (uint32_t)(P >> 32);
    const uint64_t tot = cmode ? comp : raw;
    h[8] = (uint32_t)tot; h[9] = (uint32_t)(tot >> 32);
    h[10] = (uint32_t)d.off; h[11] = (uint32_t)(d.off >> 32);
    h[12] = d.rank; h[13] = d.world; h[14] = 0; h[15] = 0;
    uint4* hp = reinterpret_cast<uint4*>(d.stream);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 o;
      o.x = h[4 * q]; o.y = h[4 * q + 1]; o.z = h[4 * q + 2]; o.w = h[4 * q + 3];
      hp[q] = o;
    }
  }
}

// Rewrites as RAW the streams whose COMPRESSED form turned out not shorter.
template <int DT>
__global__ __launch_bounds__(kThreads) void encode_fixup_kernel(const EncItem* __restrict__ items,
                                                                const EncCtl* ctl,
                                                                const uint32_t* raw_list) {
  constexpr int E = Tr<DT>::E;
  const uint32_t cnt = ctl->raw_count;
  if (cnt == 0) return;
  const uint64_t gtid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t gsz = (uint64_t)gridDim.x * blockDim.x;
  for (uint32_t k = 0; k < cnt; ++k) {
    const EncItem d = items[raw_list[k]];
    const uint64_t bytes = d.n * E;
    const uint64_t vec = bytes / 16;
    const uint4* src = reinterpret_cast<const uint4*>(d.x);
    uint4* dst = reinterpret_cast<uint4*>(d.stream + kHeader);
    for (uint64_t i = gtid; i < vec; i += gsz) dst[i] = src[i];
    for (uint64_t i = vec * 16 + gtid; i < bytes; i += gsz) d.stream[kHeader + i] = d.x[i];
  }
}

// --------------------------------------------------------------------- decode

template <int DT>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecItem* __restrict__ items,
                                                          const uint32_t* __restrict__ tile_begin,
                                                          uint32_t count, uint32_t* status_out) {
  constexpr int E = Tr<DT>::E, K = Tr<DT>::K;
  constexpr uint32_t T = kDecTile;
  __shared__ uint32_t s_item;
  __shared__ uint32_t s_hdr[16];
  __shared__ uint32_t s_lohi[2];
  __shared__ uint32_t s_expbm[2];
  __shared__ uint32_t s_err;
  __shared__ __align__(16) uint8_t s_ov[T];

  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint32_t tile = blockIdx.x;
  if (wave == 0) {
    const uint32_t it = find_item(tile_begin, count, tile);
    if (lane == 0) s_item = it;
  }
  if (tid < 2) s_expbm[tid] = 0;
  if (tid == 0) s_err = 0;
  __syncthreads();
  const DecItem d = items[s_item];
  const uint32_t rel = tile - d.tile_begin;
  const uint32_t r = rel / d.tiles_per_rank;
  const uint32_t t_in = rel - r * d.tiles_per_rank;
  const uint64_t W = d.world;
  const uint64_t q = d.rows / W, rem = d.rows % W;
  const uint64_t my_rows = q + (r < rem ? 1 : 0);
  const uint64_t off = ((uint64_t)r * q + min<uint64_t>(r, rem)) * d.cols;
  const uint64_t n = my_rows * d.cols;
  const uint64_t ts = (uint64_t)t_in * T;
  if (ts >= n && t_in != 0) return;  // past this shard (uniform)
  const uint64_t te = min<uint64_t>(n, ts + T);
  const uint8_t* st = d.streams + (uint64_t)r * d.slot;
  const uint32_t B = d.block_size;

  if (tid < 4) {
    const uint4 h = reinterpret_cast<const uint4*>(st)[tid];
    s_hdr[4 * tid] = h.x; s_hdr[4 * tid + 1] = h.y; s_hdr[4 * tid + 2] = h.z; s_hdr[4 * tid + 3] = h.w;
  }
  __syncthreads();
  // header and length validation (uniform)
  const uint32_t h_dtype = (s_hdr[1] >> 16) & 0xFFu, h_mode = s_hdr[1] >> 24;
  const uint64_t h_n = s_hdr[4] | ((uint64_t)s_hdr[5] << 32);
  const uint64_t P = s_hdr[6] | ((uint64_t)s_hdr[7] << 32);
  const uint64_t h_tot = s_hdr[8] | ((uint64_t)s_hdr[9] << 32);
  const uint64_t h_off = s_hdr[10] | ((uint64_t)s_hdr[11] << 32);
  const uint64_t nb = (n + B - 1) / B;
  const uint64_t nbm = (nb + 7) / 8;
  uint32_t bad = 0;
  if (s_hdr[0] != 0x52454943u || (s_hdr[1] & 0xFFFFu) != 1u) {
    bad = CIERA_ST_MAGIC;
  } else if (h_dtype != (uint32_t)DT || s_hdr[2] != B || h_n != n || h_off != off ||
             s_hdr[12] != r || s_hdr[13] != d.world || h_mode > 1u) {
    bad = CIERA_ST_FIELD;
  } else {
    const uint64_t want = h_mode == 0 ? kHeader + n * E
                                      : kHeader + n * K + (P ? nbm + 5 * P : 0);
    if (P > n || h_tot > d.slot || h_tot != want) bad = CIERA_ST_LENGTH;
  }
  if (bad) {
    if (t_in == 0 && tid == 0) atomicOr(status_out, bad);
    return;  // uniform
  }
  const bool aligned = (off & 15u) == 0;
  const uint64_t c0 = ts + (uint64_t)tid * kEPT;
  const int cnt = c0 < te ? (int)min<uint64_t>(16, te - c0) : 0;
  uint8_t* out = d.out + (off + c0) * E;
  uint8_t* cache = d.cache + off + c0;

  if (h_mode == 0) {  // RAW: copy and refresh the cache
    if (cnt > 0) {
      uint32_t v[16], ex[4] = {0, 0, 0, 0};
      load16<DT>(st + kHeader + c0 * E, cnt, v);
#pragma unroll
      for (int j = 0; j < 16; ++j) ex[j >> 2] |= exp_of<DT>(v[j]) << (8 * (j & 3));
      store16<DT>(out, cnt, v, aligned);
      store_bytes16(cache, cnt, aligned, ex);
    }
    return;
  }

  // COMPRESSED.  Patch range [lo, hi) of this tile, by a 64-ary search.
  const uint8_t* recs = st + kHeader + n * K + nbm;
  uint32_t lo = 0, hi = 0;
  if (P > 0) {
    if (wave == 0) {
      uint32_t bounds[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint64_t key = b == 0 ? ts : te;
        // first position p in [0, P] with idx[p] >= key (predicate idx < key assumed monotone)
        uint64_t a = 0, z = P;  // answer in [a, z]
        while (z > a) {
          const uint64_t span = z - a;
          const uint64_t step = (span + 63) / 64;
          const uint64_t p = a + (uint64_t)lane * step;
          const bool less = (p < z) && (load_u32_le(recs + 5 * p) < key);
          const uint64_t m = __ballot(less);
          if (m == 0) {
            z = a;
          } else {
            const uint32_t last = 63u - (uint32_t)__clzll(m);
            a = a + (uint64_t)last * step + 1;
            z = min<uint64_t>(z, a - 1 + step);
          }
        }
        bounds[b] = (uint32_t)a;
      }
      if (lane == 0) {
        uint32_t e = 0;
        uint32_t l = bounds[0], h = bounds[1];
        if (h < l) { e |= CIERA_ST_PATCH; h = l; }
        if (te == n && h != P) e |= CIERA_ST_PATCH;
        s_lohi[0] = l; s_lohi[1] = h;
        if (e) s_err = e;
      }
    }
    __syncthreads();
    lo = s_lohi[0];
    hi = s_lohi[1];
  }

  uint32_t sm[16], c[4];
  if (cnt > 0) {
    load_sm16<DT>(st + kHeader + c0 * K, cnt, sm);
    load_bytes16(cache, cnt, aligned, c);
  }
  uint32_t ex[4] = {c[0], c[1], c[2], c[3]};
  const bool patched = hi > lo;   // uniform
  if (patched) {
    if (cnt > 0) {
      reinterpret_cast<uint4*>(s_ov)[tid] = make_uint4(c[0], c[1], c[2], c[3]);
    }
    __syncthreads();
    const uint64_t b0 = ts / B;
    for (uint32_t p = lo + tid; p < hi; p += kThreads) {
      const uint32_t idx = load_u32_le(recs + 5 * (uint64_t)p);
      const uint8_t v = recs[5 * (uint64_t)p + 4];
      uint32_t e = 0;
      if (p > 0 && load_u32_le(recs + 5 * (uint64_t)(p - 1)) >= idx) e |= CIERA_ST_PATCH;
      if (idx < ts || idx >= te) {
        e |= CIERA_ST_PATCH;
      } else {
        s_ov[idx - ts] = v;
        const uint32_t bb = (uint32_t)(idx / B - b0);
        atomicOr(&s_expbm[bb >> 5], 1u << (bb & 31u));
      }
      if (e) atomicOr(&s_err, e);
    }
    __syncthreads();
    if (cnt > 0) {
      const uint4 o = reinterpret_cast<const uint4*>(s_ov)[tid];
      ex[0] = o.x; ex[1] = o.y; ex[2] = o.z; ex[3] = o.w;
    }
  }

  // bitmap check: this tile's bits must mark exactly the blocks holding patches
  if (P > 0 && tid == 0) {
    const uint8_t* bm = st + kHeader + n * K;
    const uint64_t b0 = ts / B;
    const uint64_t b1 = (te + B - 1) / B;
    const uint32_t nbt = (uint32_t)(b1 - b0);
    uint64_t got = 0;
    for (uint64_t by = b0 / 8; by <= (b1 - 1) / 8; ++by) got |= (uint64_t)bm[by] << (8 * (by - b0 / 8));
    got >>= (b0 & 7u);
    if (nbt < 64) got &= ((uint64_t)1 << nbt) - 1;
    const uint64_t want = (uint64_t)s_expbm[0] | ((uint64_t)s_expbm[1] << 32);
    uint32_t e = got != want ? CIERA_ST_BITMAP : 0u;
    if (te == n && (nb & 7u) != 0 && (bm[nbm - 1] >> (nb & 7u)) != 0) e |= CIERA_ST_BITMAP;
    if (e) atomicOr(&s_err, e);
  }

  if (cnt > 0) {
    uint32_t v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = join<DT>(sm[j], byte_of(ex, j));
    store16<DT>(out, cnt, v, aligned);
    if (patched && (ex[0] != c[0] || ex[1] != c[1] || ex[2] != c[2] || ex[3] != c[3]))
      store_bytes16(cache, cnt, aligned, ex);
  }
  if (P > 0) {
    __syncthreads();
    if (tid == 0 && s_err) atomicOr(status_out, s_err);
  }
}

// -------------------------------------------------------------- cache update

template <int DT>
__global__ __launch_bounds__(kThreads) void cache_update_kernel(const uint8_t* __restrict__ w,
                                                                uint8_t* __restrict__ cache,
                                                                uint64_t n) {
  constexpr int E = Tr<DT>::E;
  const bool aligned = (reinterpret_cast<uintptr_t>(cache) & 15u) == 0;
  const uint64_t chunks = (n + 15) / 16;
  for (uint64_t ch = (uint64_t)blockIdx.x * kThreads + threadIdx.x; ch < chunks;
       ch += (uint64_t)gridDim.x * kThreads) {
    const uint64_t c0 = ch * 16;
    const int cnt = (int)min<uint64_t>(16, n - c0);
    uint32_t v[16], ex[4] = {0, 0, 0, 0};
    load16<DT>(w + c0 * E, cnt, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) ex[j >> 2] |= exp_of<DT>(v[j]) << (8 * (j & 3));
    store_bytes16(cache + c0, cnt, aligned, ex);
  }
}

}  // namespace

// ------------------------------------------------------------------- launchers

hipError_t launch_encode(int dtype, int sub, const EncItem* items, const uint32_t* tile_begin,
                         uint32_t count, uint32_t total_tiles, EncCtl* ctl, uint32_t* raw_list,
                         uint64_t* status, uint32_t epoch, hipStream_t s) {
  const dim3 grid(total_tiles), block(kThreads);
#define CIERA_ENC(DT, S) \
  hipLaunchKernelGGL((encode_kernel<DT, S>), grid, block, 0, s, items, tile_begin, count, total_tiles, ctl, raw_list, status, epoch)
  if (dtype == 1) {
    switch (sub) {
      case 1: CIERA_ENC(1, 1); break;
      case 2: CIERA_ENC(1, 2); break;
      case 4: CIERA_ENC(1, 4); break;
      case 8: CIERA_ENC(1, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (sub) {
      case 1: CIERA_ENC(2, 1); break;
      case 2: CIERA_ENC(2, 2); break;
      case 4: CIERA_ENC(2, 4); break;
      case 8: CIERA_ENC(2, 8); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef CIERA_ENC
  return hipGetLastError();
}

hipError_t launch_encode_fixup(int dtype, const EncItem* items, const EncCtl* ctl,
                               const uint32_t* raw_list, hipStream_t s) {
  const dim3 grid(1024), block(kThreads);
  if (dtype == 1) hipLaunchKernelGGL((encode_fixup_kernel<1>), grid, block, 0, s, items, ctl, raw_list);
  else hipLaunchKernelGGL((encode_fixup_kernel<2>), grid, block, 0, s, items, ctl, raw_list);
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, const DecItem* items, const uint32_t* tile_begin,
                         uint32_t count, uint32_t total_tiles, uint32_t* status, hipStream_t s) {
  const dim3 grid(total_tiles), block(kThreads);
  if (dtype == 1) hipLaunchKernelGGL((decode_kernel<1>), grid, block, 0, s, items, tile_begin, count, status);
  else hipLaunchKernelGGL((decode_kernel<2>), grid, block, 0, s, items, tile_begin, count, status);
  return hipGetLastError();
}

hipError_t launch_cache_update(int dtype, const uint8_t* w, uint8_t* cache, uint64_t n,
                               hipStream_t s) {
  const uint64_t chunks = (n + 15) / 16;
  uint64_t blocks = (chunks + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((uint32_t)blocks), block(kThreads);
  if (dtype == 1) hipLaunchKernelGGL((cache_update_kernel<1>), grid, block, 0, s, w, cache, n);
  else hipLaunchKernelGGL((cache_update_kernel<2>), grid, block, 0, s, w, cache, n);
  return hipGetLastError();
}

}  // namespace ciera
