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

#include <algorithm>
#include <type_traits>

#include "ciera.h"
#include "ciera_internal.h"

namespace ciera {
namespace {

// Every device buffer is reached through these casts to the global address
// space: pointers read from descriptor tables would otherwise compile to flat
// instructions, which also count against the LDS wait counter and so make every
// LDS access and barrier wait for all outstanding HBM loads.
#define G1 __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ G1 T* gp(T* p) { return (G1 T*)p; }
template <class T>
__device__ __forceinline__ const G1 T* gp(const T* p) { return (const G1 T*)p; }

typedef uint32_t v4u __attribute__((ext_vector_type(4)));  // one 16-byte global access
__device__ __forceinline__ v4u ldg16(const void* p) { return *gp(reinterpret_cast<const v4u*>(p)); }
__device__ __forceinline__ void stg16(void* p, v4u v) { *gp(reinterpret_cast<v4u*>(p)) = v; }
// Non-temporal 16-byte store: for data no later access of this launch reads.
__device__ __forceinline__ void stg16_nt(void* p, v4u v) {
  __builtin_nontemporal_store(v, gp(reinterpret_cast<v4u*>(p)));
}

template <int DT>
struct Tr;
// E: bytes per value; SHIFT: mantissa bits; EMASK: exponent field; SMBITS:
// sign|mantissa bits per value in the stream (bf16 and fp32 whole bytes, fp16
// an 11-bit LSB-first bit stream: 16 values = 22 bytes).
template <>
struct Tr<1> {  // bf16: 1 sign, 8 exponent, 7 mantissa bits
  static constexpr int E = 2, SHIFT = 7, SMBITS = 8;
  static constexpr uint32_t EMASK = 0xFF;
};
template <>
struct Tr<2> {  // fp32: 1 sign, 8 exponent, 23 mantissa bits
  static constexpr int E = 4, SHIFT = 23, SMBITS = 24;
  static constexpr uint32_t EMASK = 0xFF;
};
template <>
struct Tr<3> {  // fp16: 1 sign, 5 exponent, 10 mantissa bits
  static constexpr int E = 2, SHIFT = 10, SMBITS = 11;
  static constexpr uint32_t EMASK = 0x1F;
};

// Bytes of the sign|mantissa section of n values, and the byte offset of value
// c0 in it (c0 a multiple of 16, so the offset is whole).
template <int DT>
__device__ __forceinline__ uint64_t sm_sec(uint64_t n) {
  return (n * Tr<DT>::SMBITS + 7) / 8;
}
template <int DT>
__device__ __forceinline__ uint64_t sm_off(uint64_t c0) {
  return c0 * Tr<DT>::SMBITS / 8;
}

template <int DT>
__device__ __forceinline__ uint32_t exp_of(uint32_t v) {
  return (v >> Tr<DT>::SHIFT) & Tr<DT>::EMASK;
}
// sign|mantissa: sign << SHIFT | mantissa (bf16 8 bits, fp32 24, fp16 11)
template <int DT>
__device__ __forceinline__ uint32_t sm_of(uint32_t v) {
  constexpr int S = Tr<DT>::SHIFT, SB = 8 * Tr<DT>::E - 1;
  return ((v >> SB) << S) | (v & ((1u << S) - 1u));
}
template <int DT>
__device__ __forceinline__ uint32_t join(uint32_t sm, uint32_t ex) {
  constexpr int S = Tr<DT>::SHIFT, SB = 8 * Tr<DT>::E - 1;
  return ((sm >> S) << SB) | (ex << S) | (sm & ((1u << S) - 1u));
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
    if constexpr (Tr<DT>::E == 2) {
      const v4u a = ldg16(p);
      const v4u b = ldg16(p + 16);
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[2 * j] = w[j] & 0xFFFFu;
        v[2 * j + 1] = w[j] >> 16;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4u a = ldg16(p + 16 * q);
        v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < cnt) {
        if constexpr (Tr<DT>::E == 2) v[j] = gp(reinterpret_cast<const uint16_t*>(p))[j];
        else v[j] = gp(reinterpret_cast<const uint32_t*>(p))[j];
      } else {
        v[j] = 0;
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ void store16(uint8_t* p, int cnt, const uint32_t v[16], bool vec = true) {
  if (cnt == 16 && vec) {
    if constexpr (Tr<DT>::E == 2) {
      v4u a, b;
      a.x = v[0] | (v[1] << 16); a.y = v[2] | (v[3] << 16);
      a.z = v[4] | (v[5] << 16); a.w = v[6] | (v[7] << 16);
      b.x = v[8] | (v[9] << 16); b.y = v[10] | (v[11] << 16);
      b.z = v[12] | (v[13] << 16); b.w = v[14] | (v[15] << 16);
      stg16(p, a);
      stg16(p + 16, b);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v4u a;
        a.x = v[4 * q]; a.y = v[4 * q + 1]; a.z = v[4 * q + 2]; a.w = v[4 * q + 3];
        stg16(p + 16 * q, a);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < cnt) {
        if constexpr (Tr<DT>::E == 2) gp(reinterpret_cast<uint16_t*>(p))[j] = (uint16_t)v[j];
        else gp(reinterpret_cast<uint32_t*>(p))[j] = v[j];
      }
    }
  }
}

// 16 bytes (cache exponents) as four little-endian words.
__device__ __forceinline__ void load_bytes16(const uint8_t* p, int cnt, bool aligned, uint32_t c[4]) {
  if (cnt == 16 && aligned) {
    const v4u a = ldg16(p);
    c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w;
  } else {
    c[0] = c[1] = c[2] = c[3] = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < cnt) c[j >> 2] |= (uint32_t)gp(p)[j] << (8 * (j & 3));
  }
}

__device__ __forceinline__ void store_bytes16(uint8_t* p, int cnt, bool aligned, const uint32_t c[4]) {
  if (cnt == 16 && aligned) {
    v4u a;
    a.x = c[0]; a.y = c[1]; a.z = c[2]; a.w = c[3];
    stg16(p, a);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < cnt) gp(p)[j] = (uint8_t)(c[j >> 2] >> (8 * (j & 3)));
  }
}

__device__ __forceinline__ uint32_t byte_of(const uint32_t c[4], int j) {
  return (c[j >> 2] >> (8 * (j & 3))) & 0xFFu;
}

// fp16: the 11-bit values of 16 elements as an LSB-first bit stream, in 6
// words (176 bits; the top half of the last word is zero).
__device__ __forceinline__ void pack11x16(const uint32_t sm[16], uint32_t o[6]) {
#pragma unroll
  for (int i = 0; i < 6; ++i) o[i] = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int b = 11 * j, w = b >> 5, r = b & 31;
    o[w] |= sm[j] << r;
    if (r > 21) o[w + 1] |= sm[j] >> (32 - r);
  }
}

// sign|mantissa records of 16 values at p: bf16 16 bytes, fp32 48 bytes (3 per
// value, LE), fp16 22 bytes (p even: the chunk starts at byte 22k of the section).
template <int DT>
__device__ __forceinline__ void store_sm16(uint8_t* p, int cnt, const uint32_t sm[16]) {
  if constexpr (DT == 3) {
    uint32_t o[6];
    pack11x16(sm, o);
    if (cnt == 16) {
      if ((reinterpret_cast<uintptr_t>(p) & 3u) == 0) {
#pragma unroll
        for (int i = 0; i < 5; ++i) gp(reinterpret_cast<uint32_t*>(p))[i] = o[i];
        gp(reinterpret_cast<uint16_t*>(p + 20))[0] = (uint16_t)o[5];
      } else {  // p = 4q + 2
        gp(reinterpret_cast<uint16_t*>(p))[0] = (uint16_t)o[0];
#pragma unroll
        for (int i = 0; i < 5; ++i)
          gp(reinterpret_cast<uint32_t*>(p + 2))[i] = (o[i] >> 16) | (o[i + 1] << 16);
      }
    } else {
      const int nb = (11 * cnt + 7) / 8;
#pragma unroll
      for (int b = 0; b < 22; ++b)
        if (b < nb) gp(p)[b] = (uint8_t)(o[b >> 2] >> (8 * (b & 3)));
    }
  } else if constexpr (DT == 1) {
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
        v4u o;
        o.x = w[4 * q]; o.y = w[4 * q + 1]; o.z = w[4 * q + 2]; o.w = w[4 * q + 3];
        stg16(p + 16 * q, o);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j < cnt) {
          gp(p)[3 * j] = (uint8_t)sm[j];
          gp(p)[3 * j + 1] = (uint8_t)(sm[j] >> 8);
          gp(p)[3 * j + 2] = (uint8_t)(sm[j] >> 16);
        }
      }
    }
  }
}

// Raw 32-bit words of nbytes <= 4*NW bytes at p (vector loads when complete and allowed).
template <int NW>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t nbytes, bool vec, uint32_t w[NW]) {
  if (vec && nbytes == NW * 4) {
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      const v4u a = ldg16(p + 16 * q);
      w[4 * q] = a.x; w[4 * q + 1] = a.y; w[4 * q + 2] = a.z; w[4 * q + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = 0;
#pragma unroll
    for (int b = 0; b < NW * 4; ++b)
      if ((uint32_t)b < nbytes) w[b >> 2] |= (uint32_t)gp(p)[b] << (8 * (b & 3));
  }
}

// Stores the first nbytes <= 4*NW bytes of the words w at p (vector stores,
// non-temporal if NT, when complete and allowed).
template <int NW, bool NT = false>
__device__ __forceinline__ void store_words(uint8_t* p, uint32_t nbytes, bool vec, const uint32_t w[NW]) {
  if (vec && nbytes == NW * 4) {
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      v4u a;
      a.x = w[4 * q]; a.y = w[4 * q + 1]; a.z = w[4 * q + 2]; a.w = w[4 * q + 3];
      if (NT) stg16_nt(p + 16 * q, a);
      else stg16(p + 16 * q, a);
    }
  } else {
#pragma unroll
    for (int b = 0; b < NW * 4; ++b)
      if ((uint32_t)b < nbytes) gp(p)[b] = (uint8_t)(w[b >> 2] >> (8 * (b & 3)));
  }
}

// bf16, four values at a time.  A pair of words w0 = (v1 << 16) | v0 and
// w1 = (v3 << 16) | v2 gives the four exponent bytes (bits 7..14 of each value
// are byte 1 of the value shifted left once) and the four sign|mantissa bytes
// (sign from each value's high byte, mantissa from its low byte) with byte
// permutes; the merge goes the other way.
__device__ __forceinline__ uint32_t bf16x4_exp(uint32_t w0, uint32_t w1) {
  return __builtin_amdgcn_perm(w1 << 1, w0 << 1, 0x07050301u);
}
__device__ __forceinline__ uint32_t bf16x4_sm(uint32_t w0, uint32_t w1) {
  const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x06040200u);
  const uint32_t hi = __builtin_amdgcn_perm(w1, w0, 0x07050301u);
  return (hi & 0x80808080u) | (lo & 0x7F7F7F7Fu);
}
__device__ __forceinline__ void bf16x4_join(uint32_t sm, uint32_t ex, uint32_t& w0, uint32_t& w1) {
  const uint32_t lo = (sm & 0x7F7F7F7Fu) | ((ex << 7) & 0x80808080u);  // low bytes of the values
  const uint32_t hi = (sm & 0x80808080u) | ((ex >> 1) & 0x7F7F7F7Fu);  // high bytes
  w0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  w1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}
// Bit j set iff byte j of the 4 words is nonzero (16 bits).
__device__ __forceinline__ uint32_t nonzero_bytes16(const uint32_t d[4]) {
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t t = (((d[q] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | d[q]) & 0x80808080u;  // bit 7 of each nonzero byte
    m |= ((t >> 7) | (t >> 14) | (t >> 21) | (t >> 28)) << (4 * q) & (0xFu << (4 * q));
  }
  return m;
}

// The sign|mantissa words of the 16-value chunk starting at value c0 of a
// section (c0 a multiple of 16).  fp16 chunks start on even bytes: a complete
// chunk is read as the 6 aligned words around it and shifted down by 16 bits
// when it starts mid-word (the words stay inside the slot, which holds a RAW
// stream of 2 bytes per value); a partial chunk is read byte by byte.
template <int DT, int SW>
__device__ __forceinline__ void load_smw(const uint8_t* sec, uint64_t c0, int cnt, uint32_t w[SW]) {
  const uint8_t* a = sec + sm_off<DT>(c0);
  if constexpr (DT == 3) {
    if (cnt == 16) {
      const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(a) & 3u);  // 0 or 2
      const G1 uint32_t* q = gp(reinterpret_cast<const uint32_t*>(a - sh));
#pragma unroll
      for (int i = 0; i < 6; ++i) w[i] = q[i];
      if (sh) {
#pragma unroll
        for (int i = 0; i < 5; ++i) w[i] = (w[i] >> 16) | (w[i + 1] << 16);
        w[5] >>= 16;
      }
    } else {
      load_words<SW>(a, (uint32_t)(11 * cnt + 7) / 8, false, w);
    }
  } else {
    load_words<SW>(a, (uint32_t)cnt * Tr<DT>::SMBITS / 8, true, w);
  }
}

// sign|mantissa of value j from the raw words of a 16-value chunk (fp16: the
// chunk's bit stream starting at bit 0 of w[0]).
template <int DT>
__device__ __forceinline__ uint32_t sm_from_words(const uint32_t* w, int j) {
  if constexpr (DT == 3) {
    const int b = 11 * j, q = b >> 5, r = b & 31;
    uint32_t v = w[q] >> r;
    if (r > 21) v |= w[q + 1] << (32 - r);
    return v & 0x7FFu;
  } else if constexpr (DT == 1) {
    return (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;
  } else {
    const int q = j >> 2, k = j & 3;
    const uint32_t w0 = w[3 * q], w1 = w[3 * q + 1], w2 = w[3 * q + 2];
    if (k == 0) return w0 & 0xFFFFFFu;
    if (k == 1) return (w0 >> 24) | ((w1 & 0xFFFFu) << 8);
    if (k == 2) return (w1 >> 16) | ((w2 & 0xFFu) << 16);
    return w2 >> 8;
  }
}

// The two aligned words that cover bits [start, start+32) of the bit array at
// p; the bits are taken out by bits_of() once the words are needed, so the
// load joins the round of loads around it.  The caller guarantees that the
// stream goes on for at least 5 bytes past the first needed byte (a patch
// record follows the bitmap), so both words start inside the stream.
struct Words2 { uint32_t w0, w1, sh; };
__device__ __forceinline__ Words2 load_bits_w(const uint8_t* p, uint64_t start) {
  const uintptr_t at = reinterpret_cast<uintptr_t>(p) + (start >> 3);
  const uint32_t o = (uint32_t)(at & 3u);
  const G1 uint32_t* w = gp(reinterpret_cast<const uint32_t*>(at - o));
  return Words2{w[0], w[1], 8u * o + (uint32_t)(start & 7u)};
}
__device__ __forceinline__ uint32_t bits_of(const Words2& r, uint32_t nbits) {
  const uint64_t v = ((uint64_t)r.w0 | ((uint64_t)r.w1 << 32)) >> r.sh;
  return nbits >= 32 ? (uint32_t)v : (uint32_t)(v & ((1u << nbits) - 1u));
}

// Patch record p (u32 index, u8 exponent, 5 bytes at recs + 5p) read as the two
// aligned words that cover it; both words start inside the stream, and the slot
// is a multiple of 16 bytes, so neither can leave it.
__device__ __forceinline__ Words2 load_rec(const uint8_t* st, uint64_t recs, uint64_t p) {
  const uint64_t o = recs + 5 * p;
  const uint64_t a = o & ~(uint64_t)3;
  const G1 uint32_t* w = gp(reinterpret_cast<const uint32_t*>(st + a));
  return Words2{w[0], w[1], (uint32_t)(o - a) * 8u};
}
__device__ __forceinline__ void rec_fields(const Words2& r, uint32_t& idx, uint32_t& ex) {
  const uint64_t v = ((uint64_t)r.w0 | ((uint64_t)r.w1 << 32)) >> r.sh;
  idx = (uint32_t)v;
  ex = (uint32_t)(v >> 32) & 0xFFu;
}
__device__ __forceinline__ void read_rec(const uint8_t* st, uint64_t recs, uint64_t p, uint32_t& idx,
                                         uint32_t& ex) {
  rec_fields(load_rec(st, recs, p), idx, ex);
}

// ORs decode status bits into the caller's word; a plain read first keeps a
// stream of identical errors (every tile of a corrupt batch) from serializing
// on one address.
__device__ __forceinline__ void report(uint32_t* status, uint32_t bits) {
  if ((__hip_atomic_load(gp(status), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & bits) != bits)
    __hip_atomic_fetch_or(gp(status), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------- decoupled look-back
// One 64-bit word per tile: [63:62] flag, [61:32] launch tag, [31:0] count.
// Words of earlier launches carry another tag and read as "not ready", so the
// array is never cleared.
constexpr uint64_t kFlagAgg = 1, kFlagIncl = 2;
constexpr uint32_t kSpinCap = 1u << 22;  // only reached if the scratch was tampered with

__device__ __forceinline__ uint64_t pack_status(uint64_t flag, uint32_t tag, uint32_t v) {
  return (flag << 62) | ((uint64_t)(tag & 0x3FFFFFFFu) << 32) | v;
}
__device__ __forceinline__ void publish(uint64_t* w, uint64_t val) {
  __hip_atomic_store(gp(w), val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t peek(uint64_t* w) {
  return __hip_atomic_load(gp(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix of tile `local`'s count among the tiles of its item
// (status words sw[0..local)).  Wave-wide.  Every tile read holds a smaller
// dynamic id of the same item, so its workgroup is already running and its
// word arrives; the spin cap only guards against a corrupted scratch.
__device__ uint32_t look_back(uint64_t* sw, uint32_t local, uint32_t tag, uint32_t* err) {
  const uint32_t lane = lane_id();
  uint32_t excl = 0;
  int64_t hi = (int64_t)local - 1;
  while (true) {
    const int64_t j = hi - (int64_t)lane;
    const bool valid = j >= 0;
    uint64_t w;
    uint32_t spins = 0;
    while (true) {
      w = valid ? peek(sw + j) : pack_status(kFlagIncl, tag, 0u);
      const bool ready = ((w >> 62) != 0) && (((uint32_t)(w >> 32) & 0x3FFFFFFFu) == (tag & 0x3FFFFFFFu));
      if (__all(ready)) break;
      if (++spins >= kSpinCap) {
        if (lane == 0) __hip_atomic_fetch_or(gp(err), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        w = ready ? w : pack_status(kFlagIncl, tag, 0u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const uint64_t incl = __ballot((w >> 62) == kFlagIncl);
    uint32_t mine = (uint32_t)w;
    if (incl) {
      const uint32_t stop = (uint32_t)__ffsll((unsigned long long)incl) - 1u;  // nearest inclusive
      if (lane > stop) mine = 0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mine += __shfl_xor(mine, o);
    excl += mine;
    if (incl) break;
    hi -= 64;
  }
  return excl;
}

// --------------------------------------------------------------------- encode
// One workgroup per tile of S*4096 values of one item; items of a group share a
// tile count, so the item is blockIdx / tpi and only the tile's place inside the
// item is taken dynamically (per-item counter), which keeps the look-back free
// of deadlock without a global hot counter.

template <int DT, int S>
__global__ __launch_bounds__(kThreads) void encode_kernel(EncArgs a, uint32_t* ctl, uint32_t batch_id) {
  constexpr int E = Tr<DT>::E;
  constexpr uint32_t T = (uint32_t)kSub * S;
  constexpr int XW = 4 * E;  // words of 16 raw values
  __shared__ uint32_t s_local, s_excl, s_tag;
  __shared__ uint32_t s_wtot[4 * S];
  __shared__ uint32_t s_bm[2 * S];  // one bit per block of the tile: T/B <= T/64 = 64*S bits

  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint32_t item = a.item0 + blockIdx.x / a.tpi;
  const EncItem d = a.items[item];
  if (d.batch_id != batch_id) return;  // the scratch holds another batch (uniform)
  if (tid == 0) {
    const uint32_t got = __hip_atomic_fetch_add(gp(a.ctr + item), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the item's last tile to take an id: every tile has taken one, so the
    // counter goes back to 0 for the next launch
    if (got == a.tpi - 1) __hip_atomic_store(gp(a.ctr + item), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_local = got;
    s_tag = *gp(ctl + kCtlEpoch);  // written before this launch, fixed during it
  }
  if (tid < 2 * S) s_bm[tid] = 0;
  __syncthreads();
  const uint32_t local = s_local, tag = s_tag;
  if (local >= a.tpi) return;  // uniform; cannot happen while counters match launches
  if (local == 0 && tid == 0) *gp(ctl + kCtlTag) = tag;  // for the fallback kernel
  const uint64_t base = (uint64_t)local * T;
  const uint64_t n = d.n;
  const uint32_t B = d.block_size;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;  // B is a power of two (checked by the API)
  const bool compress = d.compress != 0;
  const bool caligned = d.cache_aligned != 0;

  // Loads, split and compare, sign|mantissa (or RAW) stores, bitmap bits in
  // LDS.  A tile wholly inside its item with an aligned cache takes a
  // straight-line copy of this code (FULL: every chunk has 16 values).
  uint32_t mask[S];
  uint32_t expk[S][4];
  auto split_tile = [&](auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    uint32_t xw[S][XW], cw[S][4];
    int cnt[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {  // all loads of the tile first
      const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
      cnt[s] = FULL ? 16 : (c0 < n ? (int)min<uint64_t>(16, n - c0) : 0);
      if (cnt[s] > 0) {
        load_words<XW>(d.x + c0 * E, (uint32_t)cnt[s] * E, true, xw[s]);
        load_words<4>(d.cache + c0, (uint32_t)cnt[s], FULL || caligned, cw[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
      mask[s] = 0;
      expk[s][0] = expk[s][1] = expk[s][2] = expk[s][3] = 0;
      if (cnt[s] > 0) {
        if constexpr (DT == 1) {
          uint32_t smw[4], dif[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            expk[s][q] = bf16x4_exp(xw[s][2 * q], xw[s][2 * q + 1]);
            smw[q] = bf16x4_sm(xw[s][2 * q], xw[s][2 * q + 1]);
            dif[q] = expk[s][q] ^ cw[s][q];
            if (!FULL) {  // only the cnt values present
              const int nv = cnt[s] - 4 * q;
              dif[q] &= nv >= 4 ? 0xFFFFFFFFu : nv <= 0 ? 0u : (1u << (8 * nv)) - 1u;
            }
          }
          if (dif[0] | dif[1] | dif[2] | dif[3]) mask[s] = nonzero_bytes16(dif);
          if (compress) store_words<4>(d.stream + kHeader + c0, (uint32_t)cnt[s], true, smw);
          else store_words<XW>(d.stream + kHeader + c0 * E, (uint32_t)cnt[s] * E, true, xw[s]);
        } else {
          uint32_t v[16], sm[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            if constexpr (E == 2) v[j] = (xw[s][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            else v[j] = xw[s][j];
            const uint32_t e = exp_of<DT>(v[j]);
            expk[s][j >> 2] |= e << (8 * (j & 3));
            if (j < cnt[s] && e != byte_of(cw[s], j)) mask[s] |= 1u << j;
            sm[j] = sm_of<DT>(v[j]);
          }
          if (compress) store_sm16<DT>(d.stream + kHeader + sm_off<DT>(c0), cnt[s], sm);
          else store16<DT>(d.stream + kHeader + c0 * E, cnt[s], v);
        }
        if (mask[s]) {
          const uint32_t rel = ((uint32_t)s * kSub + tid * kEPT) >> lb;
          atomicOr(&s_bm[rel >> 5], 1u << (rel & 31u));
        }
      }
    }
  };
  if (caligned && base + T <= n) split_tile(std::true_type{});  // uniform
  else split_tile(std::false_type{});

  // block-wide exclusive scan of the per-thread change counts, chunk-row major
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

  uint64_t* sw = a.status + (uint64_t)(item - a.item0) * a.tpi;
  if (wave == 0) {
    uint32_t excl = 0;
    if (local == 0) {
      if (lane == 0) publish(sw, pack_status(kFlagIncl, tag, agg));
    } else {
      if (lane == 0) publish(sw + local, pack_status(kFlagAgg, tag, agg));
      excl = look_back(sw, local, tag, ctl + kCtlError);
      if (lane == 0) publish(sw + local, pack_status(kFlagIncl, tag, excl + agg));
    }
    if (lane == 0) s_excl = excl;
  }
  __syncthreads();
  const uint32_t excl = s_excl;

  const uint64_t nb = (n + B - 1) >> lb;
  const uint64_t nbm = (nb + 7) / 8;
  if (compress) {
    // bitmap bytes of this tile's blocks (a tile spans whole bitmap bytes)
    const uint64_t in_tile = min<uint64_t>(T, n > base ? n - base : 0);
    const uint32_t tblocks = (uint32_t)((in_tile + B - 1) >> lb);
    const uint32_t tbytes = (tblocks + 7) / 8;
    if (tid < tbytes)
      gp(d.stream)[kHeader + sm_sec<DT>(n) + (base >> (lb + 3)) + tid] = (uint8_t)(s_bm[tid >> 2] >> (8 * (tid & 3)));
    // (index, exponent) records
    const uint64_t pbase = kHeader + sm_sec<DT>(n) + nbm;
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
          G1 uint8_t* q = gp(d.stream + pos);
          q[0] = (uint8_t)idx; q[1] = (uint8_t)(idx >> 8);
          q[2] = (uint8_t)(idx >> 16); q[3] = (uint8_t)(idx >> 24);
          q[4] = (uint8_t)byte_of(expk[s], j);
        }
        ++g;
      }
    }
  }

  // the item's last tile knows the total and writes the header
  if (local == a.tpi - 1 && tid == 0) {
    const uint64_t P = (uint64_t)excl + agg;
    const uint64_t comp = kHeader + sm_sec<DT>(n) + (P ? nbm + 5 * P : 0);
    const uint64_t raw = kHeader + n * E;
    const bool cmode = compress && comp < raw;
    if (compress && !cmode) {
      gp(a.raw_flag)[item] = tag;
      *gp(a.any_raw) = tag;
    }
    uint32_t h[16];
    h[0] = 0x52454943u;  // "CIER"
    h[1] = 1u | ((uint32_t)DT << 16) | ((cmode ? 1u : 0u) << 24);
    h[2] = B;
    h[3] = 0;
    h[4] = (uint32_t)n; h[5] = (uint32_t)(n >> 32);
    h[6] = (uint32_t)P; h[7] = (uint32_t)(P >> 32);
    const uint64_t tot = cmode ? comp : raw;
    h[8] = (uint32_t)tot; h[9] = (uint32_t)(tot >> 32);
    h[10] = (uint32_t)d.off; h[11] = (uint32_t)(d.off >> 32);
    h[12] = d.rank; h[13] = d.world; h[14] = 0; h[15] = 0;

#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v4u o;
      o.x = h[4 * q]; o.y = h[4 * q + 1]; o.z = h[4 * q + 2]; o.w = h[4 * q + 3];
      stg16(d.stream + 16 * q, o);
    }
  }
}

// Rewrites as RAW the streams whose COMPRESSED form turned out not shorter:
// gridDim.x workgroups per item, items along y.  Returns at once when the
// launch flagged no item (the common case).  It runs after every encode launch
// and advances the epoch: the next launch's tag.
__global__ __launch_bounds__(kThreads) void encode_fixup_kernel(const EncItem* __restrict__ items, uint32_t count,
                                                                const uint32_t* raw_flag, uint32_t* ctl,
                                                                uint32_t batch_id) {
  const uint32_t tag = *gp(ctl + kCtlTag);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    *gp(ctl + kCtlEpoch) = 1u + tag % 0x3FFFFFFEu;  // never 0; no other block reads the epoch
  if (*gp(ctl + kCtlAnyRaw) != tag) return;
  const uint64_t gtid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t gsz = (uint64_t)gridDim.x * blockDim.x;
  for (uint32_t k = blockIdx.y; k < count; k += gridDim.y) {
    if (gp(raw_flag)[k] != tag) continue;
    const EncItem d = items[k];
    if (d.batch_id != batch_id) return;
    if (d.stream == nullptr) continue;
    const uint64_t bytes = d.n * d.elem_bytes;
    const uint64_t vec = bytes / 16;
    for (uint64_t i = gtid; i < vec; i += gsz) stg16(d.stream + kHeader + 16 * i, ldg16(d.x + 16 * i));
    for (uint64_t i = vec * 16 + gtid; i < bytes; i += gsz) gp(d.stream)[kHeader + i] = gp(d.x)[i];
  }
}

// --------------------------------------------------------------------- decode
// One workgroup per tile of U*4096 values of one rank's stream.  The bulk loads
// (sign|mantissa bytes and cached exponents) are issued before the header and
// the patch range are known, so their latency overlaps that chain.

template <int DT, int U>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const DecItem* __restrict__ items, uint32_t item0,
                                                          uint32_t tpr, uint32_t world, uint32_t* status_out,
                                                          const uint32_t* ctl, uint32_t batch_id) {
  constexpr int E = Tr<DT>::E;
  constexpr uint32_t T = (uint32_t)kDecRow * U;
  constexpr uint32_t BMW = (T / 64 + 31) / 32;  // words of per-tile block bits (B >= 64)
  constexpr int SW = (16 * Tr<DT>::SMBITS + 31) / 32;  // words of 16 sign|mantissa records
  __shared__ uint32_t s_hdr[16];
  __shared__ uint32_t s_expbm[BMW];  // blocks of the tile that hold a patch
  __shared__ uint32_t s_ex[T / 4];   // the tile's exponents: cached, then patched in place

  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint32_t tpi = tpr * world;
  const uint32_t blk = blockIdx.x / tpi;
  const uint32_t item = item0 + blk;
  const uint32_t rel = blockIdx.x - blk * tpi;
  const uint32_t r = rel / tpr;
  const uint32_t t_in = rel - r * tpr;
  const DecItem d = items[item];
  if (d.batch_id != batch_id) return;  // the scratch holds another batch (uniform)
  const uint64_t q = d.q, rem = d.rem;  // rows per rank, ranks with one more
  const uint64_t off = ((uint64_t)r * q + min<uint64_t>(r, rem)) * d.cols;
  const uint64_t n = (q + (r < rem ? 1u : 0u)) * d.cols;
  const uint64_t ts = (uint64_t)t_in * T;
  if (ts >= n && t_in != 0) return;  // past this shard (uniform)
  const uint64_t te = min<uint64_t>(n, ts + T);
  const uint8_t* st = d.streams + (uint64_t)r * d.slot;
  const uint32_t B = d.block_size;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;  // B is a power of two (checked by the API)
  const bool aligned = (off & 15u) == 0;
  uint8_t* const cache = d.cache + off;

  // 1. bulk loads, COMPRESSED layout (in bounds for either mode: a slot holds a RAW stream)
  uint32_t sw[U][SW], cw[U][4];
  int cnt[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t c0 = ts + (uint64_t)u * kDecRow + (uint64_t)tid * kEPT;
    cnt[u] = c0 < te ? (int)min<uint64_t>(16, te - c0) : 0;
    if (cnt[u] > 0) {
      load_smw<DT, SW>(st + kHeader, c0, cnt[u], sw[u]);
      load_words<4>(cache + c0, (uint32_t)cnt[u], aligned, cw[u]);
    }
  }
  const uint64_t nb = (n + B - 1) >> lb;
  const uint64_t nbm = (nb + 7) / 8;

  // 2. header
  if (tid < 4) {
    const v4u h = ldg16(st + 16 * tid);
    s_hdr[4 * tid] = h.x; s_hdr[4 * tid + 1] = h.y; s_hdr[4 * tid + 2] = h.z; s_hdr[4 * tid + 3] = h.w;
  }
  if (tid < BMW) s_expbm[tid] = 0;
  // the cached exponents go to LDS now: the header read above already waits
  // for the bulk loads (loads complete in order), and patches overwrite them
  // after the next barrier
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (cnt[u] > 0) {
      v4u e;
      e.x = cw[u][0]; e.y = cw[u][1]; e.z = cw[u][2]; e.w = cw[u][3];
      *reinterpret_cast<v4u*>(&s_ex[((uint32_t)u * kDecRow + tid * kEPT) / 4]) = e;
    }
  }
  __syncthreads();
  const uint32_t h_dtype = (s_hdr[1] >> 16) & 0xFFu, h_mode = s_hdr[1] >> 24;
  const uint64_t h_n = s_hdr[4] | ((uint64_t)s_hdr[5] << 32);
  const uint64_t P = s_hdr[6] | ((uint64_t)s_hdr[7] << 32);
  const uint64_t h_tot = s_hdr[8] | ((uint64_t)s_hdr[9] << 32);
  const uint64_t h_off = s_hdr[10] | ((uint64_t)s_hdr[11] << 32);
  uint32_t bad = 0;
  if (s_hdr[0] != 0x52454943u || (s_hdr[1] & 0xFFFFu) != 1u) {
    bad = CIERA_ST_MAGIC;
  } else if (h_dtype != (uint32_t)DT || s_hdr[2] != B || h_n != n || h_off != off || s_hdr[12] != r ||
             s_hdr[13] != world || h_mode > 1u) {
    bad = CIERA_ST_FIELD;
  } else {
    const uint64_t want = h_mode == 0 ? kHeader + n * E : kHeader + sm_sec<DT>(n) + (P ? nbm + 5 * P : 0);
    if (P > n || h_tot > d.slot || h_tot != want) bad = CIERA_ST_LENGTH;
  }
  if (bad) {
    if (t_in == 0 && tid == 0) report(status_out, bad);
    return;  // uniform
  }
  uint8_t* const out = d.out + off * E;

  if (h_mode == 0) {  // RAW: copy and refresh the cache
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (cnt[u] > 0) {
        const uint64_t c0 = ts + (uint64_t)u * kDecRow + (uint64_t)tid * kEPT;
        uint32_t v[16], ex[4] = {0, 0, 0, 0};
        load16<DT>(st + kHeader + c0 * E, cnt[u], v);
#pragma unroll
        for (int j = 0; j < 16; ++j) ex[j >> 2] |= exp_of<DT>(v[j]) << (8 * (j & 3));
        store16<DT>(out + c0 * E, cnt[u], v, aligned);
        store_bytes16(cache + c0, cnt[u], aligned, ex);
      }
    }
    return;
  }

  // 3. COMPRESSED: this tile's patch range [lo, hi).  Every wave finds it on its
  //    own (two searches sharing a first round of 64 probes, then 32 lanes per
  //    key), so the records can be read without a barrier in between.
  const uint64_t recs = kHeader + sm_sec<DT>(n) + nbm;
  uint32_t lo = 0, hi = 0;
  if (P > 0) {
    if (tpr == 1) {
      hi = (uint32_t)P;
    } else {
      uint64_t a0 = 0, z0 = 0, a1 = 0, z1 = 0;  // first p with idx[p] >= key lies in [a, z]
      {
        const uint64_t step = (P + 63) / 64;
        const uint64_t p = (uint64_t)lane * step;
        uint32_t idx = 0, ex = 0;
        if (p < P) read_rec(st, recs, p, idx, ex);
        const uint64_t m0 = __ballot(p < P && idx < ts), m1 = __ballot(p < P && idx < te);
        if (m0) { a0 = (uint64_t)(63u - (uint32_t)__clzll(m0)) * step + 1; z0 = min<uint64_t>(P, a0 - 1 + step); }
        if (m1) { a1 = (uint64_t)(63u - (uint32_t)__clzll(m1)) * step + 1; z1 = min<uint64_t>(P, a1 - 1 + step); }
      }
      while (z0 > a0 || z1 > a1) {
        const bool second = lane >= 32;
        const uint64_t a = second ? a1 : a0, z = second ? z1 : z0, key = second ? te : ts;
        const uint64_t step = (z - a + 31) / 32;
        const uint64_t p = a + (uint64_t)(lane & 31u) * step;
        const bool valid = z > a && p < z;
        uint32_t idx = 0, ex = 0;
        if (valid) read_rec(st, recs, p, idx, ex);
        const uint64_t m = __ballot(valid && idx < key);
        const uint32_t h0 = (uint32_t)m, h1 = (uint32_t)(m >> 32);
        if (z0 > a0) {
          const uint64_t s0 = (z0 - a0 + 31) / 32;
          if (h0 == 0) { z0 = a0; } else { a0 = a0 + (uint64_t)(31u - (uint32_t)__clz(h0)) * s0 + 1; z0 = min<uint64_t>(z0, a0 - 1 + s0); }
        }
        if (z1 > a1) {
          const uint64_t s1 = (z1 - a1 + 31) / 32;
          if (h1 == 0) { z1 = a1; } else { a1 = a1 + (uint64_t)(31u - (uint32_t)__clz(h1)) * s1 + 1; z1 = min<uint64_t>(z1, a1 - 1 + s1); }
        }
      }
      lo = (uint32_t)a0;
      hi = (uint32_t)a1;
      if (tid == 0) {
        uint32_t e = 0;
        if (hi < lo) e |= CIERA_ST_PATCH;
        if (te == n && hi != P) e |= CIERA_ST_PATCH;
        if (e) report(status_out, e);
      }
      if (hi < lo) hi = lo;
    }
  }

  // 4. patches of the tile into LDS, over the cached exponents.
  //    Each pass gives every thread c <= kRecBatch consecutive records (c as
  //    small as the pass allows, so the records spread over all waves), read
  //    as one round of aligned words; the first pass shares its round with
  //    the tile's bitmap bits.  A record's predecessor, for the ascending-order
  //    check, is the thread's previous record or the last one of the lane
  //    below (lane 0 reads it).
  const bool patched = hi > lo;  // uniform
  const uint64_t tb0 = ts >> lb, tb1 = (te + B - 1) >> lb;
  const uint32_t nbt = (uint32_t)(tb1 - tb0);
  const uint8_t* bm = st + kHeader + sm_sec<DT>(n);
  const bool bm_mine = P > 0 && tid * 32 < nbt;
  Words2 bmw{0, 0, 0};
  uint32_t bm_tail = 0;
  uint32_t bm_got = 0;
  if (bm_mine) {
    bmw = load_bits_w(bm, tb0 + tid * 32);
    bm_got = bits_of(bmw, min(32u, nbt - tid * 32));
  }
  if (P > 0 && te == n && tid == 0 && (nb & 7u) != 0) bm_tail = gp(bm)[nbm - 1] >> (nb & 7u);
  // Puts record p (index idx, exponent v) into LDS after checking it: strictly
  // after its predecessor's index pidx, and inside the tile.  The first record
  // of each block marks the block (records ascend; when they do not, the
  // order error is reported and the bitmap verdict is unspecified).
  uint8_t* const s_exb = reinterpret_cast<uint8_t*>(s_ex);
  auto put = [&](uint32_t p, uint32_t idx, uint32_t v, uint32_t pidx) {
    uint32_t e = 0;
    if (p > 0 && pidx >= idx) e |= CIERA_ST_PATCH;
    if (idx < ts || idx >= te) {
      e |= CIERA_ST_PATCH;
    } else {
      s_exb[idx - ts] = (uint8_t)v;
      if (p == lo || (pidx >> lb) != (idx >> lb)) {
        const uint32_t bb = (uint32_t)((idx >> lb) - tb0);
        atomicOr(&s_expbm[bb >> 5], 1u << (bb & 31u));
      }
    }
    if (e) report(status_out, e);
  };
  if (patched) {
    const uint64_t send = recs + 5 * P;  // end of the stream
    for (uint32_t base = lo, c; base < hi; base += c * kDecThreads) {  // uniform loop
      c = min<uint32_t>(kRecBatch, (hi - base + kDecThreads - 1) / kDecThreads);
      if (c == 1) {  // one record per thread: the two words that hold it
        const uint32_t p = base + tid;
        uint32_t idx = 0, v = 0, pidx = 0, pv;
        if (p < hi) read_rec(st, recs, p, idx, v);
        if (lane == 0 && p < hi && p > 0) read_rec(st, recs, p - 1, pidx, pv);
        const uint32_t up = __shfl_up(idx, 1);
        if (lane != 0) pidx = up;
        if (p < hi) put(p, idx, v, pidx);
        continue;
      }
      const uint32_t q0 = base + c * tid;
      const uint64_t o0 = recs + 5ull * q0, a0 = o0 & ~(uint64_t)3;
      const uint64_t wend = min<uint64_t>(send, o0 + 5u * c);  // words starting before this end
      const G1 uint32_t* wp = gp(reinterpret_cast<const uint32_t*>(st + a0));
      uint32_t w[kRecWords];
#pragma unroll
      for (int j = 0; j < kRecWords; ++j) w[j] = 0;
      Words2 pw{0, 0, 0};
      if (q0 < hi) {
        w[0] = wp[0];  // the first two words hold record q0
        w[1] = wp[1];
#pragma unroll
        for (int j = 2; j < kRecWords; ++j)
          if (a0 + 4u * j < wend) w[j] = wp[j];
        if (lane == 0 && q0 > 0) pw = load_rec(st, recs, q0 - 1);
      }
      const uint32_t b0 = (uint32_t)(o0 - a0);
      uint32_t idx[kRecBatch], v[kRecBatch];
#pragma unroll
      for (int k = 0; k < kRecBatch; ++k) {  // record k starts at byte b0 + 5k of w
        const int jl = (5 * k) >> 2;
        const uint32_t b = b0 + 5u * k;
        const bool up1 = (int)(b >> 2) != jl;
        const uint32_t x0 = up1 ? w[jl + 1] : w[jl], x1 = up1 ? w[jl + 2] : w[jl + 1];
        const uint64_t z = ((uint64_t)x0 | ((uint64_t)x1 << 32)) >> (8u * (b & 3u));
        idx[k] = (uint32_t)z;
        v[k] = (uint32_t)(z >> 32) & 0xFFu;
      }
      uint32_t pidx, pv;
      rec_fields(pw, pidx, pv);
      uint32_t last = idx[0];
#pragma unroll
      for (int k = 1; k < kRecBatch; ++k) last = (uint32_t)k < c ? idx[k] : last;
      const uint32_t up = __shfl_up(last, 1);
      if (lane != 0) pidx = up;
#pragma unroll
      for (int k = 0; k < kRecBatch; ++k) {
        const uint32_t p = q0 + (uint32_t)k;
        if ((uint32_t)k < c && p < hi) put(p, idx[k], v[k], k == 0 ? pidx : idx[k > 0 ? k - 1 : 0]);
      }
    }
  }
  if (P > 0) __syncthreads();
  uint32_t ex[U][4];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int k = 0; k < 4; ++k) ex[u][k] = cw[u][k];
    if (patched && cnt[u] > 0) {
      const v4u e = *reinterpret_cast<const v4u*>(&s_ex[((uint32_t)u * kDecRow + tid * kEPT) / 4]);
      ex[u][0] = e.x; ex[u][1] = e.y; ex[u][2] = e.z; ex[u][3] = e.w;
    }
  }

  // 5. bitmap check: the tile's bits mark exactly the blocks that hold patches
  if (P > 0) {
    uint32_t e = 0;
    if (bm_mine && bm_got != s_expbm[tid]) e |= CIERA_ST_BITMAP;
    if (bm_tail != 0) e |= CIERA_ST_BITMAP;
    if (e) report(status_out, e);
  }

  // 6. merge and store; write back the cache lines that changed
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (cnt[u] > 0) {
      const uint64_t c0 = ts + (uint64_t)u * kDecRow + (uint64_t)tid * kEPT;
      if constexpr (DT == 1) {
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) bf16x4_join(sw[u][q], ex[u][q], o[2 * q], o[2 * q + 1]);
        store_words<8>(out + c0 * E, (uint32_t)cnt[u] * E, aligned, o);
      } else {
        uint32_t v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = join<DT>(sm_from_words<DT>(sw[u], j), byte_of(ex[u], j));
        store16<DT>(out + c0 * E, cnt[u], v, aligned);
      }
    }
    // cache write-back in whole 128-byte lines (8 lanes): scattered partial
    // lines cost more HBM time than the extra bytes of full lines; the
    // stores are non-temporal (nothing in this launch reads them again)
    const bool dirty = cnt[u] > 0 && (ex[u][0] != cw[u][0] || ex[u][1] != cw[u][1] ||
                                      ex[u][2] != cw[u][2] || ex[u][3] != cw[u][3]);
    const uint64_t m = patched ? __ballot(dirty) : 0ull;
    if (cnt[u] > 0 && ((m >> (lane & ~7u)) & 0xFFu)) {
      const uint64_t c0 = ts + (uint64_t)u * kDecRow + (uint64_t)tid * kEPT;
      store_words<4, true>(cache + c0, (uint32_t)cnt[u], aligned, ex[u]);
    }
  }
}

// -------------------------------------------------------------- cache update

template <int DT>
__global__ __launch_bounds__(kThreads) void cache_update_kernel(const uint8_t* __restrict__ w,
                                                                uint8_t* __restrict__ cache, uint64_t n) {
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
// Each launcher clears the thread's last-error state first, so that the error it
// returns is the launch's own and not one left by an unrelated earlier call.

// Workgroups per launch: a grid stays well below 2^32 work-items; larger
// batches are cut into launches of whole items.
constexpr uint64_t kMaxGrid = (uint64_t)1 << 22;

static hipError_t launch_encode_part(int dtype, int sub, uint32_t nitems, const EncArgs& a, uint32_t* ctl,
                                     uint32_t batch_id, hipStream_t s) {
  (void)hipGetLastError();
  const dim3 grid(nitems * a.tpi), block(kThreads);
#define CIERA_ENC(DT, S) hipLaunchKernelGGL((encode_kernel<DT, S>), grid, block, 0, s, a, ctl, batch_id)
  if (dtype == 1) {
    switch (sub) {
      case 1: CIERA_ENC(1, 1); break;
      case 2: CIERA_ENC(1, 2); break;
      case 4: CIERA_ENC(1, 4); break;
      case 8: CIERA_ENC(1, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else if (dtype == 2) {
    switch (sub) {
      case 1: CIERA_ENC(2, 1); break;
      case 2: CIERA_ENC(2, 2); break;
      case 4: CIERA_ENC(2, 4); break;
      case 8: CIERA_ENC(2, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else if (dtype == 3) {
    switch (sub) {
      case 1: CIERA_ENC(3, 1); break;
      case 2: CIERA_ENC(3, 2); break;
      case 4: CIERA_ENC(3, 4); break;
      case 8: CIERA_ENC(3, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef CIERA_ENC
  return hipGetLastError();
}

hipError_t launch_encode(int dtype, int sub, uint32_t nitems, const EncArgs& a, uint32_t* ctl,
                         uint32_t batch_id, hipStream_t s) {
  const uint32_t per = (uint32_t)std::max<uint64_t>(1, kMaxGrid / a.tpi);
  for (uint32_t i = 0; i < nitems; i += per) {
    EncArgs c = a;
    c.item0 = a.item0 + i;
    c.status = a.status + (uint64_t)i * a.tpi;  // status words are indexed from the group's first item
    if (hipError_t e = launch_encode_part(dtype, sub, std::min(per, nitems - i), c, ctl, batch_id, s)) return e;
  }
  return hipSuccess;
}

hipError_t launch_encode_fixup(const EncItem* items, uint32_t count, uint32_t wg_per_item, const uint32_t* raw_flag,
                               uint32_t* ctl, uint32_t batch_id, hipStream_t s) {
  (void)hipGetLastError();
  if (count == 0 || wg_per_item == 0) return hipSuccess;
  const dim3 grid(wg_per_item, count < 65535u ? count : 65535u), block(kThreads);
  hipLaunchKernelGGL(encode_fixup_kernel, grid, block, 0, s, items, count, raw_flag, ctl, batch_id);
  return hipGetLastError();
}

static hipError_t launch_decode_part(int dtype, int u, const DecItem* items, uint32_t item0, uint32_t nitems,
                                     uint32_t tpr, uint32_t world, uint32_t* status, const uint32_t* ctl,
                                     uint32_t batch_id, hipStream_t s) {
  (void)hipGetLastError();
  const dim3 grid(nitems * tpr * world), block(kDecThreads);
#define CIERA_DEC(DT, U) \
  hipLaunchKernelGGL((decode_kernel<DT, U>), grid, block, 0, s, items, item0, tpr, world, status, ctl, batch_id)
  if (dtype == 1) {
    switch (u) {
      case 1: CIERA_DEC(1, 1); break;
      case 2: CIERA_DEC(1, 2); break;
      case 4: CIERA_DEC(1, 4); break;
      default: return hipErrorInvalidValue;
    }
  } else if (dtype == 2) {
    switch (u) {
      case 1: CIERA_DEC(2, 1); break;
      case 2: CIERA_DEC(2, 2); break;
      case 4: CIERA_DEC(2, 4); break;
      default: return hipErrorInvalidValue;
    }
  } else if (dtype == 3) {
    switch (u) {
      case 1: CIERA_DEC(3, 1); break;
      case 2: CIERA_DEC(3, 2); break;
      case 4: CIERA_DEC(3, 4); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef CIERA_DEC
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, int u, const DecItem* items, uint32_t item0, uint32_t nitems, uint32_t tpr,
                         uint32_t world, uint32_t* status, const uint32_t* ctl, uint32_t batch_id,
                         hipStream_t s) {
  const uint64_t tpi = (uint64_t)tpr * world;
  if (tpi * kDecThreads >= ((uint64_t)1 << 32)) return hipErrorInvalidValue;  // one item alone too large
  const uint32_t per = (uint32_t)std::max<uint64_t>(1, kMaxGrid / tpi);
  for (uint32_t i = 0; i < nitems; i += per) {
    if (hipError_t e = launch_decode_part(dtype, u, items, item0 + i, std::min(per, nitems - i), tpr, world, status,
                                          ctl, batch_id, s))
      return e;
  }
  return hipSuccess;
}

hipError_t launch_cache_update(int dtype, const uint8_t* w, uint8_t* cache, uint64_t n, hipStream_t s) {
  const uint64_t chunks = (n + 15) / 16;
  uint64_t blocks = (chunks + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return hipSuccess;
  (void)hipGetLastError();
  const dim3 grid((uint32_t)blocks), block(kThreads);
  if (dtype == 1) hipLaunchKernelGGL((cache_update_kernel<1>), grid, block, 0, s, w, cache, n);
  else if (dtype == 2) hipLaunchKernelGGL((cache_update_kernel<2>), grid, block, 0, s, w, cache, n);
  else if (dtype == 3) hipLaunchKernelGGL((cache_update_kernel<3>), grid, block, 0, s, w, cache, n);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ciera
