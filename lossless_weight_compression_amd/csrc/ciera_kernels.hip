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
#include <cstring>
#include <mutex>
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
// Non-temporal 16-byte load: for data read once (the bulk streams), which
// then does not displace reused lines.  Used where a wave's 16-byte loads of
// a chunk row cover whole 128-byte lines between them with at most two loads
// per thread: contiguous pieces, and bf16 and fp16 chunks (16 or 32 bytes per
// thread).  A thread's 48 or 64 contiguous fp32 bytes, read with three or four
// strided loads, measured 15% slower (decode) and 19% slower (encode) with
// non-temporal loads, so those load normally; the hot paths read fp32 rows as
// contiguous pieces instead (load_sm_pieces, load_x_pieces).
template <int DT>
constexpr bool kNtBulk = DT != 2;
__device__ __forceinline__ v4u ldg16_nt(const void* p) {
  return __builtin_nontemporal_load(gp(reinterpret_cast<const v4u*>(p)));
}
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

// min(k, n - x) for x < n, else 0 -- the values of a chunk, row or tile that
// starts at x in a shard of n -- with a saturating subtraction instead of a
// guarded one.  Written as `x < n ? min(k, n - x) : 0`, hipcc speculated the
// guarded `n - x` into every thread as `sub nuw` feeding a `noundef` umin call;
// constraint elimination then took n >= x as a fact for every thread, also for
// threads past the shard's end, and folded the length of the first row of a
// partial last tile to a whole row.  A saturating subtraction has no guard to
// speculate and no wrap flag to reason from.
__device__ __forceinline__ uint64_t left_in(uint64_t n, uint64_t x, uint64_t k) {
  return min<uint64_t>(k, __builtin_elementwise_sub_sat(n, x));
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

// 16 bytes (cache exponents) stored from four little-endian words.
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

// Raw 32-bit words of nbytes <= 4*NW bytes at p (vector loads, non-temporal
// if NT, when complete and allowed).
template <int NW, bool NT = false>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t nbytes, bool vec, uint32_t w[NW]) {
  if (vec && nbytes == NW * 4) {
#pragma unroll
    for (int q = 0; q < NW / 4; ++q) {
      const v4u a = NT ? ldg16_nt(p + 16 * q) : ldg16(p + 16 * q);
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
    load_words<SW, kNtBulk<DT>>(a, (uint32_t)cnt * Tr<DT>::SMBITS / 8, true, w);
  }
}

// fp32 and fp16 sign|mantissa records are 3 and 11/8 bytes per value, so a
// thread's 16-value chunk (48 or 22 bytes) is not a whole number of 16-byte
// pieces and its loads would be strided across the wave: every instruction
// would touch each line in part, and non-temporal loads then fetch lines
// again.  A wave whose 1024 values of a row are all inside the shard reads its
// row's records (3072 or 1408 bytes, 16-byte aligned) as contiguous pieces
// instead -- lane t takes pieces t, t + 64 and t + 128 -- so that each load
// covers whole lines, and the lanes then swap them through LDS.
template <int DT>
constexpr int kSmPieces = DT == 2 ? 3 : DT == 3 ? 2 : 0;  // 16-byte pieces per lane
template <int DT>
constexpr uint32_t kSmWaveRow = 1024u * Tr<DT>::SMBITS / 8;  // record bytes of a wave's row
template <int DT>
__device__ __forceinline__ void load_sm_pieces(const uint8_t* p, v4u pc[kSmPieces<DT> ? kSmPieces<DT> : 1]) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (int q = 0; q < kSmPieces<DT>; ++q) {
    const uint32_t k = 64u * q + lane;
    if (16u * k < kSmWaveRow<DT>) pc[q] = ldg16_nt(p + 16 * k);
  }
}
// The pieces to `stage` (the wave's own kSmWaveRow bytes of LDS) and back as
// this lane's chunk words, as load_smw gives them.  LDS accesses of one wave
// complete in order; the wave barriers keep the compiler from moving them.
template <int DT, int SW>
__device__ __forceinline__ void swap_sm_pieces(uint32_t* stage, const v4u pc[kSmPieces<DT> ? kSmPieces<DT> : 1],
                                               uint32_t w[SW]) {
  const uint32_t lane = lane_id();
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < kSmPieces<DT>; ++q) {
    const uint32_t k = 64u * q + lane;
    if (16u * k < kSmWaveRow<DT>) *reinterpret_cast<v4u*>(stage + 4 * k) = pc[q];
  }
  __builtin_amdgcn_wave_barrier();
  if constexpr (DT == 2) {  // 48 bytes at 48 * lane
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const v4u a = *reinterpret_cast<const v4u*>(stage + 12 * lane + 4 * q);
      w[4 * q] = a.x; w[4 * q + 1] = a.y; w[4 * q + 2] = a.z; w[4 * q + 3] = a.w;
    }
  } else {  // fp16: 22 bytes at 22 * lane, as 6 aligned words shifted when it starts mid-word
    const uint32_t b = 22u * lane, sh = b & 3u;
    const uint32_t* q = stage + (b >> 2);
#pragma unroll
    for (int i = 0; i < 6; ++i) w[i] = q[i];
    if (sh) {
#pragma unroll
      for (int i = 0; i < 5; ++i) w[i] = (w[i] >> 16) | (w[i + 1] << 16);
      w[5] >>= 16;
    }
  }
  __builtin_amdgcn_wave_barrier();
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

// 16 bytes at any alignment, as the aligned words that cover them: every word
// read starts at or before the 16th byte, so it stays inside a buffer whose
// end is 16-byte aligned.
__device__ __forceinline__ v4u load16_any(const uint8_t* p) {
  const uint32_t a = (uint32_t)(reinterpret_cast<uintptr_t>(p) & 3u);
  const G1 uint32_t* w = gp(reinterpret_cast<const uint32_t*>(p - a));
  v4u v;
  if (a == 0) {
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
  } else {
    const uint32_t x0 = w[0], x1 = w[1], x2 = w[2], x3 = w[3], x4 = w[4], sh = 8 * a;
    v.x = (x0 >> sh) | (x1 << (32 - sh));
    v.y = (x1 >> sh) | (x2 << (32 - sh));
    v.z = (x2 >> sh) | (x3 << (32 - sh));
    v.w = (x3 >> sh) | (x4 << (32 - sh));
  }
  return v;
}

// ORs decode status bits into the caller's word; a plain read first keeps a
// stream of identical errors (every tile of a corrupt batch) from serializing
// on one address.
__device__ __forceinline__ void report(uint32_t* status, uint32_t bits) {
  if ((__hip_atomic_load(gp(status), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & bits) != bits)
    __hip_atomic_fetch_or(gp(status), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// --------------------------------------------------------------------- encode
// Two kernels, and no workgroup ever waits on another.
//
// encode_kernel: one workgroup per tile of S*4096 values of one item.  Split,
// compare, the sign|mantissa (or RAW) stores, the tile's bitmap bytes, its
// change count, and its first `cap` changes as (index in tile, exponent) words
// in the tile's stash in scratch.
//
// encode_finish_kernel: per item, the sum of its tile counts decides the mode;
// the header is written, the stashed changes go to their places in the patch
// list (a tile whose changes overflowed its stash derives them again from the
// shard and the cache), or the stream is rewritten RAW when the compressed
// form turned out not shorter.

// Exponent bytes (four words) and change mask of one 16-value chunk, given its
// raw value words xw and cached exponent words cw; only the cnt values present
// count (all 16 when FULL).
template <int DT, bool FULL>
__device__ __forceinline__ uint32_t chunk_exps(const uint32_t* xw, const uint32_t cw[4], int cnt, uint32_t expk[4]) {
  uint32_t mask = 0;
  expk[0] = expk[1] = expk[2] = expk[3] = 0;
  if constexpr (DT == 1) {
    uint32_t dif[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      expk[q] = bf16x4_exp(xw[2 * q], xw[2 * q + 1]);
      dif[q] = expk[q] ^ cw[q];
      if (!FULL) {  // only the cnt values present
        const int nv = cnt - 4 * q;
        dif[q] &= nv >= 4 ? 0xFFFFFFFFu : nv <= 0 ? 0u : (1u << (8 * nv)) - 1u;
      }
    }
    if (dif[0] | dif[1] | dif[2] | dif[3]) mask = nonzero_bytes16(dif);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      uint32_t v;
      if constexpr (Tr<DT>::E == 2) v = (xw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      else v = xw[j];
      const uint32_t e = exp_of<DT>(v);
      expk[j >> 2] |= e << (8 * (j & 3));
      if ((FULL || j < cnt) && e != byte_of(cw, j)) mask |= 1u << j;
    }
  }
  return mask;
}

// Stores the chunk's sign|mantissa records (compress) or its raw values.
template <int DT>
__device__ __forceinline__ void chunk_store(uint8_t* stream, uint64_t c0, int cnt, const uint32_t* xw, bool compress) {
  constexpr int E = Tr<DT>::E;
  if constexpr (DT == 1) {
    if (compress) {
      uint32_t smw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) smw[q] = bf16x4_sm(xw[2 * q], xw[2 * q + 1]);
      store_words<4>(stream + kHeader + c0, (uint32_t)cnt, true, smw);
    } else {
      store_words<4 * E>(stream + kHeader + c0 * E, (uint32_t)cnt * E, true, xw);
    }
  } else {
    uint32_t v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (E == 2) v[j] = (xw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      else v[j] = xw[j];
    }
    if (compress) {
      uint32_t sm[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) sm[j] = sm_of<DT>(v[j]);
      store_sm16<DT>(stream + kHeader + sm_off<DT>(c0), cnt, sm);
    } else {
      store16<DT>(stream + kHeader + c0 * E, cnt, v);
    }
  }
}

// The sign|mantissa section bytes of one 16-value chunk as little-endian words
// (bf16 16 bytes in 4 words, fp32 48 in 12, fp16 22 in 6), from its raw words.
template <int DT>
constexpr int kSmWords = DT == 1 ? 4 : DT == 2 ? 12 : 6;
template <int DT>
__device__ __forceinline__ void chunk_sm_words(const uint32_t* xw, uint32_t o[kSmWords<DT>]) {
  if constexpr (DT == 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = bf16x4_sm(xw[2 * q], xw[2 * q + 1]);
  } else {
    uint32_t sm[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t v = Tr<DT>::E == 2 ? (xw[j >> 1] >> (16 * (j & 1))) & 0xFFFFu : xw[j];
      sm[j] = sm_of<DT>(v);
    }
    if constexpr (DT == 3) {
      pack11x16(sm, o);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t a = sm[4 * q], b = sm[4 * q + 1], c = sm[4 * q + 2], d = sm[4 * q + 3];
        o[3 * q] = a | (b << 24);
        o[3 * q + 1] = (b >> 8) | (c << 16);
        o[3 * q + 2] = (c >> 16) | (d << 8);
      }
    }
  }
}

// Stores the section bytes of the first cnt values of a chunk, given as the
// words chunk_sm_words made, at p = section start + the chunk's offset (16-byte
// aligned for bf16 and fp32, even for fp16).
template <int DT>
__device__ __forceinline__ void store_sm_words(uint8_t* p, int cnt, const uint32_t o[kSmWords<DT>]) {
  if constexpr (DT == 1) {
    store_words<4>(p, (uint32_t)cnt, true, o);
  } else if constexpr (DT == 2) {
    store_words<12>(p, 3u * (uint32_t)cnt, true, o);
  } else if (cnt == 16) {
    if ((reinterpret_cast<uintptr_t>(p) & 3u) == 0) {
#pragma unroll
      for (int i = 0; i < 5; ++i) gp(reinterpret_cast<uint32_t*>(p))[i] = o[i];
      gp(reinterpret_cast<uint16_t*>(p + 20))[0] = (uint16_t)o[5];
    } else {  // p = 4q + 2
      gp(reinterpret_cast<uint16_t*>(p))[0] = (uint16_t)o[0];
#pragma unroll
      for (int i = 0; i < 5; ++i) gp(reinterpret_cast<uint32_t*>(p + 2))[i] = (o[i] >> 16) | (o[i + 1] << 16);
    }
  } else {
    const int nb = (11 * cnt + 7) / 8;
#pragma unroll
    for (int b = 0; b < 22; ++b)
      if (b < nb) gp(p)[b] = (uint8_t)(o[b >> 2] >> (8 * (b & 3)));
  }
}

// The encode's side of the same exchange: a wave's 1024 values of a chunk row
// (2048 or 4096 bytes, 16-byte aligned) loaded as contiguous 16-byte pieces,
// lane t taking pieces t + 64q, and swapped through `stage` (the wave's own
// kXWaveRow bytes of LDS) into each lane's 16 values; and a wave's fp32 or
// fp16 sign|mantissa records, 48 or 22 bytes per lane, put together in
// `stage` and stored as contiguous pieces.  LDS accesses of one wave complete
// in order; the wave barriers keep the compiler from moving them.
template <int DT>
constexpr uint32_t kXWaveRow = 1024u * Tr<DT>::E;
// LDS slot (16-byte unit) of piece q of lane t when every lane holds E (2 or 4)
// consecutive pieces of a row: E * t + q, with q XOR-ed by the lane's group so
// that the 16 lanes of one LDS pass fall on 16 different bank groups (E * t
// alone would put 2 or 4 lanes on each).  Piece k of the row, lane-held by
// lane k / E, is in slot xslot<E>(k / E, k % E).
template <int E>
__device__ __forceinline__ uint32_t xslot(uint32_t t, uint32_t q) {
  return E * t + (q ^ ((t >> (E == 2 ? 3 : 2)) & (E - 1)));
}
template <int DT>
__device__ __forceinline__ void load_x_pieces(const uint8_t* p, v4u pc[Tr<DT>::E]) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (int q = 0; q < Tr<DT>::E; ++q) pc[q] = ldg16_nt(p + 16 * (64u * q + lane));
}
// load_x_pieces for a row of which only the first nb bytes (a multiple of the
// value size) lie in the shard: pieces past them read as zeros, and the piece
// that holds the last of them is read byte by byte.
template <int DT>
__device__ __forceinline__ void load_x_pieces_upto(const uint8_t* p, uint32_t nb, v4u pc[Tr<DT>::E]) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (int q = 0; q < Tr<DT>::E; ++q) {
    const uint32_t o = 16u * (64u * q + lane);
    if (o + 16u <= nb) {
      pc[q] = ldg16_nt(p + o);
    } else {
      uint32_t w[4] = {0, 0, 0, 0};
      if (o < nb) load_words<4>(p + o, nb - o, false, w);
      pc[q].x = w[0]; pc[q].y = w[1]; pc[q].z = w[2]; pc[q].w = w[3];
    }
  }
}
template <int DT>
__device__ __forceinline__ void swap_x_pieces(uint32_t* stage, const v4u pc[Tr<DT>::E], uint32_t xw[4 * Tr<DT>::E]) {
  constexpr int E = Tr<DT>::E;
  const uint32_t lane = lane_id();
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const uint32_t k = 64u * q + lane;
    *reinterpret_cast<v4u*>(stage + 4 * xslot<E>(k / E, k % E)) = pc[q];
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < E; ++q) {
    const v4u a = *reinterpret_cast<const v4u*>(stage + 4 * xslot<E>(lane, q));
    xw[4 * q] = a.x; xw[4 * q + 1] = a.y; xw[4 * q + 2] = a.z; xw[4 * q + 3] = a.w;
  }
  __builtin_amdgcn_wave_barrier();
}
template <int DT>
__device__ __forceinline__ void store_sm_pieces(uint8_t* p, uint32_t* stage, const uint32_t o[kSmWords<DT>]) {
  static_assert(DT == 2 || DT == 3, "fp32 and fp16 only");
  constexpr uint32_t R = kSmWaveRow<DT>;
  const uint32_t lane = lane_id();
  __builtin_amdgcn_wave_barrier();
  if constexpr (DT == 2) {  // 48 bytes at 48 * lane
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      v4u a;
      a.x = o[4 * q]; a.y = o[4 * q + 1]; a.z = o[4 * q + 2]; a.w = o[4 * q + 3];
      *reinterpret_cast<v4u*>(stage + 12 * lane + 4 * q) = a;
    }
  } else {  // 22 bytes at 22 * lane: whole words, and a half-word at one end
    const uint32_t b = 22u * lane;
    if ((b & 3u) == 0) {
#pragma unroll
      for (int i = 0; i < 5; ++i) stage[(b >> 2) + i] = o[i];
      reinterpret_cast<uint16_t*>(stage)[(b + 20) >> 1] = (uint16_t)o[5];
    } else {  // b = 4q + 2
      reinterpret_cast<uint16_t*>(stage)[b >> 1] = (uint16_t)o[0];
#pragma unroll
      for (int i = 0; i < 5; ++i) stage[((b + 2) >> 2) + i] = (o[i] >> 16) | (o[i + 1] << 16);
    }
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < (int)((R / 16 + 63) / 64); ++q) {
    const uint32_t k = 64u * q + lane;
    if (16u * k < R) stg16(p + 16 * k, *reinterpret_cast<const v4u*>(stage + 4 * k));
  }
  __builtin_amdgcn_wave_barrier();
}

// Exclusive prefix of v over the workgroup's threads in thread order, and the
// total.  Contains one barrier; s_red (4 words) must not be in use by another
// call until every thread has passed a later barrier.
template <class V>
__device__ __forceinline__ V block_scan(V v, V* s_red, V& total) {
  const uint32_t lane = lane_id(), wave = threadIdx.x >> 6;
  V incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const V t = __shfl_up(incl, o);
    if (lane >= (uint32_t)o) incl += t;
  }
  if (lane == 63) s_red[wave] = incl;
  __syncthreads();
  V before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const V t = s_red[w];
    if (w < (int)wave) before += t;
    tot += t;
  }
  total = tot;
  return before + incl - v;
}

// One 5-byte patch record (u32 index, u8 exponent, little-endian) at byte pos
// of the stream, if it lies inside the stream's capacity.
__device__ __forceinline__ void put_record(uint8_t* stream, uint64_t capacity, uint64_t pos, uint32_t idx, uint32_t ex) {
  if (pos + 5 <= capacity) {
    G1 uint8_t* q = gp(stream + pos);
    q[0] = (uint8_t)idx; q[1] = (uint8_t)(idx >> 8);
    q[2] = (uint8_t)(idx >> 16); q[3] = (uint8_t)(idx >> 24);
    q[4] = (uint8_t)ex;
  }
}

// A thread's consecutive patch records -- the changes of one 16-value chunk
// (mask), indices idx0 + bit, exponents from expk -- at 5-byte places from
// byte pos of the stream.  Each record but the last goes out as one unaligned
// 8-byte store that also carries the next record's first three bytes (the
// next store rewrites them with the same values); the last as a 4-byte and a
// 1-byte store, so no store reaches past the thread's own records.  gfx950
// stores to global memory at any byte alignment.
typedef uint32_t u32_any __attribute__((aligned(1)));
typedef uint64_t u64_any __attribute__((aligned(1)));
__device__ __forceinline__ void put_records(uint8_t* stream, uint64_t pos, uint32_t mask, uint32_t idx0,
                                            const uint32_t expk[4]) {
  if (!mask) return;
  int j = __ffs(mask) - 1;
  mask &= mask - 1;
  while (mask) {
    const int jn = __ffs(mask) - 1;
    mask &= mask - 1;
    const uint64_t v = (uint64_t)(idx0 + (uint32_t)j) | ((uint64_t)byte_of(expk, j) << 32) |
                       ((uint64_t)((idx0 + (uint32_t)jn) & 0xFFFFFFu) << 40);
    *(G1 u64_any*)(stream + pos) = v;
    pos += 5;
    j = jn;
  }
  *(G1 u32_any*)(stream + pos) = idx0 + (uint32_t)j;
  gp(stream)[pos + 4] = (uint8_t)byte_of(expk, j);
}

// ----------------------------------------------- block-hash variant (encode)
// [CIERA 3.1; Algorithm 1] as published: a 128-bit hash per block of B values
// (two 64-bit halves from SplitMix64's output function), compared with the
// sender's cached hash; changed blocks travel whole.  The hash of a block's
// exponent bytes, as little-endian 8-byte words w_j (zero-padded), L bytes:
//   H_s = mix64((sum_j mix64(w_j ^ (s + (j + 1) * GAMMA)) + L) mod 2^64),
// position-keyed so that the words of a block can be summed in parallel.
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;  // SplitMix64 increment
constexpr uint64_t kSeedA = 0x243F6A8885A308D3ull, kSeedB = 0x13198A2E03707344ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {  // SplitMix64 output function
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// The terms of one chunk's 16 exponent bytes (words 2*lc and 2*lc + 1 of its
// block), of which the first `valid` bytes belong to the block.
__device__ __forceinline__ void chunk_hash_terms(const uint32_t ex[4], uint32_t lc, uint32_t valid, uint64_t& ta,
                                                 uint64_t& tb) {
  const uint64_t w0 = ex[0] | ((uint64_t)ex[1] << 32), w1 = ex[2] | ((uint64_t)ex[3] << 32);
  const uint64_t k0 = (uint64_t)(2 * lc + 1) * kGamma, k1 = (uint64_t)(2 * lc + 2) * kGamma;
  ta = tb = 0;
  if (valid > 0) {
    ta += mix64(w0 ^ (kSeedA + k0));
    tb += mix64(w0 ^ (kSeedB + k0));
  }
  if (valid > 8) {
    ta += mix64(w1 ^ (kSeedA + k1));
    tb += mix64(w1 ^ (kSeedB + k1));
  }
}

// Sum over aligned groups of g lanes (g a power of two <= 64, uniform).
__device__ __forceinline__ uint64_t group_sum(uint64_t v, uint32_t g) {
  for (uint32_t o = 1; o < g; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// The 128-bit hashes of the blocks of one tile (S rows of 4096 values; ex[s]
// are the exponent bytes of this thread's 16-value chunk of row s, zero past
// n).  Afterwards the first thread of each block that starts before n has
// lead[s] set and the block's hash in ha[s], hb[s].  Contains one barrier when
// a block is wider than a wave (B > 1024); s_hp: 8 * S words of LDS.
template <int S>
__device__ __forceinline__ void tile_block_hashes(const uint32_t (&ex)[S][4], uint64_t base, uint64_t n, uint32_t B,
                                                  uint64_t* s_hp, bool (&lead)[S], uint64_t (&ha)[S],
                                                  uint64_t (&hb)[S]) {
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint32_t cpb = B >> 4;  // chunks per block, 4 .. 256: the block lies inside one row
  const uint32_t g = min(cpb, 64u);
  uint64_t L[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
    const uint64_t b0 = c0 & ~(uint64_t)(B - 1);  // the block's first value
    const uint32_t lc = (uint32_t)((c0 - b0) >> 4);
    L[s] = b0 < n ? min<uint64_t>(B, n - b0) : 0;
    const uint32_t valid = (uint32_t)left_in(L[s], 16ull * lc, 16);
    uint64_t ta, tb;
    chunk_hash_terms(ex[s], lc, valid, ta, tb);
    ha[s] = group_sum(ta, g);
    hb[s] = group_sum(tb, g);
    lead[s] = lc == 0 && L[s] > 0;
    if (cpb > 64 && lane == 0) {
      s_hp[2 * (s * 4 + wave)] = ha[s];
      s_hp[2 * (s * 4 + wave) + 1] = hb[s];
    }
  }
  if (cpb > 64) {  // uniform: the waves of a block meet in LDS
    __syncthreads();
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (lead[s]) {
        ha[s] = hb[s] = 0;
        for (uint32_t w = wave; w < wave + (cpb >> 6); ++w) {
          ha[s] += s_hp[2 * (s * 4 + w)];
          hb[s] += s_hp[2 * (s * 4 + w) + 1];
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (lead[s]) {
      ha[s] = mix64(ha[s] + L[s]);
      hb[s] = mix64(hb[s] + L[s]);
    }
  }
}

// One tile of the split kernel for an item of the block-hash variant: the
// sign|mantissa stores, the blocks' hashes against the cached ones (d.hashes
// is the shard's hash cache, 16 bytes per block, updated in place), the tile's
// bitmap bytes, its count of changed blocks, and the exponent bytes of its
// changed blocks, B per block in block order, into its stash (T bytes: every
// block fits).
template <int DT, int S>
__device__ __forceinline__ void split_tile_block(const EncItem& d, uint32_t local, const EncArgs& a) {
  constexpr int E = Tr<DT>::E;
  constexpr uint32_t T = (uint32_t)kSub * S;
  constexpr int XW = 4 * E;
  __shared__ uint64_t s_hp[8 * S];
  __shared__ uint32_t s_flag[T / 64];  // changed flag per block of the tile (B >= 64)
  const uint32_t tid = threadIdx.x;
  const uint64_t base = (uint64_t)local * T;
  const uint64_t n = d.n;
  const uint32_t B = d.block_size;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;

  uint32_t xw[S][XW], expk[S][4];
  int cnt[S];
  uint64_t ch[S][2];  // cached hash of the block this thread leads
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
    cnt[s] = (int)left_in(n, c0, 16);
    if (cnt[s] > 0) load_words<XW, kNtBulk<DT>>(d.x + c0 * E, (uint32_t)cnt[s] * E, true, xw[s]);
    ch[s][0] = ch[s][1] = 0;
    if ((c0 & (B - 1)) == 0 && c0 < n) {
      const v4u h = ldg16(d.hashes + 16 * (c0 >> lb));
      ch[s][0] = h.x | ((uint64_t)h.y << 32);
      ch[s][1] = h.z | ((uint64_t)h.w << 32);
    }
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
    expk[s][0] = expk[s][1] = expk[s][2] = expk[s][3] = 0;
    if (cnt[s] > 0) {
      const uint32_t none[4] = {0, 0, 0, 0};
      (void)chunk_exps<DT, false>(xw[s], none, cnt[s], expk[s]);
      chunk_store<DT>(d.stream, c0, cnt[s], xw[s], true);
    }
  }
  bool lead[S];
  uint64_t ha[S], hb[S];
  tile_block_hashes<S>(expk, base, n, B, s_hp, lead, ha, hb);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (lead[s]) {
      const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
      const bool changed = ha[s] != ch[s][0] || hb[s] != ch[s][1];
      if (changed) {
        v4u h;
        h.x = (uint32_t)ha[s]; h.y = (uint32_t)(ha[s] >> 32);
        h.z = (uint32_t)hb[s]; h.w = (uint32_t)(hb[s] >> 32);
        stg16(d.hashes + 16 * (c0 >> lb), h);
      }
      s_flag[(uint32_t)(c0 - base) >> lb] = changed ? 1u : 0u;
    }
  }
  __syncthreads();
  const uint64_t in_tile = left_in(n, base, T);
  const uint32_t tblocks = (uint32_t)((in_tile + B - 1) >> lb);
  if (tid == 0) {
    uint32_t c = 0;
    for (uint32_t k = 0; k < tblocks; ++k) c += s_flag[k];
    gp(a.counts)[d.tile0 + local] = c;
  }
  // bitmap bytes, when a stream with a changed block can be BLOCK at all
  const uint64_t nb = (n + B - 1) >> lb;
  const uint64_t nbm = (nb + 7) / 8;
  const uint64_t smsec = sm_sec<DT>(n);
  if (smsec + nbm + B < n * E) {
    const uint32_t tbytes = (tblocks + 7) / 8;
    if (tid < tbytes) {
      uint32_t byte = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (tid * 8 + (uint32_t)k < tblocks && s_flag[tid * 8 + k]) byte |= 1u << k;
      gp(d.stream)[kHeader + smsec + (base >> (lb + 3)) + tid] = (uint8_t)byte;
    }
  }
  // the exponent bytes of the changed blocks into the stash, compacted
  uint8_t* st = reinterpret_cast<uint8_t*>(a.stash + d.stash + (uint64_t)local * d.cap);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
    const uint32_t blk = (uint32_t)(c0 - base) >> lb;
    if (blk < tblocks && s_flag[blk]) {
      uint32_t rank = 0;
      for (uint32_t k = 0; k < blk; ++k) rank += s_flag[k];
      v4u e;
      e.x = expk[s][0]; e.y = expk[s][1]; e.z = expk[s][2]; e.w = expk[s][3];
      stg16(st + (uint64_t)rank * B + ((uint32_t)(c0 - base) & (B - 1)), e);
    }
  }
}

// The hash cache of one shard (hash_update): every block's hash, one
// workgroup per tile of S rows.
template <int DT, int S>
__global__ __launch_bounds__(kThreads) void hash_seed_kernel(const uint8_t* __restrict__ x, uint8_t* hashes, uint64_t n,
                                                             uint32_t B) {
  constexpr int E = Tr<DT>::E;
  constexpr int XW = 4 * E;
  __shared__ uint64_t s_hp[8 * S];
  const uint32_t tid = threadIdx.x;
  const uint64_t base = (uint64_t)blockIdx.x * kSub * S;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;
  uint32_t xw[S][XW], expk[S][4];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
    const int cnt = (int)left_in(n, c0, 16);
    expk[s][0] = expk[s][1] = expk[s][2] = expk[s][3] = 0;
    if (cnt > 0) {
      load_words<XW>(x + c0 * E, (uint32_t)cnt * E, true, xw[s]);
      const uint32_t none[4] = {0, 0, 0, 0};
      (void)chunk_exps<DT, false>(xw[s], none, cnt, expk[s]);
    }
  }
  bool lead[S];
  uint64_t ha[S], hb[S];
  tile_block_hashes<S>(expk, base, n, B, s_hp, lead, ha, hb);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (lead[s]) {
      const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
      v4u h;
      h.x = (uint32_t)ha[s]; h.y = (uint32_t)(ha[s] >> 32);
      h.z = (uint32_t)hb[s]; h.w = (uint32_t)(hb[s] >> 32);
      stg16(hashes + 16 * (c0 >> lb), h);
    }
  }
}

// ------------------------------------------- entropy-coded patches (encode)
// [CIERA 3.1; Algorithm 1] the changed exponents travel ANS-coded.  Each chunk
// of 4096 values (a row of a tile, from the shard's first value) codes its c
// changes with range ANS over L = min(64, ceil(c/4)) interleaved 32-bit
// states, one per lane of one wave; change j goes to state j mod L.  Per
// change four symbols, in decode order: the gap bucket b = bit length of
// (gap + 1), gap = index - previous index - 1 (previous = -1 at the chunk
// start), with geometric-model frequencies for p = c / chunk length; the
// b - 1 bits of gap + 1 below its leading one; the exponent class (+1, -1,
// ..., +7, -7 modulo 256, or escape) from a fixed table; for an escape, the
// new exponent as 8 bits.  States stay in [2^16, 2^32) and trade 16-bit
// words: the decoder takes the changes L at a time and the four symbols as
// four sub-steps, after each of which every state below 2^16, in state
// order, takes the next word; the encoder runs the same sub-steps backwards
// from states of 2^16.  Chunk data = final states (u32) | words (u16) | a zero
// word when their number is odd.  A chunk with more than 1024 changes, or
// whose coded data is not shorter, goes dense: its exponent bytes, zero-padded
// to a multiple of 4.

constexpr uint32_t kChunkMaxChanges = 1024;
constexpr uint32_t kRansLow = 1u << 16;

__device__ __forceinline__ uint32_t pad4u(uint32_t v) { return (v + 3u) & ~3u; }
__device__ __forceinline__ uint32_t rans_lanes(uint32_t c) { return min(64u, (c + 3u) / 4u); }

// Length of the row starting at value r0 of a shard of n values (0 past it).
__device__ __forceinline__ uint32_t row_len(uint64_t n, uint64_t r0) { return (uint32_t)left_in(n, r0, kSub); }

// Bytes of a chunk's data from its changes, words and form.
__device__ __forceinline__ uint32_t coded_bytes(uint32_t c, uint32_t words, bool dense, uint32_t len) {
  if (c == 0) return 0;
  return dense ? pad4u(len) : 4u * rans_lanes(c) + 2u * words + 2u * (words & 1u);
}

// Gap-bucket frequencies (sum 2^12) for c changes among len values; lane i < 13
// of each group of GS lanes gets bucket i+1's frequency f and start cum (each
// group may hold its own c and len).  q = 1 - c/len in 32-bit fixed point;
// S_i = q^(2^i - 1) by repeated squaring (S_1 = q, S_{i+1} = S_i * q^(2^i)
// and q^(2^(i+1)) = (q^(2^i))^2, each product's high 32 bits); bucket b takes
// S_{b-1} - S_b (the last, S_12) as a share of 2^12, at least 1; the largest,
// first of equals, absorbs the rounding.  Wave-wide.
template <int GS = 64>
__device__ __forceinline__ void gap_table(uint32_t c, uint32_t len, uint32_t& f, uint32_t& cum) {
  const uint32_t lane = lane_id(), gl = lane & (GS - 1u);
  const uint32_t i = min(gl, 12u);
  // q < 2^32 as c >= 1 (a whole chunk, len = 2^12, needs no division)
  const uint32_t q = len == (uint32_t)kSub ? (len - c) << 20 : (uint32_t)(((uint64_t)(len - c) << 32) / len);
  uint32_t Q = q, S = q;  // S_1 and q^(2^0); lane i advances to S_i and q^(2^(i-1))
  for (uint32_t k = 1; k < i; ++k) {
    Q = __umulhi(Q, Q);
    S = __umulhi(S, Q);
  }
  const uint32_t Qn = i >= 1 ? __umulhi(Q, Q) : q;  // q^(2^i)
  uint64_t share;
  if (i == 0) share = (1ull << 32) - q;                      // S_0 - S_1
  else if (i < 12u) share = (uint64_t)S - __umulhi(S, Qn);  // S_i - S_{i+1}
  else share = S;                                            // S_12
  uint32_t fv = gl < 13u ? max(1u, (uint32_t)(share >> 20)) : 0u;
  uint32_t tot = fv, mx = fv;
#pragma unroll
  for (int o = GS / 2; o > 0; o >>= 1) {
    tot += __shfl_xor(tot, o, GS);
    mx = max(mx, __shfl_xor(mx, o, GS));
  }
  const uint64_t tops = __ballot(gl < 13u && fv == mx);
  const uint64_t mine = GS == 64 ? tops : (tops >> (lane - gl)) & ((1ull << (GS & 63)) - 1ull);
  if (gl == (uint32_t)__ffsll((unsigned long long)mine) - 1u) fv = fv + 4096u - tot;
  uint32_t incl = fv;
#pragma unroll
  for (int o = 1; o < GS; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, GS);
    if (gl >= (uint32_t)o) incl += t;
  }
  f = fv;
  cum = incl - fv;
}

// Exponent classes: +1 -> 0, -1 -> 1, +2 -> 2, ..., +7 -> 12, -7 -> 13 (mod
// 256), 14 escape; frequencies 2032, 2032, twelve of 2, 8 (sum 2^12).
__device__ __forceinline__ uint32_t delta_class(uint32_t oldv, uint32_t newv) {
  const uint32_t d = (newv - oldv) & 0xFFu;
  if (d >= 1u && d <= 7u) return 2u * (d - 1u);
  if (d >= 249u) return 2u * (255u - d) + 1u;
  return 14u;
}
__device__ __forceinline__ uint32_t class_step(uint32_t cls) {
  const uint32_t k = cls / 2u + 1u;
  return (cls & 1u) ? 256u - k : k;
}
__device__ __forceinline__ uint32_t class_freq(uint32_t cls) { return cls < 2u ? 2032u : (cls < 14u ? 2u : 8u); }
__device__ __forceinline__ uint32_t class_start(uint32_t cls) {
  return cls < 2u ? (cls ? 2032u : 0u) : (cls < 14u ? 4064u + 2u * (cls - 2u) : 4088u);
}
__device__ __forceinline__ uint32_t class_of_slot(uint32_t slot) {
  return slot < 2032u ? 0u : slot < 4064u ? 1u : slot < 4088u ? 2u + ((slot - 4064u) >> 1) : 14u;
}

// rANS-codes one chunk's c (1..1024) changes, listed in LDS in index order as
// offset | old exponent << 12 | new exponent << 20, with one wave (gap-bucket
// frequencies and starts from gap_table in gf and gcum), and returns the
// number of words.  The words go backwards from region_end (the end of the
// chunk's 4096-byte stash region), so they lie in decode order, and the final
// states just below them when the data fits the region; nothing is written
// below region_end - 4096.
__device__ uint32_t rans_encode_chunk(const uint32_t* list, uint32_t c, uint32_t gf, uint32_t gcum,
                                      uint8_t* region_end) {
  const uint32_t lane = lane_id();
  const uint32_t L = rans_lanes(c);
  uint32_t x = kRansLow;
  uint32_t R = 0;  // words written so far, counted from the end (uniform)
  // One sub-step, backwards: states about to code a symbol of frequency f
  // (scale s) write their low word first when x >= f * 2^(32 - s).
  auto step = [&](bool act, uint32_t start, uint32_t f, uint32_t sc, bool raw) {
    const bool emit = act && (uint64_t)x >= ((uint64_t)f << (32u - sc));
    const uint64_t m = __ballot(emit);
    const uint32_t cnt = (uint32_t)__popcll(m);
    if (emit) {
      const uint32_t pos = R + cnt - lanes_below(m);  // words from the end, lower lanes first in decode order
      if (2u * pos <= 4096u) gp(reinterpret_cast<uint16_t*>(region_end - 2u * pos))[0] = (uint16_t)x;
      x >>= 16;
    }
    R += cnt;
    if (act) x = raw ? ((x << sc) | start) : ((x / f) << sc) + (x % f) + start;
  };
  const uint32_t steps = (c + L - 1u) / L;
  for (int t = (int)steps - 1; t >= 0; --t) {  // uniform
    const uint32_t j = (uint32_t)t * L + lane;
    const bool act = lane < L && j < c;
    uint32_t e = 0, prev = 0xFFFFFFFFu;  // previous offset, -1 at the chunk start
    if (act) {
      e = list[j];
      if (j > 0) prev = list[j - 1] & 0xFFFu;
    }
    const uint32_t g1 = (e & 0xFFFu) - prev;  // gap + 1
    const uint32_t b = act ? 32u - (uint32_t)__clz(g1) : 1u;
    const uint32_t oldv = (e >> 12) & 0xFFu, newv = (e >> 20) & 0xFFu;
    const uint32_t cls = delta_class(oldv, newv);
    const uint32_t fb = __shfl(gf, (int)(b - 1u)), cb = __shfl(gcum, (int)(b - 1u));
    step(act && cls == 14u, newv, 1u, 8u, true);
    step(act, class_start(cls), class_freq(cls), 12u, false);
    step(act && b > 1u, g1 - (1u << (b - 1u)), 1u, b - 1u, true);
    step(act, cb, fb, 12u, false);
  }
  if (lane < L && 4u * L + 2u * R <= 4096u) {
    G1 uint16_t* q = gp(reinterpret_cast<uint16_t*>(region_end - 2u * R - 4u * L + 4u * lane));
    q[0] = (uint16_t)x;
    q[1] = (uint16_t)(x >> 16);
  }
  return R;
}

// One tile of the split kernel for an item with coded patches: sign|mantissa
// stores, the bitmap bytes, and per chunk row its data (coded by one wave, two
// rows at a time, or dense) in the row's stash region, its info word after
// the regions, and the tile's count (data bytes | changes << 16).
template <int DT, int S>
__device__ __forceinline__ void split_tile_coded(const EncItem& d, uint32_t local, const EncArgs& a) {
  constexpr int E = Tr<DT>::E;
  constexpr uint32_t T = (uint32_t)kSub * S;
  constexpr int XW = 4 * E;
  constexpr int P2 = S < 2 ? S : 2;  // rows coded at a time, one wave each
  __shared__ uint32_t s_list[P2][kChunkMaxChanges];
  __shared__ uint32_t s_wtot[4 * P2];
  __shared__ uint64_t s_chg[4 * S];
  __shared__ uint32_t s_info[S];
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint64_t base = (uint64_t)local * T;
  const uint64_t n = d.n;
  const uint32_t B = d.block_size;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;
  const bool caligned = d.cache_aligned != 0;
  uint8_t* const regions = reinterpret_cast<uint8_t*>(a.stash + d.stash + (uint64_t)local * d.cap);

  for (int s0 = 0; s0 < S; s0 += P2) {  // uniform
    uint32_t expk[P2][4], cw[P2][4], mask[P2], pre[P2];
#pragma unroll
    for (int r = 0; r < P2; ++r) {
      const uint64_t c0 = base + (uint64_t)(s0 + r) * kSub + (uint64_t)tid * kEPT;
      const int cnt = (int)left_in(n, c0, 16);
      uint32_t xw[XW];
      mask[r] = 0;
      expk[r][0] = expk[r][1] = expk[r][2] = expk[r][3] = 0;
      cw[r][0] = cw[r][1] = cw[r][2] = cw[r][3] = 0;
      if (cnt > 0) {
        load_words<XW, kNtBulk<DT>>(d.x + c0 * E, (uint32_t)cnt * E, true, xw);
        load_words<4, kNtBulk<DT>>(d.cache + c0, (uint32_t)cnt, caligned, cw[r]);
        mask[r] = chunk_exps<DT, false>(xw, cw[r], cnt, expk[r]);
        chunk_store<DT>(d.stream, c0, cnt, xw, true);
      }
      // exclusive prefix of the change counts over the workgroup, row by row
      const uint32_t cc = (uint32_t)__popc(mask[r]);
      uint32_t p = 0, tot = 0;
#pragma unroll
      for (int bit = 0; bit < 5; ++bit) {
        const uint64_t m = __ballot((cc >> bit) & 1u);
        p += lanes_below(m) << bit;
        tot += (uint32_t)__popcll(m) << bit;
      }
      pre[r] = p;
      const uint64_t chg = __ballot(mask[r] != 0);
      if (lane == 0) {
        s_wtot[r * 4 + wave] = tot;
        s_chg[(s0 + r) * 4 + wave] = chg;
      }
    }
    __syncthreads();
    uint32_t c[P2];
#pragma unroll
    for (int r = 0; r < P2; ++r) {
      c[r] = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (w < (int)wave) pre[r] += s_wtot[r * 4 + w];
        c[r] += s_wtot[r * 4 + w];
      }
      if (c[r] <= kChunkMaxChanges) {  // list the row's changes for its coding wave
        uint32_t m = mask[r], g = pre[r];
        while (m) {
          const int k = __ffs(m) - 1;
          m &= m - 1;
          s_list[r][g++] = (tid * kEPT + (uint32_t)k) | (byte_of(cw[r], k) << 12) | (byte_of(expk[r], k) << 20);
        }
      }
    }
    __syncthreads();
    if ((int)wave < P2) {  // uniform per wave: wave r codes row s0 + r
      const int r = (int)wave;
      const uint32_t len = row_len(n, base + (uint64_t)(s0 + r) * kSub);
      uint32_t words = 0;
      bool dense = c[r] > kChunkMaxChanges;
      if (c[r] > 0 && !dense) {  // coded into the region's end (writes past its start are dropped)
        uint32_t gf, gcum;
        gap_table(c[r], len, gf, gcum);
        words = rans_encode_chunk(s_list[r], c[r], gf, gcum, regions + (uint32_t)(s0 + r + 1) * kSub);
        dense = coded_bytes(c[r], words, false, len) >= pad4u(len);  // then the dense bytes below replace it
      }
      if (lane == 0) s_info[s0 + r] = c[r] | (dense ? 0u : words << 13) | ((dense ? 1u : 0u) << 26);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < P2; ++r) {  // dense rows: their exponent bytes (zero past the shard)
      if ((s_info[s0 + r] >> 26) & 1u) {
        v4u e;
        e.x = expk[r][0]; e.y = expk[r][1]; e.z = expk[r][2]; e.w = expk[r][3];
        stg16(regions + (uint32_t)(s0 + r) * kSub + tid * kEPT, e);
      }
    }
    __syncthreads();  // s_list and s_wtot are rewritten by the next rows
  }

  // bitmap bytes of the tile's blocks (a tile spans whole bitmap bytes), when
  // they lie inside the RAW length (otherwise the stream cannot be coded)
  const uint64_t smsec = sm_sec<DT>(n);
  const uint64_t in_tile = left_in(n, base, T);
  const uint32_t tblocks = (uint32_t)((in_tile + B - 1) >> lb);
  const uint64_t nbm = (((n + B - 1) >> lb) + 7) / 8;
  if (smsec + nbm <= n * E && tid < (tblocks + 7) / 8) {
    const uint32_t Lc = B >> 4;  // 16-value groups per block, >= 4
    uint32_t byte = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t blk = tid * 8 + (uint32_t)k;
      if (blk < tblocks) {
        const uint32_t first = blk * Lc;
        uint64_t any;
        if (Lc < 64) {
          any = (s_chg[first >> 6] >> (first & 63u)) & ((1ull << Lc) - 1ull);
        } else {
          any = 0;
          for (uint32_t u = 0; u < Lc / 64; ++u) any |= s_chg[(first >> 6) + u];
        }
        if (any) byte |= 1u << k;
      }
    }
    gp(d.stream)[kHeader + smsec + (base >> (lb + 3)) + tid] = (uint8_t)byte;
  }
  if (tid < (uint32_t)S) gp(reinterpret_cast<uint32_t*>(regions + T))[tid] = s_info[tid];
  if (tid == 0) {
    uint32_t bytes = 0, chg = 0;
#pragma unroll
    for (int r = 0; r < S; ++r) {
      const uint32_t len = row_len(n, base + (uint64_t)r * kSub);
      const uint32_t w = s_info[r];
      bytes += coded_bytes(w & 0x1FFFu, (w >> 13) & 0x1FFFu, (w >> 26) & 1u, len);
      chg += w & 0x1FFFu;
    }
    gp(a.counts)[d.tile0 + local] = bytes | (chg << 16);
  }
}

// The 64-byte stream header (little-endian): "CIER", version 1, dtype, mode
// (0 RAW, 1 COMPRESSED, 2 BLOCK), block size, n, changed values (blocks for
// BLOCK) P, total length, offset, rank, world.
template <int DT>
__device__ __forceinline__ void write_header(const EncItem& d, uint64_t P, uint32_t mode, uint64_t total) {
  uint32_t h[16];
  h[0] = 0x52454943u;  // "CIER"
  h[1] = 1u | ((uint32_t)DT << 16) | (mode << 24);
  h[2] = d.block_size;
  h[3] = 0;
  h[4] = (uint32_t)d.n; h[5] = (uint32_t)(d.n >> 32);
  h[6] = (uint32_t)P; h[7] = (uint32_t)(P >> 32);
  h[8] = (uint32_t)total; h[9] = (uint32_t)(total >> 32);
  h[10] = (uint32_t)d.off; h[11] = (uint32_t)(d.off >> 32);
  h[12] = d.rank; h[13] = d.world; h[14] = 0; h[15] = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v4u o;
    o.x = h[4 * q]; o.y = h[4 * q + 1]; o.z = h[4 * q + 2]; o.w = h[4 * q + 3];
    stg16(d.stream + 16 * q, o);
  }
}

// dst[b] = src[b] for b in [lo, hi), by the whole workgroup; dst and src have
// the same alignment modulo 16 (16-byte pieces between byte-wise ends).
__device__ __forceinline__ void copy_bytes(uint8_t* dst, const uint8_t* src, uint64_t lo, uint64_t hi) {
  const uint32_t tid = threadIdx.x;
  const uint64_t a = min(hi, (lo + 15) & ~15ull), e = max(a, hi & ~15ull);
  for (uint64_t b = lo + tid; b < a; b += kThreads) gp(dst)[b] = gp(src)[b];
  for (uint64_t q = a / 16 + tid; q < e / 16; q += kThreads) stg16(dst + 16 * q, ldg16(src + 16 * q));
  for (uint64_t b = e + tid; b < hi; b += kThreads) gp(dst)[b] = gp(src)[b];
}

// ------------------------------------------- encode, tiles that finish themselves
// Element patches and RAW (compress 0 or 1) of items of at most kSelfTiles
// tiles.  After the compare each tile publishes its change count in its slot
// of the batch's sync array -- one 64-bit word, epoch << 32 | count, written
// with a device-scope atomic -- and waits until every tile of its item has
// published in this launch's epoch.  The counts give the item's total, hence
// the mode [CIERA 3.2: compressed only when smaller], and the tile's exclusive
// prefix, hence where its records go.  The tile stores each row's
// sign|mantissa bytes as soon as the row is compared (their place does not
// depend on the counts); once the
// mode is known it stores its bitmap bytes and its records, and tile 0 the
// header.  When the total makes the stream RAW although the plan compressed it
// (rare), every tile rewrites the bytes of the raw body it owns -- those its
// sign|mantissa stores went to, and an even share of the rest -- so that no
// byte has two writers and no second launch finishes the stream.
//
// The epoch is the tile's own slot's previous epoch plus one: every launch
// advances every slot of the item by one (the slots are zeroed when the batch
// is prepared), so the tiles of an item agree on it without a host value, and
// a replayed launch never mistakes the last launch's counts for its own.  The
// tiles of an item are consecutive workgroups and publish before they wait, so
// a waiting tile needs only its siblings to be dispatched: at most
// kSelfTiles / 8 + 1 of them share an XCD, far fewer than an XCD runs at once.
// The wait is a shortcut, not a dependency: after `polls` polls of a slot
// (EncArgs::polls) a tile counts that sibling's changes itself from the shard
// and the cache, so it finishes with the same result however the workgroups
// are scheduled.
constexpr uint32_t kSelfPolls = 1u << 16;  // default bound, about a millisecond

// Changes of tile k of item d (tvals values per tile), counted by the whole
// workgroup from the shard and the cache one value per thread at a time (a
// rare path, kept small so that it costs the kernel no registers).  Contains
// two barriers.
template <int DT>
__device__ __forceinline__ uint32_t tile_changes(const EncItem& d, uint64_t k, uint32_t* s_red) {
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint64_t v0 = k * d.tvals, v1 = min<uint64_t>(d.n, v0 + d.tvals);
  uint32_t c = 0;
  for (uint64_t i = v0 + tid; i < v1; i += kThreads) {
    const uint32_t v = Tr<DT>::E == 2 ? (uint32_t)gp(reinterpret_cast<const uint16_t*>(d.x))[i]
                                      : gp(reinterpret_cast<const uint32_t*>(d.x))[i];
    c += exp_of<DT>(v) != (uint32_t)gp(d.cache)[i] ? 1u : 0u;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  __syncthreads();  // s_red is free
  if (lane == 0) s_red[wave] = c;
  __syncthreads();
  return s_red[0] + s_red[1] + s_red[2] + s_red[3];
}

template <int DT, int S>
__device__ __forceinline__ void split_tile_self(const EncItem& d, uint32_t local, const EncArgs& a) {
  constexpr int E = Tr<DT>::E;
  constexpr uint32_t T = (uint32_t)kSub * S;
  constexpr int XW = 4 * E;  // words of 16 raw values
  __shared__ uint32_t s_wtot[4 * S];
  __shared__ uint64_t s_chg[4 * S];  // one bit per 16-value chunk of the tile, in value order
  __shared__ uint32_t s_sum[2];      // the item's changes, those of the tiles before
  __shared__ uint32_t s_miss[kSelfTiles / 32];  // tiles whose counts did not come in time
  __shared__ uint32_t s_red[kThreads / 64];
  __shared__ uint32_t s_stage[kThreads / 64][kXWaveRow<DT> / 4];  // each wave's exchange of pieces

  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint64_t base = (uint64_t)local * T;
  const uint64_t n = d.n;
  const uint32_t B = d.block_size;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;  // B is a power of two (checked by the API)
  uint64_t* const sync = a.sync + d.tile0;      // the item's slots
  uint64_t mine_old = 0;                        // this tile's slot as the last launch left it
  if (tid == 0) mine_old = __hip_atomic_load(sync + local, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // loads, split and compare, row by row: a wave loads its 1024 values of a
  // row as contiguous pieces (those past the shard as zeros) and swaps them
  // through LDS into each lane's 16 values; the row's sign|mantissa words are
  // stored as soon as it is compared (a RAW stream reads its values again).
  uint32_t mask[S], expk[S][4];
  uint32_t smw[DT == 1 ? 1 : S][kSmWords<DT>];  // fp32/fp16: the records, kept for the stores below
  int cnt[S];
  bool whole[S];  // uniform per wave
  {
    uint32_t cw[S][4];
    v4u pc[S][E];
    const bool full = d.cache_aligned != 0 && base + T <= n;  // uniform
    // Rows are loaded AH ahead of the one compared, so that a wave holds the
    // raw words of at most AH + 1 rows at a time (registers for occupancy)
    // while keeping that many rows of loads in flight.
    constexpr int AH = S < 2 ? S : 2;
    auto issue = [&](int s) {
      const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
      const uint64_t w0 = base + (uint64_t)s * kSub + (uint64_t)wave * 1024u;
      whole[s] = w0 + 1024u <= n;
      cnt[s] = full ? 16 : ((int)left_in(n, c0, 16));
      if (whole[s]) load_x_pieces<DT>(d.x + w0 * E, pc[s]);
      else load_x_pieces_upto<DT>(d.x + w0 * E, (uint32_t)left_in(n, w0, 1024u) * E, pc[s]);
      if (cnt[s] > 0) load_words<4, true>(d.cache + c0, (uint32_t)cnt[s], full || d.cache_aligned != 0, cw[s]);
    };
#pragma unroll
    for (int s = 0; s < AH; ++s) issue(s);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (s + AH < S) issue(s + AH);
      __builtin_amdgcn_sched_barrier(0);
      uint32_t xw[XW];
      swap_x_pieces<DT>(&s_stage[wave][0], pc[s], xw);
      mask[s] = 0;
      expk[s][0] = expk[s][1] = expk[s][2] = expk[s][3] = 0;
      if (full) mask[s] = chunk_exps<DT, true>(xw, cw[s], 16, expk[s]);
      else if (cnt[s] > 0) mask[s] = chunk_exps<DT, false>(xw, cw[s], cnt[s], expk[s]);
      if constexpr (DT == 1) {
        // bf16: the row's sign|mantissa bytes go out now, lane by lane (a
        // COMPRESSED stream keeps them; a RAW one, rare, is rewritten below
        // by the tiles that own its bytes)
        if (d.compress != 0 && cnt[s] > 0) {
          chunk_sm_words<DT>(xw, smw[0]);
          store_sm_words<DT>(d.stream + kHeader + sm_off<DT>(base + (uint64_t)s * kSub + (uint64_t)tid * kEPT),
                             cnt[s], smw[0]);
        }
      } else {
        chunk_sm_words<DT>(xw, smw[s]);
      }
    }
  }

  // the tile's change count, chunk-row major (= ascending value index)
  uint32_t lpre[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint64_t chg = __ballot(mask[s] != 0);
    const uint32_t c = (uint32_t)__popc(mask[s]);
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {
      const uint64_t m = __ballot((c >> b) & 1u);
      pre += lanes_below(m) << b;
      tot += (uint32_t)__popcll(m) << b;
    }
    lpre[s] = pre;
    if (lane == 0) {
      s_wtot[s * 4 + wave] = tot;
      s_chg[s * 4 + wave] = chg;
    }
  }
  if (tid < kSelfTiles / 32) s_miss[tid] = 0;
  __syncthreads();
  uint32_t agg = 0, before[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t t = s_wtot[s * 4 + w];
      if (w == (int)wave) before[s] = agg;
      agg += t;
    }
  }

  // publish (wave 0)
  uint32_t epoch = 0;
  if (wave == 0) {
    epoch = __shfl((uint32_t)(mine_old >> 32), 0) + 1u;
    if (lane == 0)
      __hip_atomic_store(sync + local, ((uint64_t)epoch << 32) | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // fp32/fp16: the records go out now, while the siblings' counts come in,
  // whole rows put together in LDS (the same buffer as the value swaps, so
  // not between them)
  if constexpr (DT != 1) {
    if (d.compress != 0) {  // uniform
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
        if (whole[s])
          store_sm_pieces<DT>(d.stream + kHeader + sm_off<DT>(base + (uint64_t)s * kSub + (uint64_t)wave * 1024u),
                              &s_stage[wave][0], smw[s]);
        else if (cnt[s] > 0)
          store_sm_words<DT>(d.stream + kHeader + sm_off<DT>(c0), cnt[s], smw[s]);
      }
    }
  }
  // wait for the item's other tiles (wave 0, lanes over tiles)
  if (wave == 0) {
    const uint32_t polls = a.polls ? a.polls : kSelfPolls;
    uint32_t tot = 0, pre = 0;
    for (uint32_t k = lane; k < d.tpi; k += 64) {
      uint64_t v = 0;
      bool got = false;
      for (uint32_t i = 0; i < polls; ++i) {
        v = __hip_atomic_load(sync + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(v >> 32) == epoch) {
          got = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (got) {
        tot += (uint32_t)v;
        pre += k < local ? (uint32_t)v : 0u;
      } else {
        atomicOr(&s_miss[k >> 5], 1u << (k & 31u));
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      tot += __shfl_xor(tot, o);
      pre += __shfl_xor(pre, o);
    }
    if (lane == 0) {
      s_sum[0] = tot;
      s_sum[1] = pre;
    }
  }
  __syncthreads();
  uint32_t tot_miss = 0, pre_miss = 0;  // the late tiles, counted here
  for (uint32_t w = 0; w < (d.tpi + 31) / 32; ++w) {  // uniform
    uint32_t m = s_miss[w];
    while (m) {
      const uint32_t k = 32 * w + (uint32_t)__ffs(m) - 1u;
      m &= m - 1;
      const uint32_t ck = tile_changes<DT>(d, k, s_red);
      tot_miss += ck;
      pre_miss += k < local ? ck : 0u;
    }
  }
  const uint64_t P = (uint64_t)s_sum[0] + tot_miss;
  const uint32_t excl = s_sum[1] + pre_miss;
  const uint64_t nbm = (((n + B - 1) >> lb) + 7) / 8;
  const uint64_t smsec = sm_sec<DT>(n);
  const uint64_t comp = kHeader + smsec + (P ? nbm + 5 * P : 0);
  const uint64_t raw = kHeader + n * E;
  const bool cmode = d.compress != 0 && comp < raw;

  if (d.compress == 0) {  // RAW by plan: the values as stored
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
      if (cnt[s] > 0) {
        uint32_t rw[XW];
        load_words<XW>(d.x + c0 * E, (uint32_t)cnt[s] * E, true, rw);
        store_words<XW>(d.stream + kHeader + c0 * E, (uint32_t)cnt[s] * E, true, rw);
      }
    }
  } else if (!cmode) {
    // RAW although planned compressed: the raw body (the shard's bytes) is
    // split between the tiles so that each byte has one writer -- tile k
    // takes the bytes its records went to above, [sm_off(kT), sm_off((k+1)T)),
    // and an even share of the rest, [S + kD, S + (k+1)D) with S the record
    // section's bytes.  Its own record stores are complete first (barrier).
    __syncthreads();
    const uint64_t rb = n * E;
    const uint64_t r1 = local + 1 < d.tpi ? sm_off<DT>(base + T) : smsec;
    const uint64_t D = ((rb - smsec + d.tpi - 1) / d.tpi + 15) & ~15ull;
    copy_bytes(d.stream + kHeader, d.x, sm_off<DT>(base), r1);
    copy_bytes(d.stream + kHeader, d.x, min(rb, smsec + local * D), min(rb, smsec + (local + 1) * D));
  }
  if (local == 0 && tid == 0) write_header<DT>(d, P, cmode ? 1u : 0u, cmode ? comp : raw);
  if (!cmode || P == 0) return;

  // the tile's bitmap bytes (a tile spans whole bitmap bytes)
  const uint64_t in_tile = left_in(n, base, T);
  const uint32_t tblocks = (uint32_t)((in_tile + B - 1) >> lb);
  const uint32_t tbytes = (tblocks + 7) / 8;
  if (tid < tbytes) {
    const uint32_t L = B >> 4;  // chunks per block, >= 4
    uint32_t byte = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t blk = tid * 8 + (uint32_t)k;
      if (blk < tblocks) {
        const uint32_t first = blk * L;
        uint64_t any;
        if (L < 64) {
          any = (s_chg[first >> 6] >> (first & 63u)) & ((1ull << L) - 1ull);
        } else {
          any = 0;
          for (uint32_t u = 0; u < L / 64; ++u) any |= s_chg[(first >> 6) + u];
        }
        if (any) byte |= 1u << k;
      }
    }
    gp(d.stream)[kHeader + smsec + (base >> (lb + 3)) + tid] = (uint8_t)byte;
  }

  // the tile's records at their places in the patch list (all inside comp)
  const uint64_t pbase = kHeader + smsec + nbm;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint64_t g = (uint64_t)excl + before[s] + lpre[s];
    put_records(d.stream, pbase + 5 * g, mask[s], (uint32_t)(base + (uint64_t)s * kSub + tid * kEPT), expk[s]);
  }
}

// Groups of items whose tiles finish their own streams (element patches and
// RAW of at most kSelfTiles tiles; a launch group holds no other items) take a
// kernel of their own, so that its registers and occupancy are those of that
// path alone (the other paths of encode_kernel need more).
template <int DT, int S>
__global__ __launch_bounds__(kThreads) void encode_self_kernel(EncArgs a, uint32_t batch_id) {
  const uint32_t rel_item = blockIdx.x / a.tpi;
  const uint32_t item = a.item0 + rel_item;
  const uint32_t local = blockIdx.x - rel_item * a.tpi;
  const EncItem d = a.items[item];
  if (d.batch_id != batch_id) return;  // the scratch holds another batch (uniform)
  split_tile_self<DT, S>(d, local, a);
}

template <int DT, int S>
__global__ __launch_bounds__(kThreads) void encode_kernel(EncArgs a, uint32_t batch_id) {
  constexpr int E = Tr<DT>::E;
  constexpr uint32_t T = (uint32_t)kSub * S;
  constexpr int XW = 4 * E;  // words of 16 raw values
  __shared__ uint32_t s_wtot[4 * S];
  __shared__ uint64_t s_chg[4 * S];  // one bit per 16-value chunk of the tile, in value order

  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint32_t rel_item = blockIdx.x / a.tpi;
  const uint32_t item = a.item0 + rel_item;
  const uint32_t local = blockIdx.x - rel_item * a.tpi;
  const EncItem d = a.items[item];
  if (d.batch_id != batch_id) return;  // the scratch holds another batch (uniform)
  if (d.compress == kBlockVariant) {   // uniform
    split_tile_block<DT, S>(d, local, a);
    return;
  }
  if (d.compress == kCoded) {  // uniform
    split_tile_coded<DT, S>(d, local, a);
    return;
  }
  const uint64_t base = (uint64_t)local * T;
  const uint64_t n = d.n;
  const uint32_t B = d.block_size;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;  // B is a power of two (checked by the API)
  const bool compress = d.compress != 0;
  const bool caligned = d.cache_aligned != 0;

  // Loads, split and compare, sign|mantissa (or RAW) stores.  A tile wholly
  // inside its item with an aligned cache takes a straight-line copy of this
  // code (FULL: every chunk has 16 values).
  uint32_t mask[S];
  uint32_t expk[S][4];
  auto split_tile = [&](auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    uint32_t xw[S][XW], cw[S][4];
    int cnt[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {  // all loads of the tile first
      const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
      cnt[s] = FULL ? 16 : ((int)left_in(n, c0, 16));
      if (cnt[s] > 0) {
        load_words<XW, kNtBulk<DT>>(d.x + c0 * E, (uint32_t)cnt[s] * E, true, xw[s]);
        load_words<4, kNtBulk<DT>>(d.cache + c0, (uint32_t)cnt[s], FULL || caligned, cw[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint64_t c0 = base + (uint64_t)s * kSub + (uint64_t)tid * kEPT;
      mask[s] = 0;
      expk[s][0] = expk[s][1] = expk[s][2] = expk[s][3] = 0;
      if (cnt[s] > 0) {
        mask[s] = chunk_exps<DT, FULL>(xw[s], cw[s], cnt[s], expk[s]);
        chunk_store<DT>(d.stream, c0, cnt[s], xw[s], compress);
      }
    }
  };
  if (caligned && base + T <= n) split_tile(std::true_type{});  // uniform
  else split_tile(std::false_type{});

  // chunk change flags for the bitmap; block-wide exclusive scan of the
  // per-thread change counts, chunk-row major (= ascending value index)
  uint32_t lpre[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint64_t chg = __ballot(mask[s] != 0);
    const uint32_t c = (uint32_t)__popc(mask[s]);
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {
      const uint64_t m = __ballot((c >> b) & 1u);
      pre += lanes_below(m) << b;
      tot += (uint32_t)__popcll(m) << b;
    }
    lpre[s] = pre;
    if (lane == 0) {
      s_wtot[s * 4 + wave] = tot;
      s_chg[s * 4 + wave] = chg;
    }
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
  if (tid == 0) gp(a.counts)[d.tile0 + local] = agg;
  if (!compress) return;

  // bitmap bytes of this tile's blocks (a tile spans whole bitmap bytes), when
  // a stream with a change can be COMPRESSED at all (otherwise it is never read)
  const uint64_t nb = (n + B - 1) >> lb;
  const uint64_t nbm = (nb + 7) / 8;
  const uint64_t smsec = sm_sec<DT>(n);
  if (smsec + nbm + 5 <= n * E) {
    const uint64_t in_tile = left_in(n, base, T);
    const uint32_t tblocks = (uint32_t)((in_tile + B - 1) >> lb);
    const uint32_t tbytes = (tblocks + 7) / 8;
    if (tid < tbytes) {
      const uint32_t L = B >> 4;  // chunks per block, >= 4
      uint32_t byte = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t blk = tid * 8 + (uint32_t)k;
        if (blk < tblocks) {
          const uint32_t first = blk * L;
          uint64_t any;
          if (L < 64) {
            any = (s_chg[first >> 6] >> (first & 63u)) & ((1ull << L) - 1ull);
          } else {
            any = 0;
            for (uint32_t u = 0; u < L / 64; ++u) any |= s_chg[(first >> 6) + u];
          }
          if (any) byte |= 1u << k;
        }
      }
      gp(d.stream)[kHeader + smsec + (base >> (lb + 3)) + tid] = (uint8_t)byte;
    }
  }

  // the tile's first cap changes, ascending, into its stash
  G1 uint32_t* st = gp(a.stash + d.stash + (uint64_t)local * d.cap);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    uint32_t m = mask[s];
    uint32_t g = before[s] + lpre[s];
    const uint32_t rel0 = (uint32_t)s * kSub + tid * kEPT;
    while (m) {
      const int j = __ffs(m) - 1;
      m &= m - 1;
      if (g < d.cap) st[g] = (rel0 + (uint32_t)j) | (byte_of(expk[s], j) << 16);
      ++g;
    }
  }
}

// Tiles per window of the finishing kernel: counts are scanned in LDS a window
// at a time.
constexpr uint32_t kWin = 1024;
constexpr uint64_t kGridMax = 64;  // decode: longest patch list searched from a plain grid (one round)

// Writes the patch records of tile j of item d (tvals values) again from the
// shard and the cache, the first one as record number r0.  Workgroup-wide.
template <int DT>
__device__ void rederive_tile(const EncItem& d, uint64_t j, uint32_t r0, uint64_t pbase, uint32_t* s_red) {
  constexpr int E = Tr<DT>::E;
  constexpr int XW = 4 * E;
  const uint32_t tid = threadIdx.x;
  uint32_t run = r0;
  for (uint32_t row = 0; row < d.tvals / kSub; ++row) {  // uniform
    const uint64_t c0 = j * d.tvals + (uint64_t)row * kSub + (uint64_t)tid * kEPT;
    const int cnt = (int)left_in(d.n, c0, 16);
    uint32_t xw[XW], cw[4], expk[4], mask = 0;
    if (cnt > 0) {
      load_words<XW>(d.x + c0 * E, (uint32_t)cnt * E, true, xw);
      load_words<4>(d.cache + c0, (uint32_t)cnt, d.cache_aligned != 0, cw);
      mask = chunk_exps<DT, false>(xw, cw, cnt, expk);
    }
    uint32_t tot;
    uint32_t g = run + block_scan<uint32_t>((uint32_t)__popc(mask), s_red, tot);
    while (mask) {
      const int k = __ffs(mask) - 1;
      mask &= mask - 1;
      put_record(d.stream, d.capacity, pbase + 5ull * g, (uint32_t)(c0 + k), byte_of(expk, k));
      ++g;
    }
    run += tot;
    __syncthreads();  // s_red is read before it is written again
  }
}

// Raw body bytes [b0, b1) of the shard copied into the stream (b0 a multiple
// of 16); this is thread gt of gs copying.
__device__ __forceinline__ void raw_copy(const EncItem& d, uint64_t b0, uint64_t b1, uint64_t gt, uint64_t gs) {
  const uint64_t v1 = b0 + (b1 - b0) / 16 * 16;
  for (uint64_t i = b0 + 16 * gt; i < v1; i += 16 * gs) stg16(d.stream + kHeader + i, ldg16(d.x + i));
  for (uint64_t i = v1 + gt; i < b1; i += gs) gp(d.stream)[kHeader + i] = gp(d.x)[i];
}

// len bytes (a multiple of 16) from a 16-byte aligned source to dst at any
// alignment; thread gt of gs.
__device__ __forceinline__ void copy_to_stream(uint8_t* dst, const uint8_t* src, uint64_t len, uint64_t gt,
                                               uint64_t gs) {
  const uint32_t a = (uint32_t)(reinterpret_cast<uintptr_t>(dst) & 15u);
  for (uint64_t i = gt; i < len / 16; i += gs) {
    const v4u v = ldg16(src + 16 * i);
    uint8_t* q = dst + 16 * i;
    if (a == 0) {
      stg16(q, v);
    } else if ((a & 3u) == 0) {
      G1 uint32_t* w = gp(reinterpret_cast<uint32_t*>(q));
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
      const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int b = 0; b < 16; ++b) gp(q)[b] = (uint8_t)(x[b >> 2] >> (8 * (b & 3)));
    }
  }
}

// LDS of one item's finishing work.
struct FinLds {
  uint32_t pre[kWin + 1];  // exclusive prefix of the window's tile counts, then its total
  uint32_t ovf[kWin];      // window tiles whose changes overflowed their stash
  uint64_t red64[kThreads / 64];
  uint32_t red[kThreads / 64];
};

// Finishing work of item d by workgroup g of G: the sum of its tile counts
// decides the mode; workgroup 0 writes the header; the stashed changes go to
// their places in the patch list (tiles that overflowed their stash derive
// theirs again), or the stream is rewritten RAW.  Workgroup-wide.
template <int DT>
__device__ void finish_item(const EncItem& d, const uint32_t* counts, const uint32_t* stash, uint32_t G, uint32_t g,
                            FinLds& L) {
  constexpr int E = Tr<DT>::E;
  const uint32_t tid = threadIdx.x;
  const uint32_t tpi = d.tpi;
  const G1 uint32_t* cnts = gp(counts + d.tile0);

  // Scans one window of tile counts into L.pre (and its overflowing tiles
  // into L.ovf); returns the window total and the number of overflowing
  // tiles.  `rest` adds the counts past the first window (first call only).
  auto scan_window = [&](uint32_t w0, bool with_rest, uint32_t& novf, uint32_t& rest_total) -> uint32_t {
    const uint32_t nw = min(kWin, tpi - w0);
    uint32_t c4[4], sum = 0, nov = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t i = tid * 4 + (uint32_t)k;
      c4[k] = i < nw ? cnts[w0 + i] : 0u;
      sum += c4[k];
      nov += c4[k] > d.cap ? 1u : 0u;
    }
    uint32_t rest = 0;
    if (with_rest)
      for (uint32_t i = kWin + tid; i < tpi; i += kThreads) rest += cnts[i];
    uint64_t tot64;
    const uint64_t ex = block_scan<uint64_t>((uint64_t)sum | ((uint64_t)nov << 32), L.red64, tot64);
    uint32_t rt = 0;
    if (with_rest && tpi > kWin) (void)block_scan<uint32_t>(rest, L.red, rt);
    uint32_t pre = (uint32_t)ex, o = (uint32_t)(ex >> 32);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t i = tid * 4 + (uint32_t)k;
      if (i < nw) {
        L.pre[i] = pre;
        if (c4[k] > d.cap) L.ovf[o++] = i;
      }
      pre += c4[k];
    }
    if (tid == 0) L.pre[nw] = (uint32_t)tot64;
    __syncthreads();
    novf = (uint32_t)(tot64 >> 32);
    rest_total = rt;
    return (uint32_t)tot64;
  };

  uint32_t novf, rest;
  const uint32_t wtot0 = scan_window(0, true, novf, rest);
  const uint64_t P = (uint64_t)wtot0 + rest;
  const uint64_t n = d.n;
  const uint32_t B = d.block_size;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;
  const uint64_t nbm = (((n + B - 1) >> lb) + 7) / 8;
  const uint64_t smsec = sm_sec<DT>(n);
  const uint64_t comp = kHeader + smsec + (P ? nbm + 5 * P : 0);
  const uint64_t raw = kHeader + n * E;
  const bool cmode = d.compress != 0 && comp < raw;

  if (d.compress == kBlockVariant) {  // uniform: block-hash variant, counts are changed blocks
    const uint64_t bcomp = kHeader + smsec + (P ? nbm + P * B : 0);
    const bool bmode = bcomp < raw;
    if (g == 0 && tid == 0) write_header<DT>(d, P, bmode ? kBlockVariant : 0u, bmode ? bcomp : raw);
    if (!bmode) {
      raw_copy(d, 0, n * E, (uint64_t)g * kThreads + tid, (uint64_t)G * kThreads);
      return;
    }
    uint32_t run = 0;  // changed blocks before the window
    for (uint32_t w0 = 0; P > 0 && w0 < tpi; w0 += kWin) {  // uniform
      uint32_t wtot = wtot0;
      if (w0 > 0) {
        __syncthreads();  // the previous window's LDS is no longer read
        wtot = scan_window(w0, false, novf, rest);
      }
      const uint32_t nw = min(kWin, tpi - w0);
      for (uint32_t i = g; i < nw; i += G) {  // this workgroup's tiles of the window
        const uint32_t c = L.pre[i + 1] - L.pre[i];
        if (c)
          copy_to_stream(d.stream + kHeader + smsec + nbm + (uint64_t)(run + L.pre[i]) * B,
                         reinterpret_cast<const uint8_t*>(stash + d.stash + ((uint64_t)w0 + i) * d.cap), (uint64_t)c * B,
                         tid, kThreads);
      }
      run += wtot;
    }
    return;
  }
  if (g == 0 && tid == 0) write_header<DT>(d, P, cmode ? 1u : 0u, cmode ? comp : raw);
  if (d.compress != 0 && !cmode) {  // the compressed form is not shorter: RAW
    raw_copy(d, 0, n * E, (uint64_t)g * kThreads + tid, (uint64_t)G * kThreads);
    return;
  }
  if (!cmode || P == 0) return;  // RAW as planned (written by encode_kernel), or no patches

  const uint64_t pbase = kHeader + smsec + nbm;
  uint32_t run = 0;  // records before the window
  for (uint32_t w0 = 0; w0 < tpi; w0 += kWin) {  // uniform
    uint32_t wtot = wtot0;
    if (w0 > 0) {
      __syncthreads();  // the previous window's LDS is no longer read
      wtot = scan_window(w0, false, novf, rest);
    }
    const uint32_t nw = min(kWin, tpi - w0);
    for (uint32_t r0 = g * kThreads; r0 < wtot; r0 += G * kThreads) {
      const uint32_t r = r0 + tid;
      if (r < wtot) {
        uint32_t lo = 0, hi = nw;  // L.pre[lo] <= r < L.pre[hi]
        while (hi - lo > 1) {
          const uint32_t mid = (lo + hi) >> 1;
          if (L.pre[mid] <= r) lo = mid;
          else hi = mid;
        }
        const uint32_t k = r - L.pre[lo];
        if (L.pre[lo + 1] - L.pre[lo] <= d.cap) {
          const uint64_t j = (uint64_t)w0 + lo;
          const uint32_t v = gp(stash)[d.stash + j * d.cap + k];
          put_record(d.stream, d.capacity, pbase + 5ull * (run + r), (uint32_t)(j * d.tvals + (v & 0xFFFFu)),
                     v >> 16);
        }
      }
    }
    for (uint32_t u = 0; u < novf; ++u) {  // uniform
      const uint32_t i = L.ovf[u];
      if ((w0 + i) % G == g) rederive_tile<DT>(d, (uint64_t)w0 + i, run + L.pre[i], pbase, L.red);
    }
    run += wtot;
  }
}

// gridDim.x workgroups per item, items along y.
template <int DT>
__global__ __launch_bounds__(kThreads) void encode_finish_kernel(const EncItem* __restrict__ items, uint32_t item0,
                                                                 uint32_t nitems, const uint32_t* counts,
                                                                 const uint32_t* stash, uint32_t batch_id) {
  __shared__ FinLds s_fin;
  for (uint32_t it = blockIdx.y; it < nitems; it += gridDim.y) {
    __syncthreads();  // LDS of the previous item is no longer read
    const EncItem d = items[item0 + it];
    if (d.batch_id != batch_id) return;  // uniform
    finish_item<DT>(d, counts, stash, gridDim.x, blockIdx.x, s_fin);
  }
}

// Finishing work of one tile of an item with coded patches (at most kThreads
// tiles per item): the item's totals and this tile's prefix of data bytes and
// changes decide the mode and the places; the tile writes its chunks' table
// entries (changes and data bytes of this and all earlier chunks) and copies
// its chunks' data (coded data from the end of each stash region, a zero word
// after an odd number of words; dense data from its start), or its part of
// the shard RAW.  Workgroup-wide.
constexpr uint32_t kCodedFinishThreads = 64;  // one wave per coded tile in its finishing kernel
template <int DT>
__device__ void finish_tile_coded(const FinArgs& f, const EncItem& d, uint32_t local, uint64_t t0, uint64_t sbase) {
  constexpr int E = Tr<DT>::E;
  constexpr uint32_t NT = kCodedFinishThreads;
  __shared__ uint64_t s_r[2 * (NT / 64)];
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  // sb, sc: the item's data bytes and changes (low half) and those of the
  // tiles before this one (high half)
  uint64_t sb, sc;
  if (f.prefix) {  // items of more than kThreads tiles: prefixes from the scan kernel
    const G1 uint64_t* pre = gp(f.prefix + t0);
    const uint64_t mine = pre[local], last = pre[f.tpi - 1];
    const uint32_t c_last = gp(f.counts)[t0 + f.tpi - 1];
    sb = ((uint32_t)last + (c_last & 0xFFFFu)) | ((mine & 0xFFFFFFFFull) << 32);
    sc = ((uint32_t)(last >> 32) + (c_last >> 16)) | ((mine >> 32) << 32);
  } else {  // at most kThreads tiles: the thread's share of them, then a reduction
    uint64_t vb = 0, vc = 0;
    for (uint32_t k = tid; k < f.tpi; k += NT) {
      const uint32_t c_t = gp(f.counts)[t0 + k];
      const uint32_t by = c_t & 0xFFFFu, ch = c_t >> 16;
      vb += by | ((uint64_t)(k < local ? by : 0u) << 32);
      vc += ch | ((uint64_t)(k < local ? ch : 0u) << 32);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      vb += __shfl_xor(vb, o);
      vc += __shfl_xor(vc, o);
    }
    if (lane == 0) {
      s_r[wave] = vb;
      s_r[NT / 64 + wave] = vc;
    }
    __syncthreads();
    sb = sc = 0;
#pragma unroll
    for (int w = 0; w < (int)(NT / 64); ++w) {
      sb += s_r[w];
      sc += s_r[NT / 64 + w];
    }
  }
  const uint64_t Dtot = (uint32_t)sb, P = (uint32_t)sc;
  const uint64_t n = d.n;
  const uint32_t B = d.block_size;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;
  const uint64_t nbm = (((n + B - 1) >> lb) + 7) / 8;
  const uint64_t smsec = sm_sec<DT>(n);
  const uint64_t nch = (n + kSub - 1) / kSub;
  const uint64_t bm_end = kHeader + smsec + nbm;
  const uint64_t tpos = (bm_end + 3) & ~3ull, dpos = tpos + 8 * nch;
  const uint64_t comp = P ? dpos + Dtot : kHeader + smsec;
  const uint64_t raw = kHeader + n * E;
  const bool coded = comp < raw;
  if (local == 0 && tid == 0) write_header<DT>(d, P, coded ? kCoded : 0u, coded ? comp : raw);
  if (!coded) {  // the coded form is not shorter: this tile's part RAW
    const uint64_t v0 = (uint64_t)local * d.tvals;
    const uint64_t v1 = min<uint64_t>(n, v0 + d.tvals);
    if (v0 < v1) raw_copy(d, v0 * E, v1 * E, tid, NT);
    return;
  }
  if (P == 0) return;
  if (local == 0 && bm_end + tid < tpos) gp(d.stream)[bm_end + tid] = 0;
  const uint32_t S = d.tvals / kSub;
  const uint8_t* regions = reinterpret_cast<const uint8_t*>(f.stash + sbase);
  const G1 uint32_t* info = gp(reinterpret_cast<const uint32_t*>(regions + d.tvals));
  uint64_t cc = sc >> 32, cb = sb >> 32;  // changes and bytes before the chunk
  for (uint32_t r = 0; r < S; ++r) {  // uniform
    const uint64_t k = (uint64_t)local * S + r;
    if (k >= nch) break;
    const uint32_t w = info[r];
    const uint32_t c = w & 0x1FFFu, words = (w >> 13) & 0x1FFFu;
    const bool dense = (w >> 26) & 1u;
    const uint32_t len = (uint32_t)left_in(n, k * kSub, kSub);
    const uint32_t bytes = coded_bytes(c, words, dense, len);
    uint8_t* dst = d.stream + dpos + cb;
    if (bytes > 0 && dense) {
      for (uint32_t i = tid; i < bytes / 4; i += NT)
        gp(reinterpret_cast<uint32_t*>(dst))[i] = gp(reinterpret_cast<const uint32_t*>(regions + r * kSub))[i];
    } else if (bytes > 0) {
      const uint32_t h = 2u * rans_lanes(c) + words;  // u16 of states and words
      const uint8_t* src = regions + (r + 1) * kSub - 2u * h;
      for (uint32_t i = tid; i < h; i += NT)
        gp(reinterpret_cast<uint16_t*>(dst))[i] = gp(reinterpret_cast<const uint16_t*>(src))[i];
      if (tid == 0 && (words & 1u)) gp(reinterpret_cast<uint16_t*>(dst))[h] = 0;
    }
    cc += c;
    cb += bytes;
    if (tid == 0) {
      G1 uint32_t* e = gp(reinterpret_cast<uint32_t*>(d.stream + tpos + 8 * k));
      e[0] = (uint32_t)cc;
      e[1] = (uint32_t)cb;
    }
  }
}

// Finishing kernel for coded items: one wave per tile.  A tile's work here
// is small (its chunks' table entries and data, a few hundred bytes at low
// change rates), so one wave per tile lets every tile of the batch be resident
// at once (bf16 coded encode in-step, one wave per tile instead of four: 0.1%
// 41.2 -> 36.9 us, 1% 43.2 -> 38.9 us, 10% 55.7 -> 53.0 us).
template <int DT>
__global__ __launch_bounds__(kCodedFinishThreads) void encode_finish_coded_kernel(FinArgs f, uint32_t batch_id) {
  const uint32_t rel = blockIdx.x / f.tpi;
  const uint32_t local = blockIdx.x - rel * f.tpi;
  const uint64_t t0 = f.tile0 + (uint64_t)rel * f.tpi;                // the item's first tile
  const uint64_t sbase = f.stash0 + (t0 - f.tile0 + local) * f.cap;  // this tile's stash
  const EncItem d = f.items[f.item0 + rel];
  if (d.batch_id != batch_id) return;  // uniform
  finish_tile_coded<DT>(f, d, local, t0, sbase);
}

// Coded items of more than kThreads tiles: the exclusive prefixes of the
// tiles' data bytes and changes over each item, a window of kThreads tiles at
// a time (one workgroup per item): prefix[t] = bytes before | changes before
// << 32, for the finishing kernel's workgroups to read.
template <int DT>
__global__ __launch_bounds__(kThreads) void coded_scan_kernel(FinArgs f, uint64_t* prefix, uint32_t batch_id) {
  __shared__ uint64_t s_red[kThreads / 64];
  const uint32_t tid = threadIdx.x;
  const EncItem d = f.items[f.item0 + blockIdx.x];
  if (d.batch_id != batch_id) return;  // uniform
  const uint64_t t0 = f.tile0 + (uint64_t)blockIdx.x * f.tpi;
  uint64_t run_b = 0, run_c = 0;
  for (uint32_t w0 = 0; w0 < f.tpi; w0 += kThreads) {  // uniform
    const uint32_t k = w0 + tid;
    const uint32_t c = k < f.tpi ? gp(f.counts)[t0 + k] : 0u;
    // a window's sums stay below 2^24, so the two halves never carry
    const uint64_t v = (c & 0xFFFFu) | ((uint64_t)(c >> 16) << 32);
    uint64_t tot;
    const uint64_t ex = block_scan<uint64_t>(v, s_red, tot);
    if (k < f.tpi) gp(prefix + t0)[k] = (run_b + (uint32_t)ex) | ((run_c + (ex >> 32)) << 32);
    run_b += (uint32_t)tot;
    run_c += tot >> 32;
    __syncthreads();  // s_red is read before the next window writes it
  }
}

// Finishing kernel for groups of at most kThreads tiles per item: one
// workgroup per tile, so tiles whose changes overflowed their stash are
// derived again in parallel.  The item's tile counts, the tile's first
// kThreads stash words and the descriptor are requested together; then the
// tile's records go to their places, or its part of the shard is copied RAW.
template <int DT>
__global__ __launch_bounds__(kThreads) void encode_finish_tile_kernel(FinArgs f, uint32_t batch_id) {
  constexpr int E = Tr<DT>::E;
  __shared__ uint64_t s_red64[kThreads / 64];
  __shared__ uint32_t s_red[kThreads / 64];

  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint32_t rel = blockIdx.x / f.tpi;
  const uint32_t local = blockIdx.x - rel * f.tpi;
  const uint64_t t0 = f.tile0 + (uint64_t)rel * f.tpi;                // the item's first tile
  const uint64_t sbase = f.stash0 + (t0 - f.tile0 + local) * f.cap;  // this tile's stash
  const uint32_t c_t = tid < f.tpi ? gp(f.counts)[t0 + tid] : 0u;
  const uint32_t mine = gp(f.counts)[t0 + local];
  const uint32_t sv = gp(f.stash)[sbase + tid];  // cap >= kThreads: inside the stash
  const EncItem d = f.items[f.item0 + rel];
  if (d.batch_id != batch_id) return;  // uniform

  // total and exclusive prefix of the item's tile counts, in one reduction
  uint64_t v = (uint64_t)c_t | ((uint64_t)(tid < local ? c_t : 0u) << 32);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) s_red64[wave] = v;
  __syncthreads();
  uint64_t sum = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) sum += s_red64[w];
  const uint64_t P = (uint32_t)sum;
  const uint32_t excl = (uint32_t)(sum >> 32);

  const uint64_t n = d.n;
  const uint32_t B = d.block_size;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;
  const uint64_t nbm = (((n + B - 1) >> lb) + 7) / 8;
  const uint64_t smsec = sm_sec<DT>(n);
  const uint64_t comp = kHeader + smsec + (P ? nbm + 5 * P : 0);
  const uint64_t raw = kHeader + n * E;
  const bool cmode = d.compress != 0 && comp < raw;
  if (d.compress == kBlockVariant) {  // uniform: block-hash variant
    const uint64_t bcomp = kHeader + smsec + (P ? nbm + P * d.block_size : 0);
    const bool bmode = bcomp < raw;
    if (local == 0 && tid == 0) write_header<DT>(d, P, bmode ? kBlockVariant : 0u, bmode ? bcomp : raw);
    if (!bmode) {
      const uint64_t v0 = (uint64_t)local * d.tvals;
      const uint64_t v1 = min<uint64_t>(n, v0 + d.tvals);
      if (v0 < v1) raw_copy(d, v0 * E, v1 * E, tid, kThreads);
    } else if (mine > 0) {
      copy_to_stream(d.stream + kHeader + smsec + nbm + (uint64_t)excl * d.block_size,
                     reinterpret_cast<const uint8_t*>(f.stash + sbase), (uint64_t)mine * d.block_size, tid, kThreads);
    }
    return;
  }
  if (local == 0 && tid == 0) write_header<DT>(d, P, cmode ? 1u : 0u, cmode ? comp : raw);
  if (d.compress != 0 && !cmode) {  // the compressed form is not shorter: this tile's part RAW
    const uint64_t v0 = (uint64_t)local * d.tvals;
    const uint64_t v1 = min<uint64_t>(n, v0 + d.tvals);
    if (v0 < v1) raw_copy(d, v0 * E, v1 * E, tid, kThreads);
    return;
  }
  if (!cmode || mine == 0) return;
  const uint64_t pbase = kHeader + smsec + nbm;
  if (mine <= d.cap) {
    const uint64_t tb = (uint64_t)local * d.tvals;
    for (uint32_t r = tid; r < mine; r += kThreads) {
      const uint32_t w = r < kThreads ? sv : gp(f.stash)[sbase + r];
      put_record(d.stream, d.capacity, pbase + 5ull * (excl + r), (uint32_t)(tb + (w & 0xFFFFu)), w >> 16);
    }
  } else {
    rederive_tile<DT>(d, local, excl, pbase, s_red);
  }
}

// Validation of a stream's 64-byte header h (16 words) for shard (n, off) of
// rank r: 0, or the status bit of the first failing class -- magic/version,
// a field mismatch (mode 3 only where the tensor is declared coded), or
// lengths inconsistent with the mode or beyond the slot (mode 3: only the
// table's place is checked here, the rest per chunk).
template <int DT, bool CODED>
__device__ __forceinline__ uint32_t header_status(const uint32_t* h, uint64_t n, uint64_t off, uint32_t r,
                                                  uint32_t world, uint32_t B, uint64_t nb, uint64_t nbm,
                                                  uint64_t slot) {
  constexpr int E = Tr<DT>::E;
  const uint32_t h_dtype = (h[1] >> 16) & 0xFFu, h_mode = h[1] >> 24;
  const uint64_t h_n = h[4] | ((uint64_t)h[5] << 32);
  const uint64_t P = h[6] | ((uint64_t)h[7] << 32);
  const uint64_t h_tot = h[8] | ((uint64_t)h[9] << 32);
  const uint64_t h_off = h[10] | ((uint64_t)h[11] << 32);
  if (h[0] != 0x52454943u || (h[1] & 0xFFFFu) != 1u) return CIERA_ST_MAGIC;
  if (h_dtype != (uint32_t)DT || h[2] != B || h_n != n || h_off != off || h[12] != r || h[13] != world ||
      h_mode > (CODED ? kCoded : kBlockVariant))
    return CIERA_ST_FIELD;
  if (h_mode == kCoded) {  // the chunk table gives the length; checked per chunk
    const uint64_t dpos = ((kHeader + sm_sec<DT>(n) + nbm + 3) & ~3ull) + 8 * ((n + kSub - 1) / kSub);
    if (P > n || h_tot > slot || (P ? h_tot < dpos : h_tot != kHeader + sm_sec<DT>(n))) return CIERA_ST_LENGTH;
    return 0;
  }
  const uint64_t want = h_mode == 0   ? kHeader + n * E
                        : h_mode == 1 ? kHeader + sm_sec<DT>(n) + (P ? nbm + 5 * P : 0)
                                      : kHeader + sm_sec<DT>(n) + (P ? nbm + P * B : 0);
  if (P > (h_mode == 2 ? nb : n) || h_tot > slot || h_tot != want) return CIERA_ST_LENGTH;
  return 0;
}

// Chunk k's table entries (k-1 and k: cumulative changes pc, cc and bytes pb,
// cb) checked against the chunk (len values) and the data (D bytes, nch
// chunks, P changes): true when the entry is consistent.  c and bytes: the
// chunk's changes and data bytes.
__device__ __forceinline__ bool chunk_entry_ok(uint32_t pc, uint32_t pb, uint32_t cc, uint32_t cb, uint64_t k,
                                               uint64_t nch, uint32_t len, uint64_t D, uint64_t P) {
  const uint32_t c = cc - pc, bytes = cb - pb;
  if (cc < pc || cb < pb || cb > D || c > len || (bytes & 3u) != 0 || ((c == 0) != (bytes == 0)) ||
      (k == nch - 1 && (cc != P || cb != D)))
    return false;
  // coded data holds its states and is shorter than the dense form
  return !(c > 0 && bytes != pad4u(len) && (bytes < 4u * rans_lanes(c) || bytes > pad4u(len)));
}

// Inclusive sum of v over each group of GS (16 or 64) lanes, in lane order,
// with DPP row operations (a row is 16 lanes): shifts by 1, 2, 4 and 8 within
// rows (lanes shifted in from outside the row read 0), then, for a whole wave,
// the last lane of row 0 added to row 1 and of row 2 to row 3, and the last
// lane of row 1 to rows 2 and 3.  Every lane must be active.
template <int GS>
__device__ __forceinline__ uint32_t group_incl_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  if constexpr (GS == 64) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  }
  return v;
}

// Decodes 64/GS chunks' coded data at once, one chunk per group of GS (16 or
// 64) lanes: each lane passes its group's chunk (win: the data in LDS, nbytes
// bytes; c changes among len values; c = 0 for a group without one) and, for
// change j of the chunk, an active lane calls emit(j, idx, cls, esc, ok):
// chunk offset idx, step class cls, escaped exponent esc, ok = idx inside the
// chunk; emit returns status bits.  lcum: 16 words of LDS per group for its
// gap-bucket starts, which each step searches.  Returns the lane's status
// bits: ST_PATCH for words missing or left over, a final state other than
// 2^16, a change past the chunk, and emit's.
template <int GS, class Emit>
__device__ __forceinline__ uint32_t rans_decode_groups(const uint32_t* win, uint32_t nbytes, uint32_t c,
                                                       uint32_t len, uint32_t* lcum, Emit&& emit) {
  const uint32_t lane = lane_id(), gl = lane & (GS - 1u), g0 = lane - gl;
  const uint64_t gmask = GS == 64 ? ~0ull : ((1ull << (GS & 63)) - 1ull) << g0;
  const bool live = c > 0;
  const uint32_t Lr = live ? rans_lanes(c) : 0u;
  const uint32_t navail = live ? (nbytes - 4u * Lr) / 2u : 0u;
  const uint16_t* words = reinterpret_cast<const uint16_t*>(win + Lr);
  uint32_t gf, gcum;
  gap_table<GS>(live ? c : 1u, live ? len : (uint32_t)kSub, gf, gcum);
  uint32_t* const gc = lcum + (g0 / GS) * 16u;  // the group's starts, then 4096 up to 16 entries
  if (gl < 16u) gc[gl] = gl < 13u ? gcum : 4096u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint32_t x = gl < Lr ? win[gl] : kRansLow;
  uint32_t ptr = 0, run = 0, err = 0;
  // Lanes past the states (and groups without a chunk) hold kRansLow and
  // never change, so x < kRansLow alone picks the lanes that take a word.  A
  // word past the data reads as 0; the final count check flags it.
  auto renorm = [&]() {
    const uint64_t m = __builtin_amdgcn_uicmp(x, kRansLow, 36) & gmask;  // 36: unsigned less-than
    if (x < kRansLow) {
      const uint32_t pos = ptr + lanes_below(m);
      const uint32_t w = words[pos < navail ? pos : 0u];
      x = (x << 16) | (pos < navail ? w : 0u);
    }
    ptr += (uint32_t)__popcll(m);
  };
  uint32_t steps = Lr ? (c + Lr - 1u) / Lr : 0u;  // the most rounds of any group
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) steps = max(steps, (uint32_t)__shfl_xor(steps, o));
  for (uint32_t t = 0; t < steps; ++t) {  // uniform
    const uint32_t j = t * Lr + gl;
    const bool act = gl < Lr && j < c;
    // bucket: the last start <= slot (four halving steps over 16 entries;
    // the first start is 0), its start (cb), the next one (nb), their count
    // (bk)
    uint32_t slot = x & 4095u, lo = 0;
#pragma unroll
    for (uint32_t st = 8; st > 0; st >>= 1) lo = gc[lo + st] <= slot ? lo + st : lo;
    const uint32_t bk = lo + 1u, cb = gc[lo], nb = gc[lo + 1u];
    if (act) x = __umul24(nb - cb, x >> 12) + slot - cb;  // both factors below 2^24
    renorm();
    uint32_t g1 = 1;
    if (act) {
      const uint32_t kb = bk - 1u;
      g1 = (1u << kb) | (x & ((1u << kb) - 1u));
      x >>= kb;
    }
    renorm();
    slot = x & 4095u;
    const uint32_t cls = class_of_slot(slot);
    if (act) x = class_freq(cls) * (x >> 12) + slot - class_start(cls);
    renorm();
    uint32_t esc = 0;
    if (act && cls == 14u) {
      esc = x & 0xFFu;
      x >>= 8;
    }
    renorm();
    const uint32_t incl = group_incl_sum<GS>(act ? g1 : 0u);
    const uint32_t idx = run + incl - 1u;
    run += GS == 64 ? (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) : __shfl(incl, GS - 1, GS);
    if (act) {
      const bool ok = idx < len;
      if (!ok) err |= CIERA_ST_PATCH;
      err |= emit(j, idx, cls, esc, ok);
    }
  }
  if (live && (ptr + (ptr & 1u) != navail || (gl < Lr && x != kRansLow))) err |= CIERA_ST_PATCH;
  return err;
}

// Rank r's received stream of a decode item: in the item's slot layout, or at
// the pointer the caller gave for that rank (read from the batch's scratch).
__device__ __forceinline__ const uint8_t* rank_stream(const DecItem& d, uint32_t r) {
  return d.ranks ? gp(d.ranks)[r] : d.streams + (uint64_t)r * d.slot;
}

// Coded rows decoded ahead of the merge, so that many resident waves hide the
// decoder's dependent steps.  One wave per four consecutive chunk slots of a
// rank's stream (U rows per decode tile): when each of the four chunks is small
// (at most 64 changes and 1 KB of data) it decodes all four at once, 16 lanes
// each; otherwise it decodes them one after another with all its lanes.  A chunk whose header and table entry are valid, whose data is
// coded and whose changes fit the first bytes of its own output region (4 per
// change: offset | step class << 12 | escaped exponent << 16, all ones for a
// change past the chunk, as two 16-bit stores) leaves them there; the merge
// reads them before it writes the values.  Other chunks are left to the merge.
constexpr uint32_t kPackMax = 64;        // changes of a chunk decoded in a 16-lane group
constexpr uint32_t kPackBytes = 1024;    // its data, at most
template <int DT, int U>
__global__ __launch_bounds__(64) void coded_prepass_kernel(const DecItem* __restrict__ items, uint32_t item0,
                                                            uint32_t tpr, uint32_t world, uint32_t* status_out,
                                                            uint32_t batch_id) {
  constexpr int E = Tr<DT>::E;
  __shared__ uint32_t s_h[16];
  __shared__ uint32_t s_c[4][4];           // per chunk: changes (0 unless decoded here), bytes, start, length
  __shared__ uint32_t s_w[kSub / 4];       // chunk data: one chunk's, or four of 1 KB each
  __shared__ uint32_t s_lc[64];            // gap-bucket starts, 16 entries per chunk decoded at once
  const uint32_t tid = threadIdx.x, lane = lane_id();
  const uint32_t cpr = tpr * U, qpr = (cpr + 3) / 4, qpi = qpr * world;  // chunk slots, quads
  const uint32_t blk = blockIdx.x / qpi;
  const uint32_t rel = blockIdx.x - blk * qpi;
  const uint32_t r = rel / qpr;
  const uint64_t k0 = 4ull * (rel - r * qpr);
  const DecItem d = items[item0 + blk];
  if (d.batch_id != batch_id) return;  // uniform
  const uint64_t off = ((uint64_t)r * d.q + min<uint64_t>(r, d.rem)) * d.cols;
  const uint64_t n = (d.q + (r < d.rem ? 1u : 0u)) * d.cols;
  const uint64_t nch = (n + kSub - 1) / kSub;
  if (k0 >= nch) return;
  const uint8_t* st = rank_stream(d, r);
  const uint32_t B = d.block_size;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;
  const uint64_t nb = (n + B - 1) >> lb, nbm = (nb + 7) / 8;
  if (tid < 16) s_h[tid] = gp(reinterpret_cast<const uint32_t*>(st))[tid];
  __syncthreads();
  if (header_status<DT, true>(s_h, n, off, r, world, B, nb, nbm, d.slot)) return;  // the merge reports it
  const uint64_t P = s_h[6] | ((uint64_t)s_h[7] << 32), h_tot = s_h[8] | ((uint64_t)s_h[9] << 32);
  if ((s_h[1] >> 24) != kCoded || P == 0) return;
  const uint64_t tpos = (kHeader + sm_sec<DT>(n) + nbm + 3) & ~3ull, dpos = tpos + 8 * nch;
  if (tid < 4u) {  // chunk k0 + tid's entry, checked; c stays 0 unless it is decoded here
    uint32_t c = 0, bytes = 0, pb = 0, len = 0;
    const uint64_t k = k0 + tid;
    if (k < nch) {
      const G1 uint32_t* e = gp(reinterpret_cast<const uint32_t*>(st + tpos + 8 * k));
      const uint32_t cc = e[0], cb = e[1], pc = k > 0 ? e[-2] : 0u;
      pb = k > 0 ? e[-1] : 0u;
      len = (uint32_t)left_in(n, k * kSub, kSub);
      if (chunk_entry_ok(pc, pb, cc, cb, k, nch, len, h_tot - dpos, P) && cc > pc && cb - pb != pad4u(len) &&
          cc - pc <= len * E / 4) {  // coded, and its records fit
        c = cc - pc;
        bytes = cb - pb;
      }
    }
    s_c[tid][0] = c; s_c[tid][1] = bytes; s_c[tid][2] = pb; s_c[tid][3] = len;
  }
  __syncthreads();
  bool any = false, packed = true;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    any |= s_c[g][0] > 0;
    packed &= s_c[g][0] <= kPackMax && s_c[g][1] <= kPackBytes;
  }
  if (!any) return;
  const G1 uint32_t* src = gp(reinterpret_cast<const uint32_t*>(st + dpos));
  auto decode_one = [&](uint32_t g, auto gs) -> uint32_t {
    constexpr int GS = decltype(gs)::value;
    const uint32_t cg = s_c[g][0], bg = s_c[g][1], pg = s_c[g][2], lg = s_c[g][3];
    uint32_t* const win = &s_w[GS == 16 ? g * (kPackBytes / 4) : 0];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // the window's last reader is done
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (cg) {  // only a chunk decoded here is read
      for (uint32_t w = lane & (GS - 1u); w < bg / 4; w += GS) win[w] = src[pg / 4 + w];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // the lanes read each other's words
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    G1 uint16_t* rec = gp(reinterpret_cast<uint16_t*>(d.out + (off + (k0 + g) * kSub) * E));
    auto emit = [rec](uint32_t j, uint32_t idx, uint32_t cls, uint32_t esc, bool ok) -> uint32_t {
      const uint32_t v = ok ? idx | (cls << 12) | (esc << 16) : 0xFFFFFFFFu;
      rec[2 * j] = (uint16_t)v;
      rec[2 * j + 1] = (uint16_t)(v >> 16);
      return 0u;
    };
    return rans_decode_groups<GS>(win, bg, cg, lg, s_lc, emit);
  };
  uint32_t err = 0;
  if (packed) {  // four small chunks at once, 16 lanes each
    err = decode_one(lane >> 4, std::integral_constant<int, 16>{});
  } else {  // one after another, with all lanes
    for (uint32_t g = 0; g < 4; ++g)
      if (s_c[g][0]) err |= decode_one(g, std::integral_constant<int, 64>{});  // uniform
  }
  if (err) report(status_out, err);
}

// --------------------------------------------------------------------- decode
// One workgroup per tile of U*4096 values of one rank's stream.  The bulk loads
// (sign|mantissa bytes and cached exponents) are issued before the header and
// the patch range are known, so their latency overlaps that chain.

// Decode of tile `bid` of a group: item bid / (tpr * world), rank, tile in
// the rank's stream.  Workgroup-wide; every return is uniform.
template <int DT, int U, bool CODED>
__device__ __forceinline__ void decode_tile(const DecItem* __restrict__ items, uint32_t item0, uint32_t tpr,
                                            uint32_t world, uint32_t* status_out, uint32_t batch_id,
                                            uint32_t bid) {
  constexpr int E = Tr<DT>::E;
  constexpr uint32_t T = (uint32_t)kDecRow * U;
  constexpr uint32_t BMW = (T / 64 + 31) / 32;  // words of per-tile block bits (B >= 64)
  constexpr int SW = (16 * Tr<DT>::SMBITS + 31) / 32;  // words of 16 sign|mantissa records
  __shared__ uint32_t s_hdr[16];
  __shared__ uint32_t s_expbm[BMW];  // blocks of the tile that hold a patch
  __shared__ uint32_t s_ex[T / 4];   // the tile's exponents: cached, then patched in place
  __shared__ uint32_t s_sum[kDecThreads / 64];
  constexpr bool XP = kSmPieces<DT> != 0;  // records of whole wave rows swapped through LDS
  // each wave's exchange buffer: fp32/fp16 records in, values out
  constexpr uint32_t kStage = kSmWaveRow<DT> > 1024u * E ? kSmWaveRow<DT> : 1024u * E;
  // coded patches (the tensor's streams may be CODED): each row's chunk data.
  // It shares LDS with the exchange buffers: the exchanges run before the
  // first barrier (records in) and after the patch phase (values out), the
  // chunk data only in between, with barriers on both sides.
  constexpr uint32_t kStageWords = kDecThreads / 64 * (kStage / 4);
  constexpr uint32_t kWinWords = CODED ? (uint32_t)U * (kSub / 4) : 1u;
  __shared__ uint32_t s_share[kStageWords > kWinWords ? kStageWords : kWinWords];
  uint32_t (*const s_stage)[kStage / 4] = reinterpret_cast<uint32_t (*)[kStage / 4]>(s_share);
  uint32_t (*const s_win)[CODED ? kSub / 4 : 1] = reinterpret_cast<uint32_t (*)[CODED ? kSub / 4 : 1]>(s_share);
  __shared__ uint8_t s_mark[CODED ? U : 1][64];  // coded: blocks of each row that were patched
  __shared__ uint32_t s_lcm[CODED ? U : 1][16];  // coded: gap-bucket starts of each row the merge decodes

  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint32_t tpi = tpr * world;
  const uint32_t blk = bid / tpi;
  const uint32_t item = item0 + blk;
  const uint32_t rel = bid - blk * tpi;
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
  const uint8_t* st = rank_stream(d, r);
  const uint32_t B = d.block_size;
  const uint32_t lb = (uint32_t)__ffs(B) - 1u;  // B is a power of two (checked by the API)
  const bool aligned = (off & 15u) == 0;
  uint8_t* const cache = d.cache + off;

  // 1. bulk loads, COMPRESSED layout (in bounds for either mode: a slot holds a RAW stream)
  uint32_t sw[U][SW], cw[U][4];
  v4u pc[U][XP ? kSmPieces<DT> : 1];
  bool whole[U];  // uniform per wave: the wave's 1024 values of row u are in the shard
  int cnt[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint64_t c0 = ts + (uint64_t)u * kDecRow + (uint64_t)tid * kEPT;
    const uint64_t w0 = ts + (uint64_t)u * kDecRow + (uint64_t)wave * 1024u;
    whole[u] = XP && w0 + 1024u <= te;
    cnt[u] = (int)left_in(te, c0, 16);
    if (cnt[u] > 0) {
      if (whole[u]) load_sm_pieces<DT>(st + kHeader + sm_off<DT>(w0), pc[u]);
      else load_smw<DT, SW>(st + kHeader, c0, cnt[u], sw[u]);
      load_words<4, true>(cache + c0, (uint32_t)cnt[u], aligned, cw[u]);  // 16 contiguous bytes per lane
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
  if (CODED && tid < (uint32_t)U * 64u) s_mark[tid >> 6][tid & 63u] = 0;
  if (CODED && tid < (uint32_t)U) s_sum[tid] = 0;  // coded: differences per dense row
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
  if constexpr (XP) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (whole[u]) swap_sm_pieces<DT, SW>(&s_stage[wave][0], pc[u], sw[u]);
  }
  __syncthreads();
  const uint32_t h_mode = s_hdr[1] >> 24;
  const uint64_t P = s_hdr[6] | ((uint64_t)s_hdr[7] << 32);
  const uint64_t h_tot = s_hdr[8] | ((uint64_t)s_hdr[9] << 32);
  const uint32_t bad = header_status<DT, CODED>(s_hdr, n, off, r, world, B, nb, nbm, d.slot);
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

  bool patched = false;  // uniform: some exponent of the tile comes from the stream
  if (h_mode == kBlockVariant) {
    // 3b. BLOCK: the tile's changed blocks come whole from the payload.  The
    //     bitmap bits before the tile give the first one's place (their count,
    //     summed over the workgroup); the tile's own bits go to LDS.
    const uint64_t tb0 = ts >> lb, tb1 = (te + B - 1) >> lb;
    const uint32_t nbt = (uint32_t)(tb1 - tb0);
    const uint8_t* bm = st + kHeader + sm_sec<DT>(n);
    const uint64_t pbase = kHeader + sm_sec<DT>(n) + nbm;
    uint32_t before = 0, e = 0;
    if (tid < BMW) s_expbm[tid] = 0;
    if (P > 0) {  // the payload follows the bitmap: the bit-word loads stay inside the stream
      for (uint64_t b = (uint64_t)tid * 32; b < tb0; b += 32ull * kDecThreads)
        before += (uint32_t)__popc(bits_of(load_bits_w(bm, b), (uint32_t)min<uint64_t>(32, tb0 - b)));
      if (tid * 32 < nbt) s_expbm[tid] = bits_of(load_bits_w(bm, tb0 + tid * 32), min(32u, nbt - tid * 32));
      if (te == n && tid == 0 && (nb & 7u) != 0 && (gp(bm)[nbm - 1] >> (nb & 7u)) != 0) e |= CIERA_ST_BITMAP;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) before += __shfl_xor(before, o);
    if (lane == 0) s_sum[wave] = before;
    __syncthreads();
    uint32_t prefix = 0, mine = 0;
#pragma unroll
    for (int w = 0; w < kDecThreads / 64; ++w) prefix += s_sum[w];
#pragma unroll
    for (int w = 0; w < (int)BMW; ++w) mine += (uint32_t)__popc(s_expbm[w]);
    if (te == n && tid == 0 && P > 0 && prefix + mine != P) e |= CIERA_ST_BITMAP;
    if (e) report(status_out, e);
    patched = mine > 0;
    if (patched) {
      uint8_t* const s_exb = reinterpret_cast<uint8_t*>(s_ex);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t vo = (uint32_t)u * kDecRow + tid * kEPT;  // value offset in the tile
        const uint32_t bt = vo >> lb;
        if (bt < nbt && ((s_expbm[bt >> 5] >> (bt & 31u)) & 1u)) {
          uint32_t r = prefix;
          for (uint32_t w = 0; w < (bt >> 5); ++w) r += (uint32_t)__popc(s_expbm[w]);
          r += (uint32_t)__popc(s_expbm[bt >> 5] & ((1u << (bt & 31u)) - 1u));
          if (r < P) {  // more set bits than n_changed: reported above, read nothing past the payload
            const v4u v = load16_any(st + pbase + (uint64_t)r * B + (vo & (B - 1)));
            *reinterpret_cast<v4u*>(s_exb + vo) = v;
          }
        }
      }
      __syncthreads();
    }
  } else if (h_mode == kCoded) {
    if constexpr (CODED) {  // (without CODED the header check rejects mode 3)
      // 3c. CODED: chunk row u of the tile is chunk t_in * U + u.  Its table
      //     entry (and the one before) gives its changes and data; dense data
      //     replaces the row's cached exponents (every thread its 16), coded
      //     data goes to LDS and wave u decodes it.  Each patched value marks
      //     its block; the tile's bitmap bits are compared at the end.
      patched = P > 0;
      if (P > 0) {
        const uint64_t nch = (n + kSub - 1) / kSub;
        const uint64_t bm_end = kHeader + sm_sec<DT>(n) + nbm;
        const uint64_t tpos = (bm_end + 3) & ~3ull, dpos = tpos + 8 * nch;
        const uint64_t D = h_tot - dpos;
        const uint64_t tb0 = ts >> lb, tb1 = (te + B - 1) >> lb;
        const uint32_t nbt = (uint32_t)(tb1 - tb0);
        const uint8_t* bm = st + kHeader + sm_sec<DT>(n);
        uint32_t bm_got = 0, bm_tail = 0;
        if (tid * 32 < nbt) bm_got = bits_of(load_bits_w(bm, tb0 + tid * 32), min(32u, nbt - tid * 32));
        if (te == n && tid == 0 && (nb & 7u) != 0) bm_tail = gp(bm)[nbm - 1] >> (nb & 7u);
        uint32_t c[U], nbytes[U], start[U], len[U];
        bool dense[U], coded[U], recs[U];
        uint32_t e = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint64_t k = (uint64_t)t_in * U + (uint64_t)u;
          c[u] = nbytes[u] = start[u] = len[u] = 0;
          dense[u] = coded[u] = recs[u] = false;
          if (k >= nch) continue;
          const G1 uint32_t* ent = gp(reinterpret_cast<const uint32_t*>(st + tpos + 8 * k));
          const uint32_t cc = ent[0], cb = ent[1];
          const uint32_t pc = k > 0 ? ent[-2] : 0u, pb = k > 0 ? ent[-1] : 0u;
          len[u] = (uint32_t)left_in(n, k * kSub, kSub);
          if (!chunk_entry_ok(pc, pb, cc, cb, k, nch, len[u], D, P)) {
            e |= CIERA_ST_LENGTH;
            continue;
          }
          c[u] = cc - pc;
          nbytes[u] = cb - pb;
          start[u] = pb;
          dense[u] = c[u] > 0 && nbytes[u] == pad4u(len[u]);
          coded[u] = c[u] > 0 && !dense[u];
          recs[u] = coded[u] && c[u] <= len[u] * E / 4;  // decoded ahead into the row's output region
        }
        if (tid == 0 && e) report(status_out, e);
        uint8_t* const s_exb = reinterpret_cast<uint8_t*>(s_ex);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t vo = (uint32_t)u * kDecRow + tid * kEPT;
          if (dense[u] && cnt[u] > 0) {  // this thread's 16 values of a dense row
            uint32_t dw[4];
            load_words<4>(st + dpos + start[u] + tid * kEPT, (uint32_t)cnt[u], false, dw);
            uint32_t diff = 0, wide = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const uint32_t a = byte_of(dw, j), o = byte_of(cw[u], j);
              if (j < cnt[u]) {
                diff += a != o ? 1u : 0u;
                wide |= a > Tr<DT>::EMASK ? 1u : 0u;
              }
            }
            v4u nv;
            nv.x = dw[0]; nv.y = dw[1]; nv.z = dw[2]; nv.w = dw[3];
            *reinterpret_cast<v4u*>(s_exb + vo) = nv;
            if (diff) s_mark[u][(tid * kEPT) >> lb] = 1;  // 16 values lie in one block (B >= 64)
            if (wide) report(status_out, CIERA_ST_PATCH);
            atomicAdd(&s_sum[u], diff);
          }
          if (recs[u]) {  // the row's changes, as the prepass left them, applied by every thread
            const G1 uint16_t* rec = gp(reinterpret_cast<const uint16_t*>(out + ((uint64_t)t_in * T + u * kDecRow) * E));
            uint32_t err = 0;
            for (uint32_t j = tid; j < c[u]; j += kDecThreads) {
              const uint32_t v = rec[2 * j] | ((uint32_t)rec[2 * j + 1] << 16);
              if (v == 0xFFFFFFFFu) continue;  // a change past the chunk (reported by the prepass)
              const uint32_t idx = v & 0xFFFu, cls = (v >> 12) & 0xFu, esc = (v >> 16) & 0xFFu;
              uint8_t* const rowex = s_exb + u * kDecRow;
              const uint32_t nv = cls == 14u ? esc : (rowex[idx] + class_step(cls)) & 0xFFu;
              if (nv > Tr<DT>::EMASK) {
                err |= CIERA_ST_PATCH;
              } else {
                rowex[idx] = (uint8_t)nv;
                s_mark[u][idx >> lb] = 1;
              }
            }
            if (err) report(status_out, err);
          } else if (coded[u] && tid * 16 < nbytes[u]) {  // coded data the merge decodes itself, to LDS
            const G1 uint32_t* src = gp(reinterpret_cast<const uint32_t*>(st + dpos + start[u]));
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (tid * 4 + (uint32_t)q < nbytes[u] / 4) s_win[u][tid * 4 + q] = src[tid * 4 + q];
          }
        }
        __syncthreads();
        if ((int)wave < U && coded[wave] && !recs[wave]) {  // uniform per wave: wave u decodes row u
          const uint32_t u = wave;
          uint8_t* const rowex = s_exb + u * kDecRow;
          const uint32_t err = rans_decode_groups<64>(&s_win[u][0], nbytes[u], c[u], len[u], &s_lcm[u][0],
                                                      [&](uint32_t, uint32_t idx, uint32_t cls, uint32_t esc,
                                                          bool ok) -> uint32_t {
            if (!ok) return 0u;
            const uint32_t nv = cls == 14u ? esc : (rowex[idx] + class_step(cls)) & 0xFFu;
            if (nv > Tr<DT>::EMASK) return CIERA_ST_PATCH;
            rowex[idx] = (uint8_t)nv;
            s_mark[u][idx >> lb] = 1;  // plain stores: lanes hitting one block write the same value
            return 0u;
          });
          if (err) report(status_out, err);
        }
        __syncthreads();
        if ((int)wave < U && (dense[wave] || coded[wave])) {  // the row's patched blocks into the tile's bits
          const uint32_t u = wave;
          const uint32_t nbr = (uint32_t)kSub >> lb, rb0 = u * nbr;  // blocks per row (<= 64); the row's first
          const uint64_t rowbm = __ballot(lane < nbr && s_mark[u][lane] != 0);
          if (lane == 0 && rowbm) {
            if (nbr >= 32u) {  // whole words
              atomicOr(&s_expbm[rb0 >> 5], (uint32_t)rowbm);
              if (nbr == 64u) atomicOr(&s_expbm[(rb0 >> 5) + 1], (uint32_t)(rowbm >> 32));
            } else {  // the row's bits lie inside one word
              atomicOr(&s_expbm[rb0 >> 5], (uint32_t)rowbm << (rb0 & 31u));
            }
          }
        }
        __syncthreads();
        uint32_t eb = 0;
        if (tid * 32 < nbt && bm_got != s_expbm[tid]) eb |= CIERA_ST_BITMAP;
        if (bm_tail != 0) eb |= CIERA_ST_BITMAP;
        if (tid < (uint32_t)U && dense[tid] && s_sum[tid] != c[tid]) eb |= CIERA_ST_PATCH;
        if (eb) report(status_out, eb);
      }
    }
  } else {
  // 3. COMPRESSED: this tile's patch range [lo, hi).  Every wave finds it on its
  //    own (two searches: a first round of 64 probes, then 32 lanes per key),
  //    so the records can be read without a barrier in between.
  const uint64_t recs = kHeader + sm_sec<DT>(n) + nbm;
  uint32_t lo = 0, hi = 0;
  if (P > 0) {
    if (tpr == 1) {
      hi = (uint32_t)P;
    } else {
      uint64_t a0 = 0, z0 = 0, a1 = 0, z1 = 0;  // first p with idx[p] >= key lies in [a, z]
      {
        if (P <= kGridMax) {
          // Short lists: 64 probes, one per record, find both keys at once.
          const uint64_t step = (P + 63) / 64;
          const uint64_t p = (uint64_t)lane * step;
          uint32_t idx = 0, ex = 0;
          if (p < P) read_rec(st, recs, p, idx, ex);
          const uint64_t m0 = __ballot(p < P && idx < ts), m1 = __ballot(p < P && idx < te);
          if (m0) { a0 = (uint64_t)(63u - (uint32_t)__clzll(m0)) * step + 1; z0 = min<uint64_t>(P, a0 - 1 + step); }
          if (m1) { a1 = (uint64_t)(63u - (uint32_t)__clzll(m1)) * step + 1; z1 = min<uint64_t>(P, a1 - 1 + step); }
        } else {
          // Longer lists: 32 lanes per key (lanes 0-31: ts, 32-63: te) probe a
          // window centred where the key falls if the changes are spread
          // evenly (P * key / n), S records apart, so that it spans at least
          // +-3 standard deviations of that count (sqrt(P) / 2 at most).  At
          // even change rates the next round ends the search, and a tile
          // touches only the lines around its own records: a grid over the
          // whole list would bring every line of it into the L2 of each XCD
          // that runs one of the stream's tiles.  A key outside its window
          // (clustered changes) is left in [0, w] or past the window, and the
          // rounds below narrow that 32-fold each.  (Float estimates suffice:
          // n < 2^32, and only the probe places, not the answer, depend on
          // them.)
          const uint32_t Pu = (uint32_t)P;
          const uint32_t S = (uint32_t)(0.095f * __builtin_amdgcn_sqrtf((float)Pu)) + 1u;
          const float fr = (float)Pu * __builtin_amdgcn_rcpf((float)(uint32_t)n);
          uint32_t w[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t e = min(Pu, (uint32_t)(fr * (float)(uint32_t)(k ? te : ts)));
            w[k] = e > 16u * S ? e - 16u * S : 0u;
          }
          const bool second = lane >= 32;
          const uint32_t key = (uint32_t)(second ? te : ts);
          const uint64_t p = (uint64_t)(second ? w[1] : w[0]) + (uint64_t)(lane & 31u) * S;
          uint32_t idx = 0, ex = 0;
          if (p < P) read_rec(st, recs, p, idx, ex);
          const uint64_t m = __ballot(p < P && idx < key);
          uint64_t a[2], z[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const uint32_t h = (uint32_t)(m >> (32 * k));
            if (h) {  // past probe `top`; at or before the next one (or the end)
              const uint32_t top = 31u - (uint32_t)__clz(h);
              a[k] = (uint64_t)w[k] + (uint64_t)top * S + 1;
              z[k] = top == 31u ? P : min<uint64_t>(P, a[k] - 1 + S);
            } else {  // at or before the window's first probe
              a[k] = 0;
              z[k] = w[k];
            }
          }
          a0 = a[0]; z0 = max(z[0], a[0]); a1 = a[1]; z1 = max(z[1], a[1]);
        }
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
  patched = hi > lo;
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

  // 5. bitmap check: the tile's bits mark exactly the blocks that hold patches
  if (P > 0) {
    uint32_t e = 0;
    if (bm_mine && bm_got != s_expbm[tid]) e |= CIERA_ST_BITMAP;
    if (bm_tail != 0) e |= CIERA_ST_BITMAP;
    if (e) report(status_out, e);
  }
  }  // COMPRESSED

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

  // 6. merge and store; write back the cache lines that changed
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (cnt[u] > 0) {
      const uint64_t c0 = ts + (uint64_t)u * kDecRow + (uint64_t)tid * kEPT;
      // A wave whose 1024 values of the row are all in the shard stores them as
      // contiguous pieces through its LDS buffer: whole-line stores instead of
      // 16-byte pieces strided 32 or 64 bytes apart.
      // The stores are non-temporal: written once, never read by this launch,
      // and streamed out in address order instead of left dirty in the caches
      // for the next kernel to write back (1% layer: decode 341 -> 322 us and
      // the encode after it 34.9 -> 32.6 us in-step; alone, the decode takes 8
      // us longer, as it now pays its own write-back).
      const uint64_t w0 = ts + (uint64_t)u * kDecRow + (uint64_t)wave * 1024u;
      uint32_t hv[DT == 3 ? 8 : 1];  // fp16: two values per word, joined once for either store
      if constexpr (DT == 3) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          hv[q] = join<DT>(sm_from_words<DT>(sw[u], 2 * q), byte_of(ex[u], 2 * q)) |
                  (join<DT>(sm_from_words<DT>(sw[u], 2 * q + 1), byte_of(ex[u], 2 * q + 1)) << 16);
      }
      if (aligned && w0 + 1024u <= te) {  // uniform per wave
        uint32_t v[4 * E];
        if constexpr (DT == 1) {
#pragma unroll
          for (int q = 0; q < 4; ++q) bf16x4_join(sw[u][q], ex[u][q], v[2 * q], v[2 * q + 1]);
        } else if constexpr (DT == 3) {
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = hv[q];
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) v[j] = join<DT>(sm_from_words<DT>(sw[u], j), byte_of(ex[u], j));
        }
        uint32_t* const sb = &s_stage[wave][0];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < E; ++q) {
          v4u a;
          a.x = v[4 * q]; a.y = v[4 * q + 1]; a.z = v[4 * q + 2]; a.w = v[4 * q + 3];
          *reinterpret_cast<v4u*>(sb + 4 * xslot<E>(lane, q)) = a;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < E; ++q) {
          const uint32_t k = 64u * q + lane;
          stg16_nt(out + w0 * E + 16 * k, *reinterpret_cast<const v4u*>(sb + 4 * xslot<E>(k / E, k % E)));
        }
        __builtin_amdgcn_wave_barrier();
      } else if constexpr (DT == 1) {
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) bf16x4_join(sw[u][q], ex[u][q], o[2 * q], o[2 * q + 1]);
        store_words<8>(out + c0 * E, (uint32_t)cnt[u] * E, aligned, o);
      } else if constexpr (DT == 3) {
        if (cnt[u] == 16 && aligned) {  // lane by lane: non-temporal too
          v4u a, b;
          a.x = hv[0]; a.y = hv[1]; a.z = hv[2]; a.w = hv[3];
          b.x = hv[4]; b.y = hv[5]; b.z = hv[6]; b.w = hv[7];
          stg16_nt(out + c0 * E, a);
          stg16_nt(out + c0 * E + 16, b);
        } else {
          uint32_t v[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) v[j] = (hv[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          store16<DT>(out + c0 * E, cnt[u], v, aligned);
        }
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

template <int DT, int U, bool CODED>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const DecItem* __restrict__ items, uint32_t item0,
                                                          uint32_t tpr, uint32_t world, uint32_t* status_out,
                                                          uint32_t batch_id) {
  decode_tile<DT, U, CODED>(items, item0, tpr, world, status_out, batch_id, blockIdx.x);
}

// The bf16 decode with coded rows, held to eight waves per SIMD: left to
// itself the compiler gives it 106 scalar registers, which allow seven; at
// eight it keeps the excess in vector-register lanes, without scratch
// (bf16, 10% change: coded decode 534 -> 505 us; 1%: unchanged).  fp16 and
// fp32 would spill to scratch at eight.
template <int U>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(8))) void decode_coded_bf16_kernel(
    const DecItem* __restrict__ items, uint32_t item0, uint32_t tpr, uint32_t world, uint32_t* status_out,
    uint32_t batch_id) {
  decode_tile<1, U, true>(items, item0, tpr, world, status_out, batch_id, blockIdx.x);
}

// The same decode from a grid of fewer workgroups than tiles, each taking
// tiles bid, bid + gridDim.x, ... in turn: a caller that runs the decode beside
// other work bounds the compute units it occupies.
template <int DT, int U>
__global__ __launch_bounds__(kDecThreads) void decode_bounded_kernel(const DecItem* __restrict__ items, uint32_t item0,
                                                                  uint32_t tpr, uint32_t world, uint32_t* status_out,
                                                                  uint32_t batch_id, uint32_t ntiles) {
  for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {  // uniform
    decode_tile<DT, U, false>(items, item0, tpr, world, status_out, batch_id, t);
    __syncthreads();  // the next tile reuses the LDS
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
    const int cnt = (int)left_in(n, c0, 16);
    uint32_t v[16], ex[4] = {0, 0, 0, 0};
    load16<DT>(w + c0 * E, cnt, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) ex[j >> 2] |= exp_of<DT>(v[j]) << (8 * (j & 3));
    store_bytes16(cache + c0, cnt, aligned, ex);
  }
}

}  // namespace

// ----------------------------------------------- encode without allocation
// Scratch of ciera_encode_noalloc, for callers that cannot allocate: one copy
// per device, held until the process ends.  In host code this name stands for
// the array only as a symbol; its device address comes from
// hipGetSymbolAddress (static_scratch), never from the name itself.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

// Descriptors travel as kernel arguments, kDescPack per launch.
constexpr uint32_t kDescPack = 30;
struct EncDescPack {
  EncItem item[kDescPack];
};
static_assert(sizeof(EncDescPack) <= 3584, "descriptor pack must fit the kernel arguments");

__global__ __launch_bounds__(kThreads) void enc_desc_kernel(EncDescPack p, EncItem* __restrict__ dst, uint32_t n,
                                                            uint64_t* __restrict__ zero, uint64_t nzero,
                                                            uint32_t* __restrict__ head, uint32_t batch_id) {
  constexpr uint32_t W = sizeof(EncItem) / 4;
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x, step = gridDim.x * blockDim.x;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(p.item);
  for (uint32_t i = t; i < n * W; i += step) gp(reinterpret_cast<uint32_t*>(dst))[i] = src[i];
  for (uint64_t i = t; i < nzero; i += step) gp(zero)[i] = 0;
  if (t == 0 && head) gp(head)[0] = batch_id;
}

}  // namespace

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static void* addr[kMaxDevices] = {};
  static std::mutex mu;
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_enc_desc(const EncItem* host_items, uint32_t n, EncItem* dst, uint64_t* zero, uint64_t nzero,
                           uint32_t* head, uint32_t batch_id, hipStream_t s) {
  uint32_t done = 0;
  do {  // at least one launch: it also zeroes and writes the head
    EncDescPack p;
    const uint32_t k = std::min(kDescPack, n - done);
    std::memcpy(p.item, host_items + done, sizeof(EncItem) * k);
    (void)hipGetLastError();
    const uint32_t blocks = done == 0 ? (uint32_t)std::min<uint64_t>(1024, std::max<uint64_t>(1, (nzero + kThreads - 1) / kThreads)) : 1u;
    hipLaunchKernelGGL(enc_desc_kernel, dim3(blocks), dim3(kThreads), 0, s, p, dst + done, k,
                       done == 0 ? zero : nullptr, done == 0 ? nzero : 0ull, done == 0 ? head : nullptr, batch_id);
    if (hipError_t e = hipGetLastError()) return e;
    done += k;
  } while (done < n);
  return hipSuccess;
}

// ------------------------------------------------------------------- launchers
// Each launcher clears the thread's last-error state first, so that the error it
// returns is the launch's own and not one left by an unrelated earlier call.

// Workgroups per launch: a grid stays well below 2^32 work-items; larger
// batches are cut into launches of whole items.
constexpr uint64_t kMaxGrid = (uint64_t)1 << 22;

static hipError_t launch_encode_part(int dtype, int sub, uint32_t nitems, const EncArgs& a, uint32_t batch_id,
                                     hipStream_t s) {
  (void)hipGetLastError();
  const dim3 grid(nitems * a.tpi), block(kThreads);
#define CIERA_ENC(DT, S)                                                                \
  do {                                                                                  \
    if (a.self) hipLaunchKernelGGL((encode_self_kernel<DT, S>), grid, block, 0, s, a, batch_id); \
    else hipLaunchKernelGGL((encode_kernel<DT, S>), grid, block, 0, s, a, batch_id);   \
  } while (0)
#define CIERA_ENC_DT(DT)                  \
  switch (sub) {                          \
    case 1: CIERA_ENC(DT, 1); break;      \
    case 2: CIERA_ENC(DT, 2); break;      \
    case 4: CIERA_ENC(DT, 4); break;      \
    case 8: CIERA_ENC(DT, 8); break;      \
    default: return hipErrorInvalidValue; \
  }
  if (dtype == 1) {
    CIERA_ENC_DT(1)
  } else if (dtype == 2) {
    CIERA_ENC_DT(2)
  } else if (dtype == 3) {
    CIERA_ENC_DT(3)
  } else {
    return hipErrorInvalidValue;
  }
#undef CIERA_ENC_DT
#undef CIERA_ENC
  return hipGetLastError();
}

hipError_t launch_encode(int dtype, int sub, uint32_t nitems, const EncArgs& a, uint32_t batch_id, hipStream_t s) {
  const uint32_t per = (uint32_t)std::max<uint64_t>(1, kMaxGrid / a.tpi);
  for (uint32_t i = 0; i < nitems; i += per) {
    EncArgs c = a;
    c.item0 = a.item0 + i;
    if (hipError_t e = launch_encode_part(dtype, sub, std::min(per, nitems - i), c, batch_id, s)) return e;
  }
  return hipSuccess;
}

hipError_t launch_encode_finish(int dtype, const EncItem* items, uint32_t item0, uint32_t nitems, uint32_t wg_per_item,
                                const uint32_t* counts, const uint32_t* stash, uint32_t batch_id, hipStream_t s) {
  (void)hipGetLastError();
  if (nitems == 0 || wg_per_item == 0) return hipSuccess;
  const dim3 grid(wg_per_item, nitems < 65535u ? nitems : 65535u), block(kThreads);
  if (dtype == 1) hipLaunchKernelGGL((encode_finish_kernel<1>), grid, block, 0, s, items, item0, nitems, counts, stash, batch_id);
  else if (dtype == 2) hipLaunchKernelGGL((encode_finish_kernel<2>), grid, block, 0, s, items, item0, nitems, counts, stash, batch_id);
  else if (dtype == 3) hipLaunchKernelGGL((encode_finish_kernel<3>), grid, block, 0, s, items, item0, nitems, counts, stash, batch_id);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_coded_scan(int dtype, uint32_t nitems, const FinArgs& f, uint64_t* prefix, uint32_t batch_id,
                             hipStream_t s) {
  for (uint32_t i = 0; i < nitems; i += 65535u) {
    (void)hipGetLastError();
    FinArgs c = f;
    c.item0 = f.item0 + i;
    c.tile0 = f.tile0 + (uint64_t)i * f.tpi;
    const dim3 grid(std::min(65535u, nitems - i)), block(kThreads);
    if (dtype == 1) hipLaunchKernelGGL((coded_scan_kernel<1>), grid, block, 0, s, c, prefix, batch_id);
    else if (dtype == 2) hipLaunchKernelGGL((coded_scan_kernel<2>), grid, block, 0, s, c, prefix, batch_id);
    else if (dtype == 3) hipLaunchKernelGGL((coded_scan_kernel<3>), grid, block, 0, s, c, prefix, batch_id);
    else return hipErrorInvalidValue;
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

hipError_t launch_encode_finish_tiles(int dtype, bool coded, uint32_t nitems, const FinArgs& f, uint32_t batch_id,
                                      hipStream_t s) {
  if (nitems == 0) return hipSuccess;
  const uint32_t per = (uint32_t)std::max<uint64_t>(1, kMaxGrid / f.tpi);
  for (uint32_t i = 0; i < nitems; i += per) {
    (void)hipGetLastError();
    FinArgs c = f;
    c.item0 = f.item0 + i;
    c.tile0 = f.tile0 + (uint64_t)i * f.tpi;
    c.stash0 = f.stash0 + (uint64_t)i * f.tpi * f.cap;
    const dim3 grid(std::min(per, nitems - i) * f.tpi), block(kThreads), cblock(kCodedFinishThreads);
    if (coded) {
      if (dtype == 1) hipLaunchKernelGGL((encode_finish_coded_kernel<1>), grid, cblock, 0, s, c, batch_id);
      else if (dtype == 2) hipLaunchKernelGGL((encode_finish_coded_kernel<2>), grid, cblock, 0, s, c, batch_id);
      else if (dtype == 3) hipLaunchKernelGGL((encode_finish_coded_kernel<3>), grid, cblock, 0, s, c, batch_id);
      else return hipErrorInvalidValue;
    } else {
      if (dtype == 1) hipLaunchKernelGGL((encode_finish_tile_kernel<1>), grid, block, 0, s, c, batch_id);
      else if (dtype == 2) hipLaunchKernelGGL((encode_finish_tile_kernel<2>), grid, block, 0, s, c, batch_id);
      else if (dtype == 3) hipLaunchKernelGGL((encode_finish_tile_kernel<3>), grid, block, 0, s, c, batch_id);
      else return hipErrorInvalidValue;
    }
    if (hipError_t e = hipGetLastError()) return e;
  }
  return hipSuccess;
}

template <int DT, int U>
static void launch_coded_merge(dim3 grid, hipStream_t s, const DecItem* items, uint32_t item0, uint32_t tpr,
                               uint32_t world, uint32_t* status, uint32_t batch_id) {
  if constexpr (DT == 1)
    hipLaunchKernelGGL((decode_coded_bf16_kernel<U>), grid, dim3(kDecThreads), 0, s, items, item0, tpr, world, status,
                       batch_id);
  else
    hipLaunchKernelGGL((decode_kernel<DT, U, true>), grid, dim3(kDecThreads), 0, s, items, item0, tpr, world, status,
                       batch_id);
}

static hipError_t launch_decode_part(int dtype, int u, bool coded, const DecItem* items, uint32_t item0, uint32_t nitems,
                                     uint32_t tpr, uint32_t world, uint32_t* status, uint32_t batch_id,
                                     uint32_t max_wg, hipStream_t s) {
  (void)hipGetLastError();
  const uint32_t ntiles = nitems * tpr * world;
  if (max_wg && max_wg < ntiles && !coded) {  // a bounded grid walks the tiles
    const dim3 bgrid(max_wg), block(kDecThreads);
#define CIERA_DECB(DT, U) \
  hipLaunchKernelGGL((decode_bounded_kernel<DT, U>), bgrid, block, 0, s, items, item0, tpr, world, status, batch_id, ntiles)
    switch (dtype * 8 + u) {
      case 9: CIERA_DECB(1, 1); break;
      case 10: CIERA_DECB(1, 2); break;
      case 17: CIERA_DECB(2, 1); break;
      case 18: CIERA_DECB(2, 2); break;
      case 25: CIERA_DECB(3, 1); break;
      case 26: CIERA_DECB(3, 2); break;
      default: return hipErrorInvalidValue;
    }
#undef CIERA_DECB
    return hipGetLastError();
  }
  const dim3 grid(ntiles), block(kDecThreads);
  const dim3 pgrid(nitems * world * ((tpr * (uint32_t)u + 3) / 4));  // coded prepass: four chunk slots each
#define CIERA_DEC(DT, U)                                                                                    \
  do {                                                                                                      \
    if (coded) {                                                                                            \
      hipLaunchKernelGGL((coded_prepass_kernel<DT, U>), pgrid, dim3(64), 0, s, items, item0, tpr, world, status, \
                         batch_id);                                                                         \
      launch_coded_merge<DT, U>(grid, s, items, item0, tpr, world, status, batch_id);                      \
    } else {                                                                                                \
      hipLaunchKernelGGL((decode_kernel<DT, U, false>), grid, block, 0, s, items, item0, tpr, world,        \
                         status, batch_id);                                                                 \
    }                                                                                                       \
  } while (0)
  if (dtype == 1) {
    switch (u) {
      case 1: CIERA_DEC(1, 1); break;
      case 2: CIERA_DEC(1, 2); break;
      default: return hipErrorInvalidValue;
    }
  } else if (dtype == 2) {
    switch (u) {
      case 1: CIERA_DEC(2, 1); break;
      case 2: CIERA_DEC(2, 2); break;
      default: return hipErrorInvalidValue;
    }
  } else if (dtype == 3) {
    switch (u) {
      case 1: CIERA_DEC(3, 1); break;
      case 2: CIERA_DEC(3, 2); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef CIERA_DEC
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, int u, bool coded, const DecItem* items, uint32_t item0, uint32_t nitems, uint32_t tpr,
                         uint32_t world, uint32_t* status, uint32_t batch_id, uint32_t max_wg,
                         hipStream_t s) {
  const uint64_t tpi = (uint64_t)tpr * world;
  if (tpi * kDecThreads >= ((uint64_t)1 << 32)) return hipErrorInvalidValue;  // one item alone too large
  const uint32_t per = (uint32_t)std::max<uint64_t>(1, kMaxGrid / tpi);
  for (uint32_t i = 0; i < nitems; i += per) {
    if (hipError_t e = launch_decode_part(dtype, u, coded, items, item0 + i, std::min(per, nitems - i), tpr, world, status,
                                          batch_id, max_wg, s))
      return e;
  }
  return hipSuccess;
}

// One workgroup per row of 4096 values: a block (B <= 4096) lies inside one row.
hipError_t launch_hash_seed(int dtype, const uint8_t* x, uint8_t* hashes, uint64_t n, uint32_t block_size, hipStream_t s) {
  const uint64_t tiles = (n + kSub - 1) / kSub;
  if (tiles == 0) return hipSuccess;
  if (tiles >= ((uint64_t)1 << 31)) return hipErrorInvalidValue;
  (void)hipGetLastError();
  const dim3 grid((uint32_t)tiles), block(kThreads);
  if (dtype == 1) hipLaunchKernelGGL((hash_seed_kernel<1, 1>), grid, block, 0, s, x, hashes, n, block_size);
  else if (dtype == 2) hipLaunchKernelGGL((hash_seed_kernel<2, 1>), grid, block, 0, s, x, hashes, n, block_size);
  else if (dtype == 3) hipLaunchKernelGGL((hash_seed_kernel<3, 1>), grid, block, 0, s, x, hashes, n, block_size);
  else return hipErrorInvalidValue;
  return hipGetLastError();
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
