// tq_device.h -- device helpers shared by the HIP kernels of libtq: the B3
// digit table in LDS, the per-group integer cores of both packed formats,
// and small bit utilities.  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tq_layout.h"

namespace tqdev {

constexpr int kLutCopies = 32;   // one table copy per lane of a half wave
constexpr int kLutEntries = 256; // byte values; 243..255 map to zero trits

typedef long v2l __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t s0, uint32_t s1, uint32_t sel) {
  return __builtin_amdgcn_perm(s0, s1, sel);
}

// Cross-lane reductions without an LDS round trip.  DPP moves within rows
// of 16 lanes (a VALU operand modifier, a few cycles) replace the 64-lane
// __shfl_xor ladder (a chain of ds_bpermute, each one an LDS round trip):
// swap neighbours (quad_perm [1,0,3,2]), swap pairs ([2,3,0,1]), rotate the
// row by 4 and by 8 lanes; the four row results are then read out with
// v_readlane.  Every lane of the wave must be active.
constexpr int kDppSwap1 = 0xB1, kDppSwap2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// In every lane: the maximum over its row of 16 lanes.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(dpp_move<kDppSwap1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<kDppSwap2>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_move<kDppRor4>(__float_as_int(v))));
  return fmaxf(v, __int_as_float(dpp_move<kDppRor8>(__float_as_int(v))));
}

// The maximum over the 64 lanes, wave-uniform.  fmaxf is exact and
// order-free, so this equals any other reduction order.
__device__ __forceinline__ float wave_max64(float v) {
  v = row16_max(v);
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The integer sums over lanes 0..31 (lo) and 32..63 (hi), wave-uniform.
__device__ __forceinline__ void half_sums(int v, int &lo, int &hi) {
  v += dpp_move<kDppSwap1>(v);
  v += dpp_move<kDppSwap2>(v);
  v += dpp_move<kDppRor4>(v);
  v += dpp_move<kDppRor8>(v);
  lo = __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16);
  hi = __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ float half_bits(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Streaming loads of weight bytes, each read once per call: nontemporal, so
// they do not displace reused data from the caches (a plain read of HBM
// streams about 12% faster this way on MI355X).  p: 16-, 4- and 2-byte
// aligned respectively.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3), aligned(4)));

__device__ __forceinline__ uint4 ld_stream16(const uint8_t *p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// The same 16 bytes from a 4-byte-aligned address (row-major B3R groups).
typedef uint32_t u32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ uint4 ld_stream16u(const uint8_t *p) {
  const u32x4a4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4a4 *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ uint3 ld_stream12(const uint8_t *p) {
  const u32x3 t = __builtin_nontemporal_load(reinterpret_cast<const u32x3 *>(p));
  return make_uint3(t.x, t.y, t.z);
}

__device__ __forceinline__ uint32_t ld_stream2(const uint8_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
}

// ---------------------------------------------------------------------
// B3 digit table.  For byte value v (0..242): .lo holds the trits of base-3
// digits 0..3 of v (one signed byte each), .hi the trit of digit 4 in byte 0;
// values 243..255 (never produced by the packer) decode to zero trits.
// Each workgroup builds it in LDS 32 times, entry v of copy c at byte
// (v * 32 + c) * 8.  Lane l reads copy
// l % 32, so the 32 lanes served together hit 32 distinct bank pairs
// whatever byte values they hold.
// ---------------------------------------------------------------------
__device__ __forceinline__ uint2 b3_entry(int v) {
  uint32_t lo = 0, hi = 0;
  if (v < 243) {
    int x = v;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      lo |= (uint32_t)(uint8_t)(int8_t)(x % 3 - 1) << (8 * i);
      x /= 3;
    }
    hi = (uint32_t)(uint8_t)(int8_t)(x - 1);
  }
  return make_uint2(lo, hi);
}

// Fill the 32 copies.  With a block size of 256, 512, 1024, 2048 or 4096
// every thread computes one entry v and stores it, two adjacent copies per
// 16-byte store, into 32 / (blockDim / 256) of the copies; lane l starts at copy
// pair l % 16, so the 8 lanes of a store pass hit 8 distinct bank groups.
// NT: the block size when the caller knows it at compile time (the stores
// are then unrolled and need no read of the dispatch size: about 0.3 us
// less per workgroup on a 512-thread fill), 0 to read blockDim.
template <int NT = 0>
__device__ __forceinline__ void fill_b3_lut(uint2 *lut) {
  const int nt = NT ? NT : (int)blockDim.x;
  if ((nt & 255) == 0 && (kLutCopies / 2) % (nt >> 8) == 0) {
    constexpr int kPairs = kLutCopies / 2;
    const int v = threadIdx.x & 255;
    const uint2 e = b3_entry(v);
    const uint4 e2 = make_uint4(e.x, e.y, e.x, e.y);
    uint4 *lut4 = reinterpret_cast<uint4 *>(lut);
    const int per = kPairs / (nt >> 8);
    const int k0 = (int)(threadIdx.x >> 8) * per;
    if constexpr (NT != 0) {
#pragma unroll
      for (int k = 0; k < per; k++) lut4[v * kPairs + ((threadIdx.x + k0 + k) & (kPairs - 1))] = e2;
    } else {
      for (int k = k0; k < k0 + per; k++) lut4[v * kPairs + ((threadIdx.x + k) & (kPairs - 1))] = e2;
    }
  } else {
    for (int idx = threadIdx.x; idx < kLutEntries * kLutCopies; idx += nt)
      lut[idx] = b3_entry(idx / kLutCopies);
  }
}

// Look up byte k of `word`: one v_perm builds the LDS address
// (byte value in bits 8..15, the lane's copy offset in bits 0..7).
template <int k>
__device__ __forceinline__ uint2 lut_lookup(const uint2 *lut, uint32_t word, uint32_t laneoff) {
  constexpr uint32_t sel = 0x0C0C0000u | ((4u + k) << 8);
  uint32_t addr = perm_b32(word, laneoff, sel);
  return *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(lut) + addr);
}

template <int j>
__device__ __forceinline__ uint2 b3_byte(const uint2 *lut, const uint32_t (&w)[7],
                                         uint32_t laneoff) {
  return lut_lookup<j & 3>(lut, w[j >> 2], laneoff);
}

// Activations of one group for MT rows, as 32 words per row, held in
// (scalar or vector) registers.
template <int MT>
struct XRegs {
  uint32_t v[MT][32];
  __device__ __forceinline__ uint32_t get(int m, int i) const { return v[m][i]; }
};

// Integer core of one B3 group for MT activation rows.
//   w[0..3]: device bytes 0..15, w[4..6]: bytes 16..25 and the scale.
// byte j < 25: digits 0..3 pair with activation word j, digit 4 with byte
// j % 4 of word 25 + j / 4; byte 25: digits 1..3 pair with bytes 1..3 of
// word 31 (its digit 0 is a zero-trit padding digit).
template <int MT, typename XS>
__device__ __forceinline__ void b3_group(const uint2 *lut, uint32_t laneoff,
                                         const uint32_t (&w)[7], const XS &x, int (&S)[MT]) {
  // All 26 table lookups are issued before the first dot so that the LDS
  // latency overlaps; two accumulator chains per row halve the dependency.
  uint2 e[26];
#define TQ_LK(J) e[J] = b3_byte<J>(lut, w, laneoff);
  TQ_LK(0) TQ_LK(1) TQ_LK(2) TQ_LK(3) TQ_LK(4) TQ_LK(5) TQ_LK(6) TQ_LK(7) TQ_LK(8)
  TQ_LK(9) TQ_LK(10) TQ_LK(11) TQ_LK(12) TQ_LK(13) TQ_LK(14) TQ_LK(15) TQ_LK(16)
  TQ_LK(17) TQ_LK(18) TQ_LK(19) TQ_LK(20) TQ_LK(21) TQ_LK(22) TQ_LK(23) TQ_LK(24)
  TQ_LK(25)
#undef TQ_LK
  int S2[MT];
#pragma unroll
  for (int m = 0; m < MT; m++) S2[m] = 0;
#pragma unroll
  for (int j = 0; j < 25; j++) {
#pragma unroll
    for (int m = 0; m < MT; m++) {
      S[m] = sdot4(e[j].x, x.get(m, j), S[m]);
      S2[m] = sdot4(e[j].y, x.get(m, 25 + (j >> 2)) >> (8 * (j & 3)), S2[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < MT; m++) S[m] = sdot4(e[25].x, x.get(m, 31), S[m]) + S2[m];
}

// Byte 0 of each of four words (the fifth trits of four B3 bytes, from the
// digit table's .y) packed into one word: two v_perm byte merges and one
// shift-or.
__device__ __forceinline__ uint32_t pack_y4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t lo = perm_b32(b, a, 0x0C0C0400u), hi = perm_b32(d, c, 0x0C0C0400u);
  return lo | (hi << 16);
}

// One B3 group decoded for several activation rows: the 26 digit-table
// entries of this lane's row and the fifth trits of bytes 4c..4c+3 packed
// into one word each (two byte merges and a shift-or), made once and
// dotted with each row's activation words.
struct B3Dec {
  uint2 e[26];
  uint32_t py[6];
};

__device__ __forceinline__ void b3_decode(const uint2 *lut, uint32_t laneoff, const uint32_t (&w)[7], B3Dec &d) {
  // all 26 table lookups before the first use, so that the LDS latency overlaps
#define TQ_LK(J) d.e[J] = b3_byte<J>(lut, w, laneoff);
  TQ_LK(0) TQ_LK(1) TQ_LK(2) TQ_LK(3) TQ_LK(4) TQ_LK(5) TQ_LK(6) TQ_LK(7) TQ_LK(8)
  TQ_LK(9) TQ_LK(10) TQ_LK(11) TQ_LK(12) TQ_LK(13) TQ_LK(14) TQ_LK(15) TQ_LK(16)
  TQ_LK(17) TQ_LK(18) TQ_LK(19) TQ_LK(20) TQ_LK(21) TQ_LK(22) TQ_LK(23) TQ_LK(24)
  TQ_LK(25)
#undef TQ_LK
#pragma unroll
  for (int c = 0; c < 6; c++) d.py[c] = pack_y4(d.e[4 * c].y, d.e[4 * c + 1].y, d.e[4 * c + 2].y, d.e[4 * c + 3].y);
}

// Integer core of a decoded B3 group with one row's activation words in
// VGPRs (read from LDS by the caller, the same address in every lane): the
// dots take VGPR operands, so the fifth trits go in packed (B3Dec::py), one
// dot with word 25 + c per four bytes, where the SGPR form shifts the
// activation word instead.
__device__ __forceinline__ int b3_dot_v(const B3Dec &d, const uint32_t (&x)[32]) {
  int S = 0, S2 = 0;
#pragma unroll
  for (int j = 0; j < 25; j++) S = sdot4(d.e[j].x, x[j], S);
#pragma unroll
  for (int c = 0; c < 6; c++) S2 = sdot4(d.py[c], x[25 + c], S2);
  // word 31: the fifth trit of byte 24 (byte 0) and digits 1..3 of byte 25
  S2 = sdot4(d.e[24].y, x[31], S2);
  return sdot4(d.e[25].x, x[31], S) + S2;
}

// The same with the activation words in SGPRs (XS::get(0, i)), two
// accumulator chains; the fifth trit of byte j pairs with byte j % 4 of
// word 25 + j / 4, shifted down.
template <typename XS>
__device__ __forceinline__ int b3_dot_s(const B3Dec &d, const XS &x) {
  int S = 0, S2 = 0;
#pragma unroll
  for (int j = 0; j < 25; j++) {
    S = sdot4(d.e[j].x, x.get(0, j), S);
    S2 = sdot4(d.e[j].y, x.get(0, 25 + (j >> 2)) >> (8 * (j & 3)), S2);
  }
  return sdot4(d.e[25].x, x.get(0, 31), S) + S2;
}

// One row, decode and dot together (VGPR activation words).
__device__ __forceinline__ int b3_group_v(const uint2 *lut, uint32_t laneoff, const uint32_t (&w)[7],
                                          const uint32_t (&x)[32]) {
  B3Dec d;
  b3_decode(lut, laneoff, w, d);
  return b3_dot_v(d, x);
}

// Exchange meet of one output's sums between the pieces of a block cut
// between workgroups: piece pc of npc walks the fixed binary tree over piece
// indices; at the node whose right subtree starts at `mid` both children
// swap their sums into that node's slot (slot0 + (mid - 1) * node_stride)
// with one agent-scope atomic exchange.  The piece that gets the other's
// sums back adds them (fp32 addition commutes, so the total does not depend
// on which arrives first), empties the slot and goes on up; the other is
// done with this output.  Slots hold fp32 bits xor the +inf pattern, so the
// all-zero word (both halves +inf, never a sum of finite terms) means empty.
// NMAT 2 carries both matrices' sums in one 64-bit word.  Returns whether
// this thread ends up holding the total (in tot).
__device__ __forceinline__ uint32_t meet_enc(float x) { return __float_as_uint(x) ^ 0x7F800000u; }
__device__ __forceinline__ float meet_dec(uint32_t e) { return __uint_as_float(e ^ 0x7F800000u); }

template <int NMAT>
__device__ __forceinline__ bool meet_tree(float (&tot)[NMAT], bool live, int pc, int npc, void *slot0_v,
                                          size_t node_stride) {
  using S = typename std::conditional<NMAT == 1, uint32_t, uint64_t>::type;
  S *slot0 = reinterpret_cast<S *>(slot0_v);
  S v = (S)meet_enc(tot[0]);
  if constexpr (NMAT == 2) v |= (S)meet_enc(tot[1]) << 32;
  bool holder = live;
  for (int l = 0; (1 << l) < npc; l++) {
    const int mid = (((pc >> l) & ~1) + 1) << l;  // first piece of the right subtree
    if (holder && mid < npc) {
      S *slot = slot0 + (size_t)(mid - 1) * node_stride;
      const S old = __hip_atomic_exchange(slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old == 0) {
        holder = false;
      } else {
        S w = (S)meet_enc(meet_dec((uint32_t)old) + meet_dec((uint32_t)v));
        if constexpr (NMAT == 2)
          w |= (S)meet_enc(meet_dec((uint32_t)(old >> 32)) + meet_dec((uint32_t)(v >> 32))) << 32;
        v = w;
        __hip_atomic_store(slot, (S)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  tot[0] = meet_dec((uint32_t)v);
  if constexpr (NMAT == 2) tot[1] = meet_dec((uint32_t)(v >> 32));
  return holder;
}

// The same meet for MT token rows at once: row r's slots lie r * row_stride
// words after row 0's; holder[r] (in: the thread has row r's sums; out: it
// holds row r's total).  Each tree level issues the rows' exchanges
// together, so the rows share its round trip.
template <int NMAT, int MT>
__device__ __forceinline__ void meet_tree(float (&tot)[MT][NMAT], bool (&holder)[MT], int pc, int npc,
                                          void *slot0_v, size_t node_stride, size_t row_stride) {
  using S = typename std::conditional<NMAT == 1, uint32_t, uint64_t>::type;
  S *slot0 = reinterpret_cast<S *>(slot0_v);
  S v[MT];
#pragma unroll
  for (int r = 0; r < MT; r++) {
    v[r] = (S)meet_enc(tot[r][0]);
    if constexpr (NMAT == 2) v[r] |= (S)meet_enc(tot[r][1]) << 32;
  }
  for (int l = 0; (1 << l) < npc; l++) {
    const int mid = (((pc >> l) & ~1) + 1) << l;  // first piece of the right subtree
    if (mid >= npc) continue;
    S old[MT];
#pragma unroll
    for (int r = 0; r < MT; r++) {
      old[r] = 0;
      if (holder[r])
        old[r] = __hip_atomic_exchange(slot0 + r * row_stride + (size_t)(mid - 1) * node_stride, v[r],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int r = 0; r < MT; r++) {
      if (!holder[r]) continue;
      if (old[r] == 0) {
        holder[r] = false;
      } else {
        S w = (S)meet_enc(meet_dec((uint32_t)old[r]) + meet_dec((uint32_t)v[r]));
        if constexpr (NMAT == 2)
          w |= (S)meet_enc(meet_dec((uint32_t)(old[r] >> 32)) + meet_dec((uint32_t)(v[r] >> 32))) << 32;
        v[r] = w;
        __hip_atomic_store(slot0 + r * row_stride + (size_t)(mid - 1) * node_stride, (S)0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < MT; r++) {
    tot[r][0] = meet_dec((uint32_t)v[r]);
    if constexpr (NMAT == 2) tot[r][1] = meet_dec((uint32_t)(v[r] >> 32));
  }
}

// Integer core of one 2B group.  Device byte 4c' + c, bits 2s hold
// k = 16c' + 4s + c, so field s of word c' pairs with activation word
// 4c' + s.  Codes d = t + 1 are dotted directly (fields masked in place, so
// field s arrives multiplied by 4^s, or by 16 for s = 3 after a 2-bit shift)
// and the group's activation sum is subtracted: sum t*x = sum d*x - sum x.
template <int MT, typename XS>
__device__ __forceinline__ void tb_group(const uint32_t (&w)[9], const XS &x,
                                         const int (&xsum)[MT], int (&S)[MT]) {
  int a1[MT], a4[MT], a16[MT];
#pragma unroll
  for (int m = 0; m < MT; m++) a1[m] = a4[m] = a16[m] = 0;
#pragma unroll
  for (int c = 0; c < 8; c++) {
    const uint32_t v = w[c];
    const uint32_t f0 = v & 0x03030303u, f1 = v & 0x0C0C0C0Cu, f2 = v & 0x30303030u,
                   f3 = (v >> 2) & 0x30303030u;
#pragma unroll
    for (int m = 0; m < MT; m++) {
      a1[m] = sdot4(f0, x.get(m, 4 * c + 0), a1[m]);
      a4[m] = sdot4(f1, x.get(m, 4 * c + 1), a4[m]);
      a16[m] = sdot4(f2, x.get(m, 4 * c + 2), a16[m]);
      a16[m] = sdot4(f3, x.get(m, 4 * c + 3), a16[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < MT; m++) S[m] = a1[m] + (a4[m] >> 2) + (a16[m] >> 4) - xsum[m];
}

// Integer core of one BP group (one activation row).  Word c of a plane
// holds, in byte b bit s, k = 32c + 4s + b: masking bit s of every byte gives
// four trits' worth of 2^s (bit 7 reads as -128), dotted with activation
// word 8c + s into an accumulator per s.  With the nonzero plane z (w[0..3])
// and the sign plane n (w[4..7]): sum t x = sum_z x - 2 sum_n x.
template <typename XS>
__device__ __forceinline__ int bp_group(const uint32_t (&w)[9], const XS &x) {
  int az[8], an[8];
#pragma unroll
  for (int s = 0; s < 8; s++) az[s] = an[s] = 0;
#pragma unroll
  for (int c = 0; c < 4; c++)
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const uint32_t m = 0x01010101u << s;
      az[s] = sdot4(w[c] & m, x.get(0, 8 * c + s), az[s]);
      an[s] = sdot4(w[4 + c] & m, x.get(0, 8 * c + s), an[s]);
    }
  int S = 0;
#pragma unroll
  for (int s = 0; s < 7; s++) S += (az[s] >> s) - 2 * (an[s] >> s);
  return S - (az[7] >> 7) + 2 * (an[7] >> 7);  // bit 7 weighed -128
}

}  // namespace tqdev
