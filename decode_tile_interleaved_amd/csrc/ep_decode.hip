// ep_decode.hip -- fused lattice-rANS tile decode and weight reconstruction
// for gfx950 (MI355X).
//
// The EntroPack abstract (mlsanity index page) states that the coordinates
// are entropy-coded in independently decodable tiles so that symbol decoding
// and numerical reconstruction fuse on the GPU.  This file is that pass.
//
// Work mapping.  A wave decodes one unit of 64 rANS states: one tile of 64
// states, or four tiles of 16 (lanes 16r..16r+15 hold tile r's states, one
// tile per DPP row).  Lane q of a tile owns state q and decodes the tile's
// local vectors q, q + S, q + 2S, ... (S states per tile): V = tile_vecs / S
// vectors per lane, 8, 16, 32 or 64.  Each step's vectors of a tile are
// contiguous, so a lane writes one 8-coordinate vector per step (16 bytes
// for BF16/FP16, 8 for FP8/INT8) next to its neighbours'.
//
// Per workgroup (up to 16 waves, one workgroup per CU):
//   1. every wave starts its global loads, all vector loads that need only the
//      kernel arguments: its tiles' word offsets, one context's frequencies,
//      the row scales of its first 8 vectors per lane;
//   2. one wave per context prefix-sums the frequencies (DPP scan), lists the
//      used symbols, sets a bitmap of the slots where a symbol starts, and
//      expands the context's table 64 slots at a time: a slot's symbol is the
//      number of starts up to it, which v_mbcnt counts from the row's bitmap;
//      the other waves copy the words of all the workgroup's tiles (one range
//      of the stream) into LDS with global_load_lds;
//   3. each wave reads its tiles' start states and word pointers from LDS
//      and decodes.
// Streams with more tiles than one such round of workgroups covers take the
// multi-tile kernel instead: one workgroup of up to 16 waves per CU builds
// the tables once, and each wave then loads and decodes one unit after
// another on its own.
//
// A tile in the stream: S/2 pair-count bytes (words in the region of states
// 2k and 2k+1), S length nibbles (W - 12, W the bit length of a start
// state), the start states' bits below their leading one, bit-packed, then
// region k: state 2k's words front to back, state 2k+1's back to front.  A
// lane finds its start state from the nibbles' prefix sum (DPP) and three
// 16-bit reads, and its first word from the pair counts' prefix sum; it then
// walks its words with a private pointer and a step of +2 or -2 bytes and
// always holds its next word in a register.
//
// Decode step for state x in [2^11, 2^27), kept as X = 8x so that the table
// address is one AND-OR:  8*slot = X & 0x1ff8;  e = table[ctx][slot];
//   x' = f * (x >> 10) + (slot - cum);  if x' < 2^11: x = x' << 16 | w
// where w is the state's next word.
//
// The step is software-pipelined around its one serial dependence, table
// lookup -> multiply-add -> compare -> select -> address -> next lookup (on
// gfx950 a dependent VALU op costs ten-odd cycles, an eight-byte LDS lookup
// about sixty).  The refilled state (x' with the held word shifted in) is
// formed in parallel with the compare, one v_cndmask selects the next state,
// one v_bitop3 or v_and_or makes its address, and the next lookup leaves.  Only
// then do the refilling lanes, under the exec mask, read their following
// word, which is first needed one step later.  Eight VALU instructions per
// step.
//
// Table entries (2^10 slots of 8 bytes per context; one ds_read_b64 meets
// fewer LDS bank conflicts than two dword reads), d1 = 8 (slot - cum) and
//   narrow (every used value in [-128, 127]): d0 = 8f | v << 24 (v as a
//     signed byte), so that X' = mad_u32_u24(d0, X >> 13, d1) and the value
//     converts in place (SDWA, byte 3 sign-extended);
//   wide (values in [-2048, 2047]): d0 = 8f | v << 16, whose low 13 bits
//     (one AND) are the multiplier and whose high half converts in place.
// Either way bits 0 and 1 of v sit at a fixed place in d0 (24/25 or 16/17):
// bit 0 is the coset bit b, and the XOR of bit 1 over coordinates 0..6 is the
// parity p that selects the last coordinate's context.
//
// LDS context order: F, C_0, C_1, then E_{b,p} at index 3 + b + 2p, 8 KB
// apart.  The fixed part of a context's base (C_0 or E_{0,0}) rides in the
// lookup's instruction offset; the lane's part (b or b + 2p, times 8 KB)
// comes from the entry.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "ep.h"
#include "ep_encode.hpp"
#include "ep_stream.hpp"

namespace ep {
namespace {

constexpr int kMaxWaves = 16;      // waves per workgroup (four per SIMD cover the decode chain)
constexpr uint32_t kCtxBytes = kProbTotal * 8;             // 8 KB per context
constexpr uint32_t kTableBytes = kContexts * kCtxBytes;     // 57344
constexpr uint32_t kRows = kProbTotal / 64;                // 16 rows of 64 slots per context
constexpr uint32_t kMarkWords = kProbTotal / 32;           // 32 bitmap words per context
constexpr uint32_t kLdsLimit = 160 * 1024;
constexpr uint32_t kMaxVecsPerLane = kTileVecsLarge / kStatesLow;  // 64
// Slack after the last word buffer.  A lane's pointer starts clamped to its
// tile's words and moves by at most one word per decoded symbol, 8 per
// vector, so even in a corrupt tile it stays within 16 V bytes past the tile
// (forward) or before it (backward, where the tables lie below the buffers);
// the start-state reads of a corrupt tile reach at most 64 + 2 + 208 + 6
// bytes past its start.
constexpr uint32_t kLdsPad = 16 * kMaxVecsPerLane + 16;
static_assert(kLdsPad >= 16 * kMaxVecsPerLane + 6 && kLdsPad >= 280, "LDS slack below a lane's worst overrun");
static_assert(kTableBytes >= 16 * kMaxVecsPerLane, "a backward lane's worst underrun stays inside the tables");
constexpr int kOutSym = 4;         // int16 lattice coordinates; 0..3 are the container dtypes

static_assert(kProbBits == 10, "table addressing below assumes 2^10 slots per context");
static_assert(kStateLow == (1u << 11) && kStateTop == 27, "X = 8x must fit 32 bits and refill below 8 L");

// Kernel arguments: section pointers computed on the host (the word
// section is 16-byte aligned), then the fields the first loads need, all in
// the first 80 bytes so that one round of scalar loads brings them.
struct Args {
  const uint16_t *freq;   // frequency section
  const uint32_t *toff;   // tile offsets: first word of each tile, then the word count
  const uint8_t *words;   // word section
  const float *scales;    // row scales
  uint32_t waves, n_units, n_tiles, words_off;  // units: groups of 64 / states consecutive tiles, one per wave
  uint32_t ctx_freq[kContexts];  // context c: index of its first frequency | symbol count << 16
  uint32_t nzbase[kContexts];
  int32_t smin[kContexts];
  void *out;
  uint64_t cols;                  // columns of the output (padded layouts only)
  uint32_t rows, vpr;             // rows; vectors per row
  uint32_t row_magic, row_shift;  // vec / vpr = umulhi(vec, row_magic) >> row_shift  (vpr > 1)
  uint32_t n_vec;
  uint32_t rec_off, mark_off, desc_off;  // LDS byte offsets
  uint32_t wg_q, wg_rem;  // multi-tile kernel: workgroup b decodes wg_q units, one more if b < wg_rem
  uint32_t wbuf;          // multi-tile kernel: bytes of each wave's word buffer
};
static_assert(offsetof(Args, ctx_freq) + sizeof(uint32_t) * kContexts <= 80, "early fields in the first 80 bytes");

typedef __attribute__((address_space(1))) void *gptr_t;
typedef __attribute__((address_space(3))) void *lptr_t;
typedef __attribute__((address_space(3))) const uint16_t *lds_u16_ptr;

// LDS loads by byte address; the decode kernel declares no static LDS, so its
// dynamic LDS starts at address 0
__device__ __forceinline__ uint32_t lds_u16(uint32_t byte) { return *(lds_u16_ptr)(uintptr_t)byte; }
__device__ __forceinline__ uint32_t lds_u8(uint32_t byte) {
  return *(__attribute__((address_space(3))) const uint8_t *)(uintptr_t)byte;
}

// hides a value from the compiler's folding: a table address stays one
// instruction with the context base in the lookup's offset, and an f32
// product stays rounded before it is narrowed
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// the same for a wave-uniform address, which stays in one SGPR pair;
// readfirstlane states the uniformity and costs nothing on a scalar value
typedef __attribute__((address_space(1))) uint8_t *gbyte_t;
__device__ __forceinline__ gbyte_t opaque_s(gbyte_t p) {
  uint64_t u = (uint64_t)p;
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u), hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  asm volatile("" : "+s"(lo), "+s"(hi));
  return (gbyte_t)(((uint64_t)hi << 32) | lo);
}

// a[i] for a wave-uniform i without indexing the kernel arguments by a
// register (which costs a dependent scalar load)
template <class T>
__device__ __forceinline__ T pick(const T (&a)[kContexts], uint32_t i) {
  uint32_t r = 0;
#pragma unroll
  for (uint32_t k = 0; k < (uint32_t)kContexts; ++k) r |= (uint32_t)a[k] & (0u - (uint32_t)(i == k));
  return (T)r;
}

// per-lane select by an SGPR lane mask: mask bit set -> if1.  Written as one
// instruction so that the compiler keeps the order of dependent selects.
__device__ __forceinline__ uint32_t select_mask(uint64_t mask, uint32_t if0, uint32_t if1) {
  uint32_t r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if0), "v"(if1), "s"(mask));
  return r;
}

// inclusive prefix sum over the 16 lanes of each DPP row
__device__ __forceinline__ uint32_t row16_inclusive_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  return v;
}

// inclusive prefix sum over the wavefront
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v = row16_inclusive_sum(v);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

__device__ __forceinline__ int32_t symbol_value(uint32_t c, int32_t s) {
  if (c == 0) return s;
  if (c <= 2) return 2 * s + (int32_t)(c - 1);
  const int32_t bp = (int32_t)c - 3;  // 2b + p
  return 4 * s + 2 * (bp & 1) + (bp >> 1);
}

// Per-lane pipeline state of a tile's decode.
struct Lane {
  uint32_t d0, d1;  // this step's table entry (the lookup is in flight when a step starts)
  uint32_t q;       // X >> 13 of this step's state
  uint32_t r;       // the state's next word (its read may be in flight when a step starts)
  uint32_t p;       // LDS byte address of that word
  uint32_t dp;      // +2 (even states read their region forward) or -2 (odd states, backward)
};

// BASE: the fixed part of the context's LDS address, folded into the
// instruction's offset
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const u32x2 *lds_u64_ptr;

template <uint32_t BASE>
__device__ __forceinline__ void table_read(uint32_t a, uint32_t &d0, uint32_t &d1) {
  const u32x2 v = *(lds_u64_ptr)(uintptr_t)(a + BASE);
  d0 = v.x;
  d1 = v.y;
}

// one rANS decode step of every active lane: decodes this step's symbol,
// issues the lookup for the next step (context base BASE + nb) and, in
// refilling lanes, the read of the following word; returns this step's entry.
// BOP3 forms the lookup address with v_bitop3 instead of v_and_or.
template <bool WIDE, uint32_t BASE, bool BOP3>
__device__ __forceinline__ uint32_t rans_step(Lane &L, uint32_t nb, bool active) {
  const uint32_t e = L.d0;
  uint32_t x;
  if constexpr (WIDE) {
    x = __umul24(e & 0x1fffu, L.q) + L.d1;  // v sits in bits 16..31, partly inside the 24-bit operand
  } else {
    x = __umul24(e, L.q) + L.d1;
  }
  // the word read last step returns right after this step's entry; using it
  // here (after the multiply-add, which starts the chain) keeps its use out
  // of the refill block
  uint32_t r8;
  asm volatile("v_lshlrev_b32 %0, 3, %1" : "=v"(r8) : "v"(L.r), "v"(x));
  const bool need = active && x < (kStateLow << 3);  // x' < L, in units of X = 8x
  const uint64_t m = __ballot(need);
  const uint32_t X = select_mask(m, x, (x << 16) | r8);  // next state: refilling lanes shift the held word in
  // the address (X & 0x1ff8) | nb; opaque keeps BASE in the lookup's offset
  // instead of an add into nb
  if constexpr (BOP3)
    table_read<BASE>(opaque(__builtin_amdgcn_bitop3_b32(X, 0x1ff8u, nb, 0xea)), L.d0, L.d1);  // truth table of (a & b) | c
  else
    table_read<BASE>(opaque((X & 0x1ff8u) | nb), L.d0, L.d1);
  __builtin_amdgcn_sched_barrier(0);  // the next lookup goes out before the refill
  if (need) {  // refilling lanes only: read the following word
    L.p += L.dp;
    L.r = lds_u16(L.p);
  }
  L.q = X >> 13;
  return e;
}

template <bool WIDE>
__device__ __forceinline__ int32_t entry_value(uint32_t e) {
  if constexpr (WIDE) return (int32_t)e >> 16;
  return (int32_t)e >> 24;
}

template <bool WIDE>
__device__ __forceinline__ float entry_weight(uint32_t e, float g) {
  // the value converts in place from its byte or half (SDWA); one rounding
  if constexpr (WIDE) return (float)(int16_t)(e >> 16) * g;
  return (float)(int8_t)(e >> 24) * g;
}

__device__ __forceinline__ uint32_t int8_byte(float y) {
  const float c = __builtin_fminf(__builtin_fmaxf(y, -127.0f), 127.0f);
  return __float_as_uint(c + 12582912.0f);  // 1.5 * 2^23: rounds to an integer, ties to even
}

// d with byte K replaced by int8_byte(y)'s low byte (K = 0: the other bytes
// cleared).  The add writes only its low byte, into byte K of d (SDWA
// destination select), so four of them pack a word with no shifts or perms.
template <int K>
__device__ __forceinline__ uint32_t int8_into(uint32_t d, float y, float magic) {
  const float c = __builtin_fminf(__builtin_fmaxf(y, -127.0f), 127.0f);
  if constexpr (K == 0)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD"
        : "=v"(d) : "v"(c), "v"(magic));
  else if constexpr (K == 1)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(d) : "v"(c), "v"(magic));
  else if constexpr (K == 2)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(d) : "v"(c), "v"(magic));
  else
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(d) : "v"(c), "v"(magic));
  return d;
}

__device__ __forceinline__ float fp8_clamp(float y) { return __builtin_fminf(__builtin_fmaxf(y, -448.0f), 448.0f); }

typedef float f2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

template <int OUT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  f2v v = {a, b};
  if constexpr (OUT == EP_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2v));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2v));
}

// writes one decoded vector: at dst (unpadded layouts), or, with PADDED,
// the C mod 8 leading elements of global vector vec element by element
template <int OUT, bool WIDE, bool PADDED>
__device__ __forceinline__ void emit_vector(const Args &A, gbyte_t dst, uint32_t vec, const uint32_t (&e)[8],
                                            float g) {
  if constexpr (OUT == kOutSym) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = ((uint32_t)entry_value<WIDE>(e[2 * k]) & 0xffffu) | ((uint32_t)entry_value<WIDE>(e[2 * k + 1]) << 16);
    const u32x4 pk = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(pk, (__attribute__((address_space(1))) u32x4 *)dst);
    return;
  } else {
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = entry_weight<WIDE>(e[j], g);
    if constexpr (!PADDED) {
      if constexpr (OUT == EP_BF16 || OUT == EP_FP16) {
        const u32x4 pk = {pack2<OUT>(y[0], y[1]), pack2<OUT>(y[2], y[3]), pack2<OUT>(y[4], y[5]), pack2<OUT>(y[6], y[7])};
        __builtin_nontemporal_store(pk, (__attribute__((address_space(1))) u32x4 *)dst);
      } else if constexpr (OUT == EP_FP8_E4M3FN) {
        // the first conversion of each word fills its low half; the high half
        // it keeps (here the first input's bits) is overwritten by the second,
        // so the word needs no zeroing first
        const float c0 = fp8_clamp(y[0]), c4 = fp8_clamp(y[4]);
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c0, fp8_clamp(y[1]), __float_as_int(c0), false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(y[2]), fp8_clamp(y[3]), lo, true);
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c4, fp8_clamp(y[5]), __float_as_int(c4), false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(y[6]), fp8_clamp(y[7]), hi, true);
        const u32x2 pk = {(uint32_t)lo, (uint32_t)hi};
        __builtin_nontemporal_store(pk, (__attribute__((address_space(1))) u32x2 *)dst);
      } else {
        const float magic = 12582912.0f;
        uint32_t lo = 0, hi = 0;
        lo = int8_into<0>(lo, y[0], magic);
        hi = int8_into<0>(hi, y[4], magic);
        lo = int8_into<1>(lo, y[1], magic);
        hi = int8_into<1>(hi, y[5], magic);
        lo = int8_into<2>(lo, y[2], magic);
        hi = int8_into<2>(hi, y[6], magic);
        lo = int8_into<3>(lo, y[3], magic);
        hi = int8_into<3>(hi, y[7], magic);
        const u32x2 pk = {lo, hi};
        __builtin_nontemporal_store(pk, (__attribute__((address_space(1))) u32x2 *)dst);
      }
    } else {
      const uint32_t r = vec / A.vpr, k = vec - r * A.vpr;
      const uint64_t base = (uint64_t)r * A.cols + 8ull * k;
      const uint32_t left = (uint32_t)(A.cols - 8ull * k);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((uint32_t)j >= left) break;
        if constexpr (OUT == EP_BF16 || OUT == EP_FP16) {
          // y is hidden from the conversion: otherwise the compiler folds the
          // multiply and the narrowing into one v_fma_mixlo_f16, a single
          // rounding where the reconstruction rounds to f32 first
          const float yj = __uint_as_float(opaque(__float_as_uint(y[j])));
          reinterpret_cast<uint16_t *>(A.out)[base + j] = (uint16_t)(pack2<OUT>(yj, 0.0f) & 0xffffu);
        } else if constexpr (OUT == EP_FP8_E4M3FN) {
          reinterpret_cast<uint8_t *>(A.out)[base + j] =
              (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(y[j]), 0.0f, 0, false) & 0xff);
        } else {
          reinterpret_cast<uint8_t *>(A.out)[base + j] = (uint8_t)(int8_byte(y[j]) & 0xffu);
        }
      }
    }
  }
}

// the row of vector vec (the last row for vectors past the end)
__device__ __forceinline__ uint32_t row_of(const Args &A, uint32_t vec) {
  const uint32_t last = A.rows - 1u, one = A.vpr == 1u ? 0xffffffffu : 0u;
  const uint32_t r = ((__umulhi(vec, A.row_magic) >> A.row_shift) & ~one) | (vec & one);
  return r < last ? r : last;
}

// the row scale of vector vec (the last row's for vectors past the end)
__device__ __forceinline__ float row_scale(const Args &A, uint32_t vec) { return A.scales[row_of(A, vec)]; }

// The lanes of a wave's unit: unit u holds tiles u * 64/NS .. (64/NS tiles of
// NS states; lanes 16r.. hold tile r's states when NS = 16).
struct UnitLane {
  uint32_t tile;  // the lane's tile (the stream's last for a tile past its end)
  uint32_t q;     // the lane's state in its tile
  uint32_t n;     // vectors in the lane's tile (0 past the stream's end)
  uint32_t row;   // the row of the tile's first vector
  bool one_row;   // wave-uniform: every lane's tile lies in one row of the matrix
};

template <int NS, int V>
__device__ __forceinline__ UnitLane unit_lane(const Args &A, uint32_t unit, uint32_t lane) {
  constexpr uint32_t kTv = (uint32_t)(NS * V);
  UnitLane u;
  const uint32_t t = unit * (64u / NS) + lane / NS;
  u.q = lane % NS;
  const bool have = t < A.n_tiles;
  u.tile = have ? t : A.n_tiles - 1u;
  u.n = have ? min(kTv, A.n_vec - t * kTv) : 0u;
  u.row = row_of(A, u.tile * kTv);
  const bool split = u.n > 1u && row_of(A, u.tile * kTv + u.n - 1u) != u.row;
  u.one_row = __ballot(split) == 0;
  return u;
}

// the row scales of lane's vectors 8g .. 8g + 7 (lanes past the end read the
// last row; their values are unused).  Tiles inside one row (every tile when
// the rows hold whole tiles) take one scale for all.
template <int NS, int V>
__device__ __forceinline__ void group_scales(const Args &A, const UnitLane &u, uint32_t g, float (&gs)[8]) {
  constexpr uint32_t kTv = (uint32_t)(NS * V);
  if (u.one_row) {
    const float v = A.scales[u.row];
#pragma unroll
    for (uint32_t s = 0; s < 8; ++s) gs[s] = v;
    return;
  }
#pragma unroll
  for (uint32_t s = 0; s < 8; ++s) gs[s] = row_scale(A, u.tile * kTv + (8u * g + s) * NS + u.q);
}

// wave priority (s_setprio): the SIMD's arbiter issues from higher-priority
// waves first
template <uint32_t P>
__device__ __forceinline__ void set_priority() {
  __builtin_amdgcn_s_setprio((int16_t)P);
}

// Priority by the work still ahead of a wave, in quarters of the largest
// load any wave of the workgroup carries: 3 with more than three quarters of
// that left, down to 0.  Among waves of equal priority a SIMD issues from the
// oldest first, so without this the oldest waves race through their units and
// the youngest decode their last ones nearly alone; raising the waves with
// the most left (the longest remaining first) keeps all of them busy to the
// end.  left, most: groups of 8 vectors (most 0: leave the priority).
__device__ __forceinline__ void priority_by_work_left(uint32_t left, uint32_t most) {
  if (most == 0u) return;
  const uint32_t left4 = (4u * left + most - 1u) / most;  // ceil(4 * left / most), 1..4
  if (left4 >= 4u) set_priority<3>();
  else if (left4 == 3u) set_priority<2>();
  else if (left4 == 2u) set_priority<1>();
  else set_priority<0>();
}

// A lane's start: its state (as X = 8x) and its word pointer, with the first
// word read.  wt, we: LDS byte addresses of the first word of the lane's
// tile and of its end.  The lane reads its start state (length nibble, bit
// offset by a prefix sum over its tile's states, three 16-bit reads) and its
// first word (pair counts' prefix sum; odd states start at their region's
// end and read backwards).  Reads the tile's words only, not the tables.
struct Start {
  uint32_t X;
  Lane L;
};
template <int NS>
__device__ __forceinline__ Start parse_start(const UnitLane &u, uint32_t wt, uint32_t we, uint32_t lane) {
  constexpr uint32_t kNs = (uint32_t)NS;
  const uint32_t q = u.q;
  // ---- start state: W - 1 bits after the bits of the states before it
  const uint32_t nb = ((lds_u8(wt + kNs / 2u + (q >> 1)) >> ((q & 1u) << 2)) & 15u) + 11u;
  const uint32_t bincl = NS == 64 ? wave_inclusive_sum(nb) : row16_inclusive_sum(nb);
  const uint32_t bo = bincl - nb;
  const uint32_t btotal = NS == 64 ? (uint32_t)__builtin_amdgcn_readlane((int)bincl, 63)
                                   : (uint32_t)__builtin_amdgcn_ds_bpermute((int)((lane | 15u) << 2), (int)bincl);
  const uint32_t wa = wt + kNs + ((bo >> 4) << 1);
  const uint32_t lo = lds_u16(wa) | (lds_u16(wa + 2u) << 16), hi = lds_u16(wa + 4u);
  const uint32_t x = (__builtin_amdgcn_alignbit(hi, lo, bo & 15u) & ((1u << nb) - 1u)) | (1u << nb);
  // ---- first word: pair k's region starts after the regions before it
  const uint32_t pc = (q & 1u) ? 0u : lds_u8(wt + (q >> 1));
  const uint32_t pincl = NS == 64 ? wave_inclusive_sum(pc) : row16_inclusive_sum(pc);
  const uint32_t region = wt + kNs + (((btotal + 15u) >> 4) << 1);
  uint32_t p = (q & 1u) ? region + 2u * pincl - 2u : region + 2u * (pincl - pc);
  p = p < wt ? wt : (p > we ? we : p);  // a corrupt tile's pointers stay inside it
  Start S;
  S.L.dp = (q & 1u) ? 0xfffffffeu : 2u;
  S.L.p = p;
  S.L.r = lds_u16(p);
  S.X = x << 3;
  return S;
}

// Decodes a wave's unit from its lanes' starts: V vectors per lane in groups
// of 8, each group's row scales loaded during the group before (gs0: the
// first group's).  PARTIAL: some lane's tile holds fewer vectors than a full
// one (the stream's last unit).
template <int OUT, bool WIDE, bool PADDED, bool PARTIAL, bool BOP3, int NS, int V, bool PRIO>
__device__ __forceinline__ void decode_unit(const Args &A, const UnitLane &u, const Start &S0, const float (&gs0)[8],
                                            uint32_t lane, uint32_t left, uint32_t most) {
  static_assert((NS == 64 && (V == 8 || V == 16)) || (NS == 16 && (V == 32 || V == 64)), "tile geometry");
  constexpr uint32_t kNs = (uint32_t)NS, kTv = (uint32_t)(NS * V), kGroups = (uint32_t)V / 8u;
  const uint32_t q = u.q;
  Lane L = S0.L;
  table_read<0u>(S0.X & 0x1ff8u, L.d0, L.d1);  // context F
  L.q = S0.X >> 13;
  constexpr uint32_t kC = kCtxBytes, kE = 3u * kCtxBytes;  // LDS bases of C_0 and E_{0,0}
  constexpr uint32_t kBitB = WIDE ? 16u : 24u;  // where bit 0 of v sits in d0
  constexpr uint32_t kVecBytes = (OUT == EP_FP8_E4M3FN || OUT == EP_INT8) ? 8u : 16u;
  const uint32_t tile = u.tile, n = u.n;
  float gs[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) gs[s] = gs0[s];
#pragma unroll 1
  for (uint32_t grp = 0; grp < kGroups; ++grp) {
    if constexpr (PRIO) priority_by_work_left(left - grp, most);
    float gn[8];
    if (grp + 1u < kGroups && !u.one_row) group_scales<NS, V>(A, u, grp + 1u, gn);  // one row: gs holds its scale
#pragma unroll
    for (uint32_t s8 = 0; s8 < 8; ++s8) {
      const uint32_t s = grp * 8u + s8;  // step
      const uint32_t i = s * kNs + q;    // the lane's vector in its tile
      const bool act = PARTIAL ? i < n : true;
      uint32_t e[8];
      // C_b at LDS context 1 + b; the coset bit is in the entry of coordinate 0
      const uint32_t cb = __builtin_amdgcn_ubfe(L.d0, kBitB, 1u) << 13;
      e[0] = rans_step<WIDE, kC, BOP3>(L, cb, act);
#pragma unroll
      for (int j = 1; j < 6; ++j) e[j] = rans_step<WIDE, kC, BOP3>(L, cb, act);
      // the XOR's copy of v's bit 0 is b (all eight coordinates share it), its
      // copy of bit 1 is p
      uint32_t acc = __builtin_amdgcn_bitop3_b32(e[0], e[1], e[2], 0x96);
      acc = __builtin_amdgcn_bitop3_b32(acc, e[3], e[4], 0x96);
      acc = __builtin_amdgcn_bitop3_b32(acc, e[5], L.d0, 0x96);
      const uint32_t eb = __builtin_amdgcn_ubfe(acc, kBitB, 2u) << 13;
      e[6] = rans_step<WIDE, kE, BOP3>(L, eb, act);
      e[7] = rans_step<WIDE, 0u, BOP3>(L, 0u, act);
      if (act) {
        // one tile per wave: the step's 64 vectors are one run at a
        // wave-uniform address; four tiles: each row's 16 vectors are one
        gbyte_t dst;
        if constexpr (NS == 64)
          dst = opaque_s((gbyte_t)A.out + ((uint64_t)tile * kTv + s * kNs) * kVecBytes) + kVecBytes * lane;
        else
          dst = (gbyte_t)A.out + ((uint64_t)tile * kTv + i) * kVecBytes;
        emit_vector<OUT, WIDE, PADDED>(A, dst, tile * kTv + i, e, gs[s8]);
      }
    }
    if (grp + 1u < kGroups && !u.one_row) {
#pragma unroll
      for (int s = 0; s < 8; ++s) gs[s] = gn[s];
    }
  }
}

// The table build, per context: prefix sums of the frequencies (DPP scan),
// the used symbols' records, a bitmap of the slots where a symbol starts,
// then the context's 16 table rows of 64 slots, where a slot's record is the
// number of starts up to it (v_mbcnt over the row's bitmap).
//
// context_rows: everything up to the rows.  Returns, in lane t < 16, row
// t's row descriptor: its start bits shifted down by one (lo, hi) and the
// record index before it.  fpre holds the first 256 frequency slots of
// context `wave` (loaded early; slots past its symbols are masked here).
struct RowDesc {
  uint32_t lo, hi, base;
};
__device__ __forceinline__ RowDesc context_rows(const Args &A, uint8_t *lds, uint32_t c, uint32_t wave, uint32_t lane,
                                               const uint32_t (&fpre)[4], bool wide) {
  const uint16_t *freq = A.freq;
  uint2 *rec = reinterpret_cast<uint2 *>(lds + A.rec_off);          // (d0, cum term) per used symbol
  uint32_t *mark = reinterpret_cast<uint32_t *>(lds + A.mark_off);  // [ctx][32] start bits
  const uint32_t cf = pick(A.ctx_freq, c), n = cf >> 16, fidx = cf & 0xffffu, nzbase = pick(A.nzbase, c);
  const int32_t smin = pick(A.smin, c);
  if (lane < kMarkWords) mark[c * kMarkWords + lane] = 0u;
  uint32_t carry = 0, nzb = nzbase;
  // symbols base .. base + 63, lane's frequency f (0 past the context's end)
  auto chunk = [&](uint32_t base, uint32_t f) {
    const uint32_t s = base + lane;
    const uint32_t incl = wave_inclusive_sum(f);
    const uint32_t cum = carry + incl - f;
    const bool used = f != 0;
    const uint64_t m = __ballot(used);
    const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, nzb));
    if (used && cum < kProbTotal) {
      const int32_t v = symbol_value(c, smin + (int32_t)s);
      rec[r] = make_uint2((f << 3) | (wide ? ((uint32_t)v & 0xffffu) << 16 : ((uint32_t)v & 0xffu) << 24), cum << 3);
      atomicOr(&mark[c * kMarkWords + (cum >> 5)], 1u << (cum & 31u));
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
    nzb += (uint32_t)__popcll(m);
  };
  // The first 256 symbols of the wave's own context come from fpre, with
  // the loop unrolled so that each use waits for its own load only.
  if (c == wave) {
#pragma unroll
    for (uint32_t i = 0; i < 4; ++i)
      if (64u * i < n) chunk(64u * i, 64u * i + lane < n ? fpre[i] : 0u);
  }
  for (uint32_t base = c == wave ? 256u : 0u; base < n; base += 64) {
    const uint32_t s = base + lane;
    chunk(base, s < n ? freq[fidx + s] : 0u);
  }
  RowDesc d{0u, 0u, 0u};
  uint32_t lo = 0, hi = 0;
  if (lane < kRows) {
    lo = mark[c * kMarkWords + 2 * lane];
    hi = mark[c * kMarkWords + 2 * lane + 1];
  }
  const uint32_t cnt = (uint32_t)(__popc(lo) + __popc(hi));
  const uint32_t first = nzbase + row16_inclusive_sum(cnt) - cnt;
  d.lo = __builtin_amdgcn_alignbit(hi, lo, 1u);
  d.hi = hi >> 1;
  d.base = first + (lo & 1u) - 1u;
  return d;
}

// LDS context index of context c: F, C_0, C_1, then E_{b,p} at 3 + b + 2p
__device__ __forceinline__ uint32_t lds_context(uint32_t c) {
  return c < 3u ? c : 3u + ((c - 3u) >> 1) + 2u * ((c - 3u) & 1u);
}

// slot record = first + (starts at or below the slot) - 1
//             = base + popcount of (lo, hi) below the lane.
__device__ __forceinline__ uint32_t slot_record(uint32_t lo, uint32_t hi, uint32_t base) {
  return __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, base));
}

// One wave builds whole contexts: waves 0..k-1 take contexts wave, wave + k,
// ...  The row descriptors reach every lane through LDS: lanes 0..15 store
// them in the wave's own 256 bytes and each row's is read back with one
// uniform (broadcast) read, three VALU instructions per row fewer than
// v_readlane broadcasts need.  All sixteen records are read before any
// table write: the compiler cannot tell the record list and the table apart,
// so interleaving would put an LDS round trip on every row.
template <bool WIDE>
__device__ __forceinline__ void build_tables(const Args &A, uint8_t *lds, uint32_t wave, uint32_t lane, uint32_t k,
                                             const uint32_t (&fpre)[4]) {
  typedef __attribute__((address_space(3))) u32x4 *lds_u128_ptr;
  typedef __attribute__((address_space(3))) const u32x2 *lds_u64_cptr;
  uint32_t *tab = reinterpret_cast<uint32_t *>(lds);
  const uint32_t dsc = A.desc_off + 256u * wave;  // this wave's row descriptors
  for (uint32_t c = wave; c < (uint32_t)kContexts; c += k) {
    if ((pick(A.ctx_freq, c) >> 16) == 0u) continue;  // context without symbols: its table is never read
    const RowDesc d = context_rows(A, lds, c, wave, lane, fpre, WIDE);
    const uint32_t lc = lds_context(c);
    // (lo, hi, LDS address of the record before the row)
    if (lane < kRows) *(lds_u128_ptr)(uintptr_t)(dsc + 16u * lane) = u32x4{d.lo, d.hi, A.rec_off + 8u * d.base, 0u};
    u32x2 rc[kRows];
#pragma unroll
    for (uint32_t row = 0; row < kRows; ++row) {
      const u32x4 r = *(lds_u128_ptr)(uintptr_t)(dsc + 16u * row);
      rc[row] = *(lds_u64_cptr)(uintptr_t)(r.z + 8u * slot_record(r.x, r.y, 0u));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (uint32_t row = 0; row < kRows; ++row) {
      const uint32_t slot = row * 64u + lane, idx = 2u * (lc * kProbTotal + slot);
      tab[idx] = rc[row].x;
      tab[idx + 1u] = (slot << 3) - rc[row].y;
    }
  }
}

// Multi-tile kernel: workgroup b decodes the consecutive units
// [wg_first(b), wg_first(b + 1)); the counts differ by at most one unit.
__device__ __forceinline__ uint32_t wg_first(const Args &A, uint32_t b) {
  return b * A.wg_q + (b < A.wg_rem ? b : A.wg_rem);
}

// What a wave needs to decode one unit: its lanes' tiles, the row scales of
// each lane's first 8 vectors, and where the lane's tile's words land in LDS.
struct UnitIn {
  UnitLane u;
  float gs[8];
  uint32_t wt, we;  // LDS byte addresses of the lane's tile's first word and of its end
};

// The 16-byte pieces of the word section that hold words [w_lo, w_hi):
// pieces c0 .. c1 - 1.
__device__ __forceinline__ uint32_t first_piece(uint32_t w_lo) { return w_lo >> 3; }
__device__ __forceinline__ uint32_t end_piece(uint32_t w_hi) { return (w_hi + 7u) >> 3; }

// Copies pieces [c0, c1) of the word section into LDS at buf, 1 KB per
// instruction; lanes past the end of the last, partial kilobyte re-read its
// last piece.  Blocks k0, k0 + dk, ... are this wave's share.
__device__ __forceinline__ void copy_pieces(const Args &A, uint8_t *lds, uint32_t c0, uint32_t c1, uint32_t buf,
                                            uint32_t lane, uint32_t k0, uint32_t dk) {
  const uint32_t n = c1 - c0;
  const gbyte_t src = (gbyte_t)(A.words + 16ull * c0);
  for (uint32_t i = k0; 64u * i < n; i += dk) {
    const uint32_t ch = 64u * i + lane;
    __builtin_amdgcn_global_load_lds((gptr_t)(src + 16u * (ch < n ? ch : n - 1u)), (lptr_t)(lds + buf + 1024u * i),
                                     16, 0, 0);
  }
}

// The same copy through registers, for waves that also build tables (after
// a copy straight into LDS the compiler makes every later LDS access of the
// wave wait for it).  stage_pieces loads the wave's first kStage blocks
// (blocks k0, k0 + dk, ...; every lane loads, lanes past the end re-reading
// the last piece, so that no load sits behind a branch and each wait counts
// exactly); store_pieces writes them and copies any further blocks.
constexpr uint32_t kStage = 4;
__device__ __forceinline__ void stage_pieces(const Args &A, uint32_t c0, uint32_t c1, uint32_t lane, uint32_t k0,
                                             uint32_t dk, u32x4 (&cp)[kStage]) {
  const uint32_t n = c1 - c0;
  const gbyte_t src = (gbyte_t)(A.words + 16ull * c0);
#pragma unroll
  for (uint32_t i = 0; i < kStage; ++i) {
    const uint32_t ch = 64u * (k0 + i * dk) + lane;
    cp[i] = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)(src + 16ull * (ch < n ? ch : n - 1u)));
  }
}
__device__ __forceinline__ void store_pieces(const Args &A, uint32_t c0, uint32_t c1, uint32_t buf, uint32_t lane,
                                             uint32_t k0, uint32_t dk, const u32x4 (&cp)[kStage]) {
  typedef __attribute__((address_space(3))) u32x4 *lds_u128_ptr;
  const uint32_t n = c1 - c0;
#pragma unroll
  for (uint32_t i = 0; i < kStage; ++i) {
    const uint32_t ch = 64u * (k0 + i * dk) + lane;
    if (ch < n) *(lds_u128_ptr)(uintptr_t)(buf + 16u * ch) = cp[i];
  }
  const gbyte_t src = (gbyte_t)(A.words + 16ull * c0);
  for (uint32_t b = k0 + kStage * dk; 64u * b < n; b += dk) {
    const uint32_t ch = 64u * b + lane;
    if (ch < n)
      *(lds_u128_ptr)(uintptr_t)(buf + 16u * ch) =
          __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)(src + 16ull * ch));
  }
}

// Issues a unit's loads: its lanes' tile offsets and row scales (vector
// loads), the unit's word range (scalar loads), and the copy of its words
// into LDS at buf.  Only the copy's addresses wait, for the word range.
template <int NS, int V>
__device__ __forceinline__ UnitIn issue_unit(const Args &A, uint8_t *lds, uint32_t unit, uint32_t buf,
                                             uint32_t lane) {
  UnitIn T;
  T.u = unit_lane<NS, V>(A, unit, lane);
  group_scales<NS, V>(A, T.u, 0u, T.gs);
  const uint32_t tb = A.toff[T.u.tile], te = A.toff[T.u.tile + 1u];
  typedef __attribute__((address_space(4))) const uint32_t *cptr_u32;
  const cptr_u32 toff = (cptr_u32)A.toff;
  const uint32_t t0 = unit * (64u / NS), t1 = min(t0 + 64u / NS, A.n_tiles);
  const uint32_t c0 = first_piece(toff[t0]);
  copy_pieces(A, lds, c0, end_piece(toff[t1]), buf, lane, 0u, 1u);
  T.wt = buf + 2u * tb - 16u * c0;
  T.we = T.wt + 2u * (te - tb);
  return T;
}

// workgroup barrier that orders LDS accesses: every LDS access before it has
// completed, none after it has started
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// the first 256 frequency slots of this wave's first context, which need
// nothing but the kernel arguments; slots past the context's symbols hold
// its first frequency and are masked where they are used
__device__ __forceinline__ void first_frequencies(const Args &A, uint32_t wave, uint32_t lane, uint32_t (&fpre)[4]) {
  // one scalar load of the argument word (a select over the seven would
  // cost fourteen scalar instructions, and the workgroup's waves share one
  // scalar unit)
  const uint32_t cf = A.ctx_freq[__builtin_amdgcn_readfirstlane(wave < (uint32_t)kContexts ? wave : 0u)];
  const uint32_t n0 = cf >> 16, f0 = cf & 0xffffu;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t s = 64u * i + lane;
    fpre[i] = A.freq[f0 + (s < n0 ? s : 0u)];
  }
}

// PRIO: set the wave's priority by the work left to it (left, from this unit
// on) against the most any wave of its workgroup carries (most), both in
// groups of 8 vectors
template <int OUT, bool WIDE, bool PADDED, bool BOP3, int NS, int V, bool PRIO = false>
__device__ __forceinline__ void decode_unit_any(const Args &A, const UnitLane &u, const Start &S, const float (&gs)[8],
                                                uint32_t lane, uint32_t left = 0u, uint32_t most = 0u) {
  constexpr uint32_t kTv = (uint32_t)(NS * V);
  if (__ballot(u.n != kTv) == 0)
    decode_unit<OUT, WIDE, PADDED, false, BOP3, NS, V, PRIO>(A, u, S, gs, lane, left, most);
  else
    decode_unit<OUT, WIDE, PADDED, true, BOP3, NS, V, PRIO>(A, u, S, gs, lane, left, most);
}

// Streams with more units than one round of workgroups covers: one
// workgroup per CU builds the tables once, then each of its k waves decodes
// units first + wave, first + wave + k, ... of the workgroup's run on its
// own, copying each unit's words into a buffer of its own.  After the tables
// no wave waits for another: while one waits for its next unit's loads, the
// other waves of its SIMD keep the VALU busy (four waves per SIMD cover the
// decode chain's latency).
template <int OUT, bool WIDE, bool PADDED, int NS, int V, bool PRIO>
__global__ void __launch_bounds__(64 * kMaxWaves) decode_waves_kernel(Args A) {
  extern __shared__ __align__(16) uint8_t lds[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t k = A.waves;
  const uint32_t end = wg_first(A, blockIdx.x + 1u);
  const uint32_t buf = A.words_off + wave * A.wbuf;  // this wave's word buffer
  constexpr bool kNarrowOut = OUT == EP_FP8_E4M3FN || OUT == EP_INT8;  // lookup address by v_bitop3

  // the arguments the first loads need, read in one round of scalar loads
  asm volatile("" ::"s"(A.freq), "s"(A.toff), "s"(A.words), "s"(A.waves), "s"(A.n_tiles), "s"(A.wg_q),
               "s"(A.wg_rem));
  uint32_t unit = wg_first(A, blockIdx.x) + wave;
  const uint32_t uc = unit < end ? unit : end - 1u;  // waves without a unit load a valid one and drop it
  // Waves that build no table copy their first unit's words into LDS now and
  // start decoding right after the barrier.  The table builders (at raised
  // priority until their table is built) issue theirs after their table: the
  // compiler waits for every copy into LDS before the wave's next LDS access.
  // (Loading a builder's first words into registers before its build and
  // storing them after it measured 1% faster on 8192^2 INT8 and 6% slower on
  // 3072x12288.)
  const bool builder = wave < (uint32_t)kContexts;
  UnitIn T;
  if (builder) {
    set_priority<2>();
    uint32_t fpre[4];
    first_frequencies(A, wave, lane, fpre);
    build_tables<WIDE>(A, lds, wave, lane, k, fpre);
    set_priority<0>();
    T = issue_unit<NS, V>(A, lds, uc, buf, lane);
  } else {
    T = issue_unit<NS, V>(A, lds, uc, buf, lane);
  }
  lds_barrier();  // tables built (every wave's LDS writes done)

  // PRIO (every wave of every workgroup has the same number of units): work
  // left to this wave and the most any wave of the workgroup has, in groups of
  // 8 vectors, for its priority.  When some waves have one unit more, those
  // are the oldest (units go to waves in turn), which the SIMD's oldest-first
  // issue already favours; priorities measured 2% slower there (3072x12288:
  // 18 units on 16 waves).
  constexpr uint32_t kGroups = (uint32_t)V / 8u;
  const uint32_t most = kGroups * ((end - wg_first(A, blockIdx.x)) / k);
  uint32_t left = unit < end ? kGroups * ((end - unit + k - 1u) / k) : 0u;
  while (unit < end) {
    __builtin_amdgcn_s_waitcnt(0);  // the unit's offsets, scales and words have landed
    decode_unit_any<OUT, WIDE, PADDED, kNarrowOut, NS, V, PRIO>(A, T.u, parse_start<NS>(T.u, T.wt, T.we, lane), T.gs,
                                                                lane, left, most);
    left -= kGroups;
    unit += k;
    if (unit < end) {
      __builtin_amdgcn_s_waitcnt(0);  // every read of the finished unit's words is done before they are overwritten
      T = issue_unit<NS, V>(A, lds, unit, buf, lane);
    }
  }
}

// Kernel arguments of the single-round kernel: the common ones and the first
// word of each workgroup's range of tile words (entry `grid`: the end of the
// last range).  Scalar loads from the arguments cost one short round trip at
// the start of a wave; loading these words from the tile offsets would put a
// memory round trip in front of the word copy.
constexpr uint32_t kMaxRoundWgs = 256;
struct RoundArgs {
  Args a;
  uint32_t wg_word[kMaxRoundWgs + 1];
};

// Streams that one round of workgroups covers: workgroups of up to 16 waves,
// one unit each.  Waves 0..6 build one context's table each (at raised
// priority: until the tables exist nothing else can decode); the others copy
// the workgroup's words into LDS with global_load_lds, 1 KB per instruction,
// each taking every (waves - 7)th kilobyte.  With fewer than eight waves
// every wave builds, and each also copies its share through registers.  Every wave then decodes its
// unit.  The two kinds of wave run separate code up to the barrier: after a
// copy into LDS the compiler waits for every load before the next LDS
// access, which a table builder must not do.
template <int OUT, bool WIDE, bool PADDED, int NS, int V>
__global__ void __launch_bounds__(64 * kMaxWaves) decode_kernel(RoundArgs R) {
  extern __shared__ __align__(16) uint8_t lds[];
  const Args &A = R.a;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t nwaves = A.waves;
  // the arguments the first loads need, read in one round of scalar loads
  asm volatile("" ::"s"(A.freq), "s"(A.words), "s"(A.waves), "s"(A.n_units), "s"(A.n_tiles),
               "s"(R.wg_word[blockIdx.x]), "s"(R.wg_word[blockIdx.x + 1u]));
  const uint32_t builders = nwaves < (uint32_t)kContexts + 1u ? nwaves : (uint32_t)kContexts;
  const uint32_t unit = blockIdx.x * nwaves + wave;
  const bool has_unit = unit < A.n_units;
  // the workgroup's words: pieces c0 .. c1 - 1 of the word section
  const uint32_t c0 = first_piece(R.wg_word[blockIdx.x]), c1 = end_piece(R.wg_word[blockIdx.x + 1u]);
  UnitLane u;
  uint32_t tb, te;
  float gs[8];
  if (wave < builders) {
    set_priority<2>();
    uint32_t fpre[4];
    first_frequencies(A, wave, lane, fpre);
    // fewer than eight waves, all building tables: each also copies every
    // (waves)th block of the words, through registers
    const bool copies = builders == nwaves;
    u32x4 cp[kStage];
    if (copies) stage_pieces(A, c0, c1, lane, wave, nwaves, cp);
    __builtin_amdgcn_sched_barrier(0);
    u = unit_lane<NS, V>(A, has_unit ? unit : A.n_units - 1u, lane);
    tb = A.toff[opaque(u.tile)];  // vector loads: a scalar load's only wait, lgkmcnt(0), would also wait for LDS work
    te = A.toff[opaque(u.tile + 1u)];
    __builtin_amdgcn_sched_barrier(0);
    build_tables<WIDE>(A, lds, wave, lane, builders, fpre);
    set_priority<0>();
    if (copies) store_pieces(A, c0, c1, A.words_off, lane, wave, nwaves, cp);
    // first needed at the first store, a vector's decode after the barrier,
    // so the barrier does not wait for them
    group_scales<NS, V>(A, u, 0u, gs);
  } else {
    copy_pieces(A, lds, c0, c1, A.words_off, lane, wave - builders, nwaves - builders);
    __builtin_amdgcn_sched_barrier(0);
    u = unit_lane<NS, V>(A, has_unit ? unit : A.n_units - 1u, lane);
    tb = A.toff[opaque(u.tile)];
    te = A.toff[opaque(u.tile + 1u)];
    group_scales<NS, V>(A, u, 0u, gs);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed in LDS
  }
  lds_barrier();  // tables built, words copied

  if (!has_unit) return;
  const uint32_t wt = A.words_off + 2u * tb - 16u * c0;  // LDS address of the tile's first word
  decode_unit_any<OUT, WIDE, PADDED, true, NS, V>(A, u, parse_start<NS>(u, wt, wt + 2u * (te - tb), lane), gs, lane);
}

// ---------------------------------------------------------------------------
// Streams in the blocks layout: each tile is a 64 x 64 block of W (rows
// 64 nb .., columns 64 kb ..; local vector i at block row i / 8, vector
// column i % 8), so lane q decodes, at step s, the vector of block row
// 8 s + q / 8 and vector column q % 8.  A vector of 8 consecutive weights of
// one row is exactly what one lane supplies to a BF16 matrix-core multiply
// as its B operand (8 consecutive k of one column n of B = W^T), so the
// decoded block goes to LDS as it is and feeds the MFMA.
//
// Fused linear Y = X W^T (X: M x K BF16, W: N x K in the stream, Y: M x N).
// A workgroup of 8 waves owns the output block of kLinRows * RB rows of X
// (RB row-blocks of 16 per wave) and one block row of W (64 output columns):
//   1. waves 0..6 build the tables (one context each);
//   2. per chunk of up to 8 consecutive tiles of the block row (512 columns
//      of K): all waves copy the chunk's words into LDS; wave j decodes tile
//      j of the chunk, multiplies by the row scales, rounds to BF16 and
//      writes the block into LDS slot j (64 rows of 144 bytes: 128 of data
//      and 16 of pad, so the 16 rows one B read touches fall in distinct
//      banks); then every wave multiplies its rows of X by the chunk's
//      blocks with v_mfma_f32_16x16x32_bf16, A fragments loaded straight
//      from global memory (16 bytes of one row of X per lane);
//   3. the FP32 accumulators go to Y (FP32 or BF16, rounded to nearest even).
// The same kernel decodes blocks-layout streams for ep_decompress (BF16
// weights) and ep_decode_symbols (int16 coordinates), one chunk per
// workgroup, writing each vector to global memory instead of LDS.
constexpr int kLinWaves = 8;
constexpr uint32_t kSlotRowBytes = 144;
constexpr uint32_t kSlotBytes = 64 * kSlotRowBytes;
constexpr uint32_t kLinMaxChunk = 8;
enum LinMode : int { kLinGemm = 0, kLinWeights = 1, kLinSymbols = 2 };

struct LinArgs {
  Args a;                  // tables, scales, tile offsets, words; a.out: weights or symbols (modes 1, 2)
  const uint16_t *x;       // X, M x K BF16 row-major (GEMM)
  void *y;                 // Y, M x N (GEMM)
  uint32_t m, n, k;        // M; N = rows of W; K = columns of W
  uint32_t kb_n, nb_n;     // blocks per block row (ceil(K / 64)); block rows (ceil(N / 64))
  uint32_t chunks;         // chunks per block row: ceil(kb_n / chunk)
  uint32_t chunk;          // tiles per chunk (at most 8, as the LDS allows)
  uint32_t mb_n;           // GEMM: workgroups along M
  uint32_t slots_off;      // LDS byte offset of the block slots
  uint32_t y_f32;          // GEMM: Y is FP32 (1) or BF16 (0)
  uint32_t grid;           // workgroups
  uint32_t split, cps;     // GEMM: workgroups per output block along K; chunks (K-blocks for
                           // linear_waves_kernel) each
  float *part;             // split > 1: FP32 partial sums, split x M x N
  uint32_t waves_kernel;   // nonzero: the plan launches linear_waves_kernel with this many waves
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 *lds_u128_wptr;
typedef __attribute__((address_space(3))) const u32x4 *lds_u128_rptr;

// Workgroup b runs on XCD b % 8 (round-robin dispatch).  The logical index
// gives each XCD a contiguous run, so that the workgroups sharing one XCD's
// L2 share their rows of X (consecutive logical indices differ in the block
// row of W only).
__device__ __forceinline__ uint32_t xcd_logical(uint32_t b, uint32_t grid) {
  const uint32_t q = grid / 8u, r = grid % 8u, x = b % 8u, j = b / 8u;
  return x < r ? x * (q + 1u) + j : r * (q + 1u) + (x - r) * q + j;
}

// Decodes one block tile whose words are at LDS [wt, we): 8 steps, each
// giving the lane's vector of block row 8 s + lane / 8 to sink(s, act, e).
// present: bit s set where that vector exists (absent vectors come last in
// a lane's sequence: rows past the matrix, or a vector column past it).
// FULL: every vector of the tile exists (present is all ones), so that the
// refill test is the state comparison alone, with no per-lane mask in the
// serial chain.
template <bool WIDE, bool FULL, class Sink>
__device__ __forceinline__ void decode_block(uint32_t wt, uint32_t we, uint32_t lane, uint32_t present, Sink &&sink) {
  UnitLane u{};
  u.q = lane;
  const Start S0 = parse_start<64>(u, wt, we, lane);
  Lane L = S0.L;
  table_read<0u>(S0.X & 0x1ff8u, L.d0, L.d1);  // context F
  L.q = S0.X >> 13;
  constexpr uint32_t kC = kCtxBytes, kE = 3u * kCtxBytes;
  constexpr uint32_t kBitB = WIDE ? 16u : 24u;
#pragma unroll
  for (uint32_t s = 0; s < 8; ++s) {
    const bool act = FULL ? true : ((present >> s) & 1u) != 0u;
    uint32_t e[8];
    const uint32_t cb = __builtin_amdgcn_ubfe(L.d0, kBitB, 1u) << 13;
    e[0] = rans_step<WIDE, kC, true>(L, cb, act);
#pragma unroll
    for (int j = 1; j < 6; ++j) e[j] = rans_step<WIDE, kC, true>(L, cb, act);
    uint32_t acc = __builtin_amdgcn_bitop3_b32(e[0], e[1], e[2], 0x96);
    acc = __builtin_amdgcn_bitop3_b32(acc, e[3], e[4], 0x96);
    acc = __builtin_amdgcn_bitop3_b32(acc, e[5], L.d0, 0x96);
    const uint32_t eb = __builtin_amdgcn_ubfe(acc, kBitB, 2u) << 13;
    e[6] = rans_step<WIDE, kE, true>(L, eb, act);
    e[7] = rans_step<WIDE, 0u, true>(L, 0u, act);
    sink(s, act, e);
  }
}

// the 8 weights of a decoded vector as BF16, 16 bytes (zeros if absent)
template <bool WIDE>
__device__ __forceinline__ u32x4 block_weights(const uint32_t (&e)[8], float g, bool act) {
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = entry_weight<WIDE>(e[j], g);
  u32x4 pk = {pack2<EP_BF16>(y[0], y[1]), pack2<EP_BF16>(y[2], y[3]), pack2<EP_BF16>(y[4], y[5]),
              pack2<EP_BF16>(y[6], y[7])};
  if (!act) pk = u32x4{0u, 0u, 0u, 0u};
  return pk;
}

// The lane's A fragments of one block slot: rows row0 + 16 i + lane % 16 of
// X, 8 values at k = kbase + 32 h + 8 (lane / 16), h = 0, 1 (zeros past M or
// K; K is a multiple of 8, so a fragment is all in or all out).
template <int RB>
__device__ __forceinline__ void load_x(const LinArgs &P, uint32_t row0, uint32_t kbase, uint32_t lane,
                                       u32x4 (&a)[RB][2]) {
  const uint32_t lr = lane & 15u, lk = lane >> 4;
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t row = row0 + 16u * (uint32_t)i + lr, kg = kbase + 32u * (uint32_t)h + 8u * lk;
      const bool ok = row < P.m && kg < P.k;
      const uint64_t at = ok ? (uint64_t)row * P.k + kg : 0ull;
      const u32x4 v = *(const __attribute__((address_space(1))) u32x4 *)(P.x + at);
      a[i][h] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
}

// RB: 16-row blocks of X per wave (GEMM)
template <int MODE, bool WIDE, int RB>
__global__ void __launch_bounds__(64 * kLinWaves) linear_kernel(LinArgs P) {
  extern __shared__ __align__(16) uint8_t lds[];
  const Args &A = P.a;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t L = xcd_logical(blockIdx.x, P.grid);
  uint32_t nb, mb, c_begin, c_end, sp = 0u;
  if constexpr (MODE == kLinGemm) {
    // consecutive logical indices: the splits of one output block, then the
    // block rows of W, then the row blocks of X
    const uint32_t blk = L / P.split;
    sp = L - blk * P.split;
    mb = blk / P.nb_n;
    nb = blk - mb * P.nb_n;
    c_begin = sp * P.cps;
    c_end = min(c_begin + P.cps, P.chunks);
  } else {
    nb = L / P.chunks;
    mb = 0u;
    c_begin = L - nb * P.chunks;
    c_end = c_begin + 1u;
  }
  typedef __attribute__((address_space(4))) const uint32_t *cptr_u32;
  const cptr_u32 toff = (cptr_u32)A.toff;
  // the tables (waves 0..6, one context each); meanwhile the last wave copies
  // the first chunk's words into LDS
  if (wave < (uint32_t)kContexts) {
    uint32_t fpre[4];
    first_frequencies(A, wave, lane, fpre);
    build_tables<WIDE>(A, lds, wave, lane, (uint32_t)kContexts, fpre);
  } else if (wave == (uint32_t)kLinWaves - 1u) {
    const uint32_t kb0 = c_begin * P.chunk, t0 = nb * P.kb_n + kb0, nt = min(P.chunk, P.kb_n - kb0);
    copy_pieces(A, lds, first_piece(toff[t0]), end_piece(toff[t0 + nt]), A.words_off, lane, 0u, 1u);
  }
  // the lane's block rows 8 s + lane / 8 and their scales (the last row's
  // past the matrix; those vectors are absent)
  const uint32_t r0 = 64u * nb + (lane >> 3), vcol = lane & 7u;
  float gs[8];
#pragma unroll
  for (uint32_t s = 0; s < 8; ++s) gs[s] = A.scales[min(r0 + 8u * s, A.rows - 1u)];
  uint32_t present_rows = 0;
#pragma unroll
  for (uint32_t s = 0; s < 8; ++s) present_rows |= (r0 + 8u * s < A.rows ? 1u : 0u) << s;

  constexpr int kCb = 4;  // 16-column blocks of the 64 output columns
  f32x4 acc[RB][kCb];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < kCb; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t m0 = (mb * (uint32_t)kLinWaves + wave) * 16u * (uint32_t)RB;  // the wave's first row of X

  for (uint32_t c = c_begin; c < c_end; ++c) {
    const uint32_t kb0 = c * P.chunk, nt = min(P.chunk, P.kb_n - kb0);
    const uint32_t t0 = nb * P.kb_n + kb0;
    const uint32_t p0 = first_piece(toff[t0]);
    // the chunk's words were copied during the table build (first chunk) or
    // during the last chunk's products; this barrier also ends every read of
    // the last chunk's slots
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    // GEMM: the A fragments of the chunk's first kRing - 1 slots load during
    // its decode; each later slot's load leaves kRing - 1 slots ahead of its
    // use.  With few rows per wave a slot's products are too short to cover
    // a load, so the whole chunk's fragments load during the decode.
    constexpr uint32_t kRing = RB == 1 ? kLinMaxChunk + 1u : (RB == 2 ? 4u : 3u);
    u32x4 xa[kRing][RB][2];
    if constexpr (MODE == kLinGemm) {
#pragma unroll
      for (uint32_t i = 0; i + 1u < kRing; ++i)
        if (i < nt && m0 < P.m) load_x<RB>(P, m0, 64u * (kb0 + i), lane, xa[i]);
    }
    if (wave < nt) {
      const uint32_t t = t0 + wave;
      const uint32_t tb = toff[t], te = toff[t + 1u];
      const uint32_t wt = A.words_off + 2u * tb - 16u * p0;
      const uint32_t kv = 8u * (kb0 + wave) + vcol;  // the lane's vector column in W
      const uint32_t present = kv < A.vpr ? present_rows : 0u;
      const bool full = __ballot(present != 0xffu) == 0;
      // one decode of the tile through sink, in its whole-block or edge form
      auto decode = [&](auto &&sink) {
        if (full)
          decode_block<WIDE, true>(wt, wt + 2u * (te - tb), lane, present, sink);
        else
          decode_block<WIDE, false>(wt, wt + 2u * (te - tb), lane, present, sink);
      };
      if constexpr (MODE == kLinGemm) {
        const uint32_t slot = P.slots_off + wave * kSlotBytes + (lane >> 3) * kSlotRowBytes + 16u * vcol;
        decode([&](uint32_t s, bool act, const uint32_t(&e)[8]) {
          *(lds_u128_wptr)(uintptr_t)(slot + 8u * s * kSlotRowBytes) = block_weights<WIDE>(e, gs[s], act);
        });
      } else if constexpr (MODE == kLinWeights) {
        decode([&](uint32_t s, bool act, const uint32_t(&e)[8]) {
          if (act) {
            const uint64_t at = (uint64_t)(r0 + 8u * s) * A.cols + 8ull * kv;
            __builtin_nontemporal_store(block_weights<WIDE>(e, gs[s], true),
                                        (__attribute__((address_space(1))) u32x4 *)((uint16_t *)A.out + at));
          }
        });
      } else {
        decode([&](uint32_t s, bool act, const uint32_t(&e)[8]) {
          if (act) {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              w[k] = ((uint32_t)entry_value<WIDE>(e[2 * k]) & 0xffffu) | ((uint32_t)entry_value<WIDE>(e[2 * k + 1]) << 16);
            const uint64_t at = (uint64_t)(r0 + 8u * s) * (8ull * A.vpr) + 8ull * kv;
            __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]},
                                        (__attribute__((address_space(1))) u32x4 *)((int16_t *)A.out + at));
          }
        });
      }
    }
    if constexpr (MODE != kLinGemm) {
      if (c + 1u < c_end) {
        lds_barrier();  // every wave is done with the chunk's words
        const uint32_t kb1 = kb0 + P.chunk, t1 = nb * P.kb_n + kb1, n1 = min(P.chunk, P.kb_n - kb1);
        copy_pieces(A, lds, first_piece(toff[t1]), end_piece(toff[t1 + n1]), A.words_off, lane, wave,
                    (uint32_t)kLinWaves);
      }
    } else {
      lds_barrier();  // the chunk's blocks are in their slots; its words are no longer read
      // the next chunk's words load into registers during this chunk's
      // products (a copy straight into LDS would make the products' LDS reads
      // wait for it) and go to LDS after them
      const bool more = c + 1u < c_end;
      uint32_t q0 = 0, q1 = 0;
      u32x4 cp[kStage];
      if (more) {
        const uint32_t kb1 = kb0 + P.chunk, t1 = nb * P.kb_n + kb1, n1 = min(P.chunk, P.kb_n - kb1);
        q0 = first_piece(toff[t1]);
        q1 = end_piece(toff[t1 + n1]);
        stage_pieces(A, q0, q1, lane, wave, (uint32_t)kLinWaves, cp);
      }
      // lane's fragments: A row m0 + 16 i + lane % 16, k 8 (lane / 16) ..;
      // B column (W row) 16 j + lane % 16 of the block, same k
      const uint32_t lr = lane & 15u, lk = lane >> 4;
      const bool rows = m0 < P.m;  // wave-uniform: waves whose rows all lie past M skip the products
      // B fragments of slot sl, both halves of its 64 columns of K; with few
      // rows per wave (registers to spare) the next slot's are read before
      // this slot's products, so that no product waits for an LDS read
      constexpr bool kAheadB = RB <= 2;
      auto read_b = [&](uint32_t sl, u32x4 (&b)[2][kCb]) {
#pragma unroll
        for (uint32_t kh = 0; kh < 2u; ++kh)
#pragma unroll
          for (int j = 0; j < kCb; ++j)
            b[kh][j] = *(lds_u128_rptr)(uintptr_t)(P.slots_off + sl * kSlotBytes +
                                                   (16u * (uint32_t)j + lr) * kSlotRowBytes + 16u * (4u * kh + lk));
      };
      u32x4 bq[2][2][kCb];
      if (kAheadB && rows) read_b(0u, bq[0]);
#pragma unroll
      for (uint32_t sl = 0; sl < kLinMaxChunk; ++sl) {
        if (rows && sl < nt) {
          if (sl + kRing - 1u < nt)
            load_x<RB>(P, m0, 64u * (kb0 + sl + kRing - 1u), lane, xa[(sl + kRing - 1u) % kRing]);
          if constexpr (kAheadB) {
            if (sl + 1u < nt) read_b(sl + 1u, bq[(sl + 1u) & 1u]);
          } else {
            read_b(sl, bq[sl & 1u]);
          }
          const u32x4(&b)[2][kCb] = bq[sl & 1u];
#pragma unroll
          for (uint32_t kh = 0; kh < 2u; ++kh)
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
              for (int j = 0; j < kCb; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[sl % kRing][i][kh]),
                                                                    __builtin_bit_cast(bf16x8, b[kh][j]), acc[i][j], 0,
                                                                    0, 0);
        }
      }
      if (more) store_pieces(A, q0, q1, A.words_off, lane, wave, (uint32_t)kLinWaves, cp);
    }
  }
  if constexpr (MODE == kLinGemm) {
    // lane holds D[4 (lane / 16) + r][lane % 16] of each 16 x 16 block
    // (split: this workgroup's share of the sum over K, to its partial slab)
    const uint32_t lr = lane & 15u, lk = lane >> 4;
#pragma unroll
    for (int j = 0; j < kCb; ++j) {
      const uint32_t col = 64u * nb + 16u * (uint32_t)j + lr;
      if (col >= P.n) continue;
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (uint32_t r = 0; r < 4u; ++r) {
          const uint32_t row = m0 + 16u * (uint32_t)i + 4u * lk + r;
          if (row >= P.m) continue;
          const uint64_t at = (uint64_t)row * P.n + col;
          if (P.split > 1u)
            P.part[(uint64_t)sp * P.m * P.n + at] = acc[i][j][r];
          else if (P.y_f32)
            reinterpret_cast<float *>(P.y)[at] = acc[i][j][r];
          else
            reinterpret_cast<uint16_t *>(P.y)[at] = (uint16_t)(pack2<EP_BF16>(acc[i][j][r], 0.0f) & 0xffffu);
        }
    }
  }
}

// Few rows of X (m <= 16 RB, RB <= 2): every wave works on its own.  A
// workgroup of 16 waves owns one block row of W (64 output columns) and a
// range of K-blocks; wave w decodes blocks w, w + 16, ... of the range, each
// from its own copy of the block's words, with nothing shared but the
// tables.  Every two decode steps give 16 consecutive rows of the block;
// the wave stages them in its own 16 x 144-byte LDS area, reads them back
// as B fragments (no other wave touches the area, and one wave's LDS
// accesses complete in order) and multiplies them by its A fragments of X
// right away.  After the last block the 16 waves' FP32 sums are added in a
// fixed tree order in LDS and wave 0 writes Y or the split's partial slab.
// Without slots shared by all waves, 16 waves fit beside the tables: the
// decode runs at the width of the standalone decoder.
constexpr int kLwWaves = 16;
constexpr uint32_t kStageBytes = 16 * kSlotRowBytes;
constexpr uint32_t kCbBytes = 4 * 1024;  // one wave's sums of a 16-row block of X: 4 x 16 x 16 FP32

// NW waves per workgroup: 16 for RB <= 2, 8 for RB = 4 (two waves per SIMD
// leave room for four row blocks' sums and fragments)
template <bool WIDE, int RB, int NW>
__global__ void __launch_bounds__(64 * NW) linear_waves_kernel(LinArgs P) {
  extern __shared__ __align__(16) uint8_t lds[];
  const Args &A = P.a;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t L = xcd_logical(blockIdx.x, P.grid);
  const uint32_t nb = L / P.split, sp = L - nb * P.split;
  const uint32_t kb_lo = sp * P.cps, kb_hi = min(kb_lo + P.cps, P.kb_n);
  typedef __attribute__((address_space(4))) const uint32_t *cptr_u32;
  const cptr_u32 toff = (cptr_u32)A.toff;
  if (wave < (uint32_t)kContexts) {
    uint32_t fpre[4];
    first_frequencies(A, wave, lane, fpre);
    build_tables<WIDE>(A, lds, wave, lane, (uint32_t)kContexts, fpre);
  }
  const uint32_t r0 = 64u * nb + (lane >> 3), vcol = lane & 7u, lr = lane & 15u, lk = lane >> 4;
  float gs[8];
#pragma unroll
  for (uint32_t s = 0; s < 8; ++s) gs[s] = A.scales[min(r0 + 8u * s, A.rows - 1u)];
  uint32_t present_rows = 0;
#pragma unroll
  for (uint32_t s = 0; s < 8; ++s) present_rows |= (r0 + 8u * s < A.rows ? 1u : 0u) << s;
  constexpr int kCb = 4;
  f32x4 acc[RB][kCb];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < kCb; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t buf = A.words_off + wave * A.wbuf;            // this wave's words
  const uint32_t stg = P.slots_off + wave * kStageBytes;       // this wave's 16 staged rows
  const uint32_t put = stg + (lane >> 3) * kSlotRowBytes + 16u * vcol;  // + 8 rows for odd steps
  const uint32_t get = stg + lr * kSlotRowBytes + 16u * lk;             // + 64 bytes for the upper half of K
  lds_barrier();  // tables built
  for (uint32_t kb = kb_lo + wave; kb < kb_hi; kb += (uint32_t)NW) {
    const uint32_t t = nb * P.kb_n + kb;
    const uint32_t tb = toff[t], te = toff[t + 1u];
    const uint32_t c0 = first_piece(tb);
    copy_pieces(A, lds, c0, end_piece(te), buf, lane, 0u, 1u);
    u32x4 xa[RB][2];
    load_x<RB>(P, 0u, 64u * kb, lane, xa);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's words and X fragments have landed
    const uint32_t wt = buf + 2u * tb - 16u * c0;
    const uint32_t present = 8u * kb + vcol < A.vpr ? present_rows : 0u;
    auto sink = [&](uint32_t s, bool act, const uint32_t(&e)[8]) {
      *(lds_u128_wptr)(uintptr_t)(put + (s & 1u) * 8u * kSlotRowBytes) = block_weights<WIDE>(e, gs[s], act);
      if (s & 1u) {  // block rows 16 (s / 2) .. + 15 are staged: one product per half of K
#pragma unroll
        for (uint32_t h = 0; h < 2u; ++h) {
          const u32x4 b = *(lds_u128_rptr)(uintptr_t)(get + 64u * h);
#pragma unroll
          for (int i = 0; i < RB; ++i)
            acc[i][s >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[i][h]),
                                                                     __builtin_bit_cast(bf16x8, b), acc[i][s >> 1], 0,
                                                                     0, 0);
        }
      }
    };
    if (__ballot(present != 0xffu) == 0)
      decode_block<WIDE, true>(wt, wt + 2u * (te - tb), lane, present, sink);
    else
      decode_block<WIDE, false>(wt, wt + 2u * (te - tb), lane, present, sink);
  }
  // the waves' sums, added in a fixed tree order: at distance d, wave w with
  // w mod 2d = d stores its sums and wave w - d adds them
  const uint32_t red = A.words_off;  // the word buffers are no longer read after the next barrier
#pragma unroll
  for (uint32_t d = 1; d < (uint32_t)NW; d *= 2u) {
    lds_barrier();
    if (wave % (2u * d) == d) {
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < kCb; ++j)
          *(__attribute__((address_space(3))) f32x4 *)(uintptr_t)(red + (wave / (2u * d)) * (uint32_t)RB * kCbBytes +
                                                                  (uint32_t)(i * kCb + j) * 1024u + 16u * lane) =
              acc[i][j];
    }
    lds_barrier();
    if (wave % (2u * d) == 0u && wave + d < (uint32_t)NW) {
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < kCb; ++j)
          acc[i][j] += *(__attribute__((address_space(3))) const f32x4 *)(uintptr_t)(
              red + (wave / (2u * d)) * (uint32_t)RB * kCbBytes + (uint32_t)(i * kCb + j) * 1024u + 16u * lane);
    }
  }
  if (wave != 0u) return;
#pragma unroll
  for (int j = 0; j < kCb; ++j) {
    const uint32_t col = 64u * nb + 16u * (uint32_t)j + lr;
    if (col >= P.n) continue;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (uint32_t r = 0; r < 4u; ++r) {
        const uint32_t row = 16u * (uint32_t)i + 4u * lk + r;
        if (row >= P.m) continue;
        const uint64_t at = (uint64_t)row * P.n + col;
        if (P.split > 1u)
          P.part[(uint64_t)sp * P.m * P.n + at] = acc[i][j][r];
        else if (P.y_f32)
          reinterpret_cast<float *>(P.y)[at] = acc[i][j][r];
        else
          reinterpret_cast<uint16_t *>(P.y)[at] = (uint16_t)(pack2<EP_BF16>(acc[i][j][r], 0.0f) & 0xffffu);
      }
  }
}

// Y = the sum of the split partial slabs, in slab order (so the result does
// not depend on which workgroup finished first), as FP32 or BF16.
__global__ void __launch_bounds__(256) linear_reduce_kernel(const float *part, uint32_t split, uint64_t mn, void *y,
                                                            uint32_t y_f32) {
  const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (i >= mn) return;
  float s = part[i];
  for (uint32_t k = 1; k < split; ++k) s += part[(uint64_t)k * mn + i];
  if (y_f32)
    reinterpret_cast<float *>(y)[i] = s;
  else
    reinterpret_cast<uint16_t *>(y)[i] = (uint16_t)(pack2<EP_BF16>(s, 0.0f) & 0xffffu);
}

typedef const void *KernelFn;  // a kernel's address: decode_waves_kernel takes Args, decode_kernel RoundArgs

template <int OUT, bool WIDE, bool PADDED, int NS, int V>
KernelFn pick1(bool multi, bool prio) {
  if (!multi) return (KernelFn)decode_kernel<OUT, WIDE, PADDED, NS, V>;
  return prio ? (KernelFn)decode_waves_kernel<OUT, WIDE, PADDED, NS, V, true>
              : (KernelFn)decode_waves_kernel<OUT, WIDE, PADDED, NS, V, false>;
}

template <int OUT, bool WIDE, bool PADDED>
KernelFn pick4(bool multi, bool prio, int ns, int tv) {
  if (ns == kStatesLow) {
    if (tv == kTileVecsSmall) return pick1<OUT, WIDE, PADDED, 16, 32>(multi, prio);
    return pick1<OUT, WIDE, PADDED, 16, 64>(multi, prio);
  }
  if (tv == kTileVecsSmall) return pick1<OUT, WIDE, PADDED, 64, 8>(multi, prio);
  return pick1<OUT, WIDE, PADDED, 64, 16>(multi, prio);
}

template <int OUT>
KernelFn pick(bool wide, bool padded, bool multi, bool prio, int ns, int tv) {
  if (wide) return padded ? pick4<OUT, true, true>(multi, prio, ns, tv) : pick4<OUT, true, false>(multi, prio, ns, tv);
  return padded ? pick4<OUT, false, true>(multi, prio, ns, tv) : pick4<OUT, false, false>(multi, prio, ns, tv);
}

// multi: the multi-tile kernel; prio: its variant with wave priorities (every
// wave of every workgroup has the same number of units)
KernelFn pick_kernel(int out, bool wide, bool padded, bool multi, bool prio, int ns, int tv) {
  switch (out) {
    case EP_BF16: return pick<EP_BF16>(wide, padded, multi, prio, ns, tv);
    case EP_FP16: return pick<EP_FP16>(wide, padded, multi, prio, ns, tv);
    case EP_FP8_E4M3FN: return pick<EP_FP8_E4M3FN>(wide, padded, multi, prio, ns, tv);
    case EP_INT8: return pick<EP_INT8>(wide, padded, multi, prio, ns, tv);
    default: return pick<kOutSym>(wide, false, multi, prio, ns, tv);
  }
}

// compute units of the current device (one workgroup each in the multi-tile
// kernel)
int64_t num_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

int32_t host_symbol_value(int c, int32_t s) {
  if (c == 0) return s;
  if (c <= 2) return 2 * s + (c - 1);
  const int bp = c - 3;
  return 4 * s + 2 * (bp & 1) + (bp >> 1);
}

// magic number for n / d with n < 2^31: umulhi(n, m) >> (s - 1), s = ceil(log2 d), d >= 2
void row_divider(uint32_t d, uint32_t &m, uint32_t &shift) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  m = (uint32_t)(((uint64_t(1) << (31 + s)) + d - 1) / d);
  shift = s - 1;
}

// Everything a decode launch needs that depends on the stream alone: the
// kernel, its geometry and its arguments (all but the output pointer).
struct Plan {
  bool raw = false;        // raw container: a device-to-device copy of the payload
  size_t raw_bytes = 0;
  const void *dev_blob = nullptr;
  KernelFn fn = nullptr;
  uint32_t grid = 0, block = 0, lds_bytes = 0;
  bool multi = false;      // multi-tile kernel: its argument is R.a alone
  RoundArgs R{};
  bool blocks = false;     // blocks layout: linear_kernel in a weights or symbols mode, argument L
  LinArgs L{};
};

// Tile offsets: monotone, inside the word section, room for the pair counts
// and length codes.  Returns 0 or EP_ERR_FORMAT.
int check_tile_offsets(const uint8_t *hb, const StreamView &s) {
  const uint8_t *toff = hb + s.off_tile_offsets;
  auto first_word = [&](int64_t t) { return rd<uint32_t>(toff + 4 * t); };
  for (int64_t t = 0; t < s.tiles; ++t) {
    const uint32_t b = first_word(t), e = first_word(t + 1);
    if (e < b || e > s.n_words || e - b < (uint32_t)s.states / 2u) {
      set_error("corrupt tile offsets");
      return EP_ERR_FORMAT;
    }
  }
  if (first_word(s.tiles) != s.n_words) {
    set_error("corrupt tile offsets");
    return EP_ERR_FORMAT;
  }
  return EP_OK;
}

// Tables: frequencies sum to 2^10, used values inside the entry field; fills
// the table fields of A.  wide: some used value lies outside [-128, 127].
// Returns 0 or EP_ERR_FORMAT.
int check_tables(const uint8_t *hb, const StreamView &s, Args &A, bool &wide, uint32_t &nz_total) {
  wide = false;
  nz_total = 0;
  for (int c = 0; c < kContexts; ++c) {
    A.smin[c] = s.smin[c];
    // symbol counts and frequency indexes share a word per context: 16 bits
    // each, far above what the 12-bit value field allows an encoder
    if (s.nsym[c] > (uint32_t)(kValueMax - kValueMin + 1) || s.freq_index[c] + s.nsym[c] > 0xffffu) {
      set_error("frequency table larger than the decoder's 16-bit indexes");
      return EP_ERR_FORMAT;
    }
    A.ctx_freq[c] = (uint32_t)s.freq_index[c] | (uint32_t)s.nsym[c] << 16;
    A.nzbase[c] = nz_total;
    uint32_t sum = 0;
    for (uint32_t i = 0; i < s.nsym[c]; ++i) {
      const uint16_t f = rd<uint16_t>(hb + s.off_freq + 2 * (s.freq_index[c] + i));
      if (!f) continue;
      sum += f;
      ++nz_total;
      const int32_t v = host_symbol_value(c, s.smin[c] + (int32_t)i);
      if (v < kValueMin || v > kValueMax || f >= kProbTotal) {
        set_error("table entry outside the decoder's range");
        return EP_ERR_FORMAT;
      }
      if (v < -128 || v > 127) wide = true;
    }
    if (s.nsym[c] && sum != kProbTotal) {
      set_error("frequencies do not sum to 2^10");
      return EP_ERR_FORMAT;
    }
  }
  return EP_OK;
}

// host-side checks and launch geometry; returns 0 or an ep_status
int prepare(const uint8_t *hb, const StreamView &s, const void *dev_blob, int out, Plan &P) {
  if (!dev_blob) {
    set_error("null device pointer");
    return EP_ERR_ARG;
  }
  if ((uintptr_t)dev_blob & 15) {
    set_error("device buffers must be 16-byte aligned");
    return EP_ERR_ARG;
  }
  if (const int rc = check_tile_offsets(hb, s); rc != EP_OK) return rc;
  const uint8_t *toff = hb + s.off_tile_offsets;
  auto first_word = [&](int64_t t) { return rd<uint32_t>(toff + 4 * t); };
  Args A{};
  bool wide = false;
  uint32_t nz_total = 0;
  if (const int rc = check_tables(hb, s, A, wide, nz_total); rc != EP_OK) return rc;
  // LDS layout: tables | records | bitmap | row descriptors | words | pad.
  // A wave decodes a unit of 64 / states consecutive tiles; the words of a
  // workgroup's consecutive units are one range, copied in whole kilobytes
  // from a 16-byte boundary.
  const int64_t tpw = 64 / s.states;
  const int64_t units = (s.tiles + tpw - 1) / tpw;
  uint32_t off = kTableBytes;
  A.rec_off = off;
  off += 8 * nz_total;
  A.mark_off = off;
  off = (uint32_t)align16(off + 4 * kContexts * kMarkWords);
  A.desc_off = off;  // 256 bytes of row descriptors per table-building wave
  off += 256 * kContexts;
  A.words_off = off;
  // bytes the copy of tiles [t0, t1) takes
  auto copy_bytes = [&](int64_t t0, int64_t t1) {
    const uint64_t a0 = (s.off_words + 2ull * first_word(t0)) & ~15ull;
    const uint64_t a1 = (s.off_words + 2ull * first_word(t1) + 15ull) & ~15ull;
    return (a1 - a0 + 1023ull) & ~1023ull;
  };
  // the largest copy of k consecutive units
  auto span_for = [&](int64_t k) {
    uint64_t span = 0;
    for (int64_t u0 = 0; u0 < units; u0 += k)
      span = std::max<uint64_t>(span, copy_bytes(u0 * tpw, std::min<int64_t>((u0 + k) * tpw, s.tiles)));
    return span;
  };
  // Waves per workgroup: as many as the LDS allows, up to 16 (four per
  // SIMD), but no more than spreads the units over every CU: a stream of few
  // units (low rates: few states, long chains) decodes faster with one wave
  // per SIMD on every CU than with four per SIMD on a quarter of them.
  uint32_t waves = 0;
  uint64_t span = 0;
  const int64_t per_cu = (units + num_cus() - 1) / num_cus();
  for (int64_t k = std::min<int64_t>({(int64_t)kMaxWaves, units, std::max<int64_t>(per_cu, 4)}); k >= 1; --k) {
    span = span_for(k);
    if (off + span + kLdsPad <= kLdsLimit) {
      waves = (uint32_t)k;
      break;
    }
  }
  if (!waves) {
    set_error("tile too large for the decoder's LDS budget");
    return EP_ERR_FORMAT;
  }
  uint32_t lds_bytes = off + (uint32_t)span + kLdsPad;
  uint32_t grid = (uint32_t)((units + waves - 1) / waves);
  // More workgroups than compute units: the multi-tile kernel instead, with
  // one workgroup per CU that builds the tables once.
  const bool multi = (int64_t)grid > std::min<int64_t>(num_cus(), kMaxRoundWgs);
  if (multi) {
    // One workgroup per CU, each with a run of consecutive units (counts that
    // differ by at most one); its k waves take the run's units in turn.  k is
    // as many waves as the run and the LDS allow (at most 16, four per SIMD).
    // Every wave has a buffer for one unit's words.
    const uint64_t wbuf = span_for(1);
    const uint64_t room = kLdsLimit - std::min<uint64_t>(kLdsLimit, (uint64_t)A.words_off + kLdsPad);
    const int64_t kmax = std::min<int64_t>(kMaxWaves, (int64_t)(room / wbuf));
    if (kmax < 1) {
      set_error("tile too large for the decoder's LDS budget");
      return EP_ERR_FORMAT;
    }
    const int64_t g = std::min<int64_t>(units, num_cus());
    const int64_t q = units / g, rem = units % g, qmax = q + (rem ? 1 : 0);
    waves = (uint32_t)std::min<int64_t>(kmax, qmax);
    grid = (uint32_t)g;
    A.wg_q = (uint32_t)q;
    A.wg_rem = (uint32_t)rem;
    A.wbuf = (uint32_t)wbuf;
    lds_bytes = A.words_off + waves * (uint32_t)wbuf + kLdsPad;
  }
  const uint8_t *db = reinterpret_cast<const uint8_t *>(dev_blob);
  A.freq = reinterpret_cast<const uint16_t *>(db + s.off_freq);
  A.toff = reinterpret_cast<const uint32_t *>(db + s.off_tile_offsets);
  A.words = db + s.off_words;
  A.scales = reinterpret_cast<const float *>(db + s.off_scales);
  A.out = nullptr;
  A.cols = (uint64_t)s.cols;
  A.rows = (uint32_t)s.rows;
  A.vpr = (uint32_t)(s.cols8 / 8);
  if (A.vpr > 1) row_divider(A.vpr, A.row_magic, A.row_shift);
  A.n_vec = (uint32_t)s.n_vec;
  A.n_tiles = (uint32_t)s.tiles;
  A.n_units = (uint32_t)units;
  const bool padded = out != kOutSym && (s.cols % 8) != 0;
  const bool prio = multi && A.wg_rem == 0 && A.wg_q % waves == 0;
  A.waves = waves;
  P.raw = false;
  P.dev_blob = dev_blob;
  P.fn = pick_kernel(out, wide, padded, multi, prio, s.states, s.tile_vecs);
  P.grid = grid;
  P.block = 64 * waves;
  P.lds_bytes = lds_bytes;
  P.multi = multi;
  P.R.a = A;
  if (!multi)
    for (uint32_t b = 0; b <= grid; ++b)
      P.R.wg_word[b] = first_word(std::min<int64_t>((int64_t)b * waves * tpw, s.tiles));
  return EP_OK;
}

// the plan of a raw container: its payload is copied as it is
int prepare_raw(const StreamView &s, const void *dev_blob, Plan &P) {
  if (!dev_blob) {
    set_error("null device pointer");
    return EP_ERR_ARG;
  }
  P.raw = true;
  P.dev_blob = dev_blob;
  P.raw_bytes = (size_t)s.rows * (size_t)s.cols * elem_bytes(s.dtype);
  return EP_OK;
}

template <int MODE, bool WIDE>
KernelFn pick_linear_rb(int rb) {
  if (rb == 1) return (KernelFn)linear_kernel<MODE, WIDE, 1>;
  if (rb == 2) return (KernelFn)linear_kernel<MODE, WIDE, 2>;
  return (KernelFn)linear_kernel<MODE, WIDE, 4>;
}
KernelFn pick_linear(int mode, bool wide, int rb) {
  if (mode == kLinGemm) return wide ? pick_linear_rb<kLinGemm, true>(rb) : pick_linear_rb<kLinGemm, false>(rb);
  if (mode == kLinWeights)
    return wide ? (KernelFn)linear_kernel<kLinWeights, true, 1> : (KernelFn)linear_kernel<kLinWeights, false, 1>;
  return wide ? (KernelFn)linear_kernel<kLinSymbols, true, 1> : (KernelFn)linear_kernel<kLinSymbols, false, 1>;
}

// Plans linear_kernel on a blocks-layout stream: the tables and tile offsets
// checked, the LDS layout (tables | table-build scratch, later the chunk's
// words | pad | block slots), the chunk size (up to 8 tiles, as many as the
// LDS holds for the stream's largest chunk) and the grid.  GEMM: one
// workgroup per (row block of X, block row of W), every chunk; weights and
// symbols: one workgroup per chunk.  rb: 16-row blocks of X per wave.
int prepare_linear(const uint8_t *hb, const StreamView &s, const void *dev_blob, int mode, int64_t m, int rb,
                   LinArgs &L, KernelFn &fn, uint32_t &grid, uint32_t &lds_bytes) {
  if (!dev_blob) {
    set_error("null device pointer");
    return EP_ERR_ARG;
  }
  if ((uintptr_t)dev_blob & 15) {
    set_error("device buffers must be 16-byte aligned");
    return EP_ERR_ARG;
  }
  if (const int rc = check_tile_offsets(hb, s); rc != EP_OK) return rc;
  Args A{};
  bool wide = false;
  uint32_t nz_total = 0;
  if (const int rc = check_tables(hb, s, A, wide, nz_total); rc != EP_OK) return rc;
  const uint8_t *toff = hb + s.off_tile_offsets;
  auto first_word = [&](int64_t t) { return rd<uint32_t>(toff + 4 * t); };
  uint32_t off = kTableBytes;
  A.rec_off = off;
  off += 8 * nz_total;
  A.mark_off = off;
  off = (uint32_t)align16(off + 4 * kContexts * kMarkWords);
  A.desc_off = off;
  off += 256 * kContexts;
  const uint32_t build_end = off;
  A.words_off = (uint32_t)align16(build_end);  // the first chunk's words arrive during the build
  const int64_t vpr = s.cols8 / 8, kb_n = (vpr + kBlockVecs - 1) / kBlockVecs, nb_n = (s.rows + kBlockRows - 1) / kBlockRows;
  auto copy_bytes = [&](int64_t t0, int64_t t1) {
    const uint64_t a0 = (s.off_words + 2ull * first_word(t0)) & ~15ull;
    const uint64_t a1 = (s.off_words + 2ull * first_word(t1) + 15ull) & ~15ull;
    return (a1 - a0 + 1023ull) & ~1023ull;
  };
  uint32_t chunk = 0;
  uint64_t wbuf = 0, need = 0, slots_off = 0;
  for (int64_t ch = kLinMaxChunk; ch >= 1; --ch) {
    wbuf = 0;
    for (int64_t nb = 0; nb < nb_n; ++nb)
      for (int64_t k0 = 0; k0 < kb_n; k0 += ch)
        wbuf = std::max<uint64_t>(wbuf, copy_bytes(nb * kb_n + k0, nb * kb_n + std::min<int64_t>(k0 + ch, kb_n)));
    slots_off = align16(A.words_off + wbuf + kLdsPad);
    need = mode == kLinGemm ? slots_off + (uint64_t)ch * kSlotBytes : slots_off;
    if (need <= kLdsLimit) {
      chunk = (uint32_t)ch;
      break;
    }
  }
  if (!chunk) {
    set_error("tile too large for the fused decoder's LDS budget");
    return EP_ERR_FORMAT;
  }
  const uint8_t *db = reinterpret_cast<const uint8_t *>(dev_blob);
  A.freq = reinterpret_cast<const uint16_t *>(db + s.off_freq);
  A.toff = reinterpret_cast<const uint32_t *>(db + s.off_tile_offsets);
  A.words = db + s.off_words;
  A.scales = reinterpret_cast<const float *>(db + s.off_scales);
  A.cols = (uint64_t)s.cols;
  A.rows = (uint32_t)s.rows;
  A.vpr = (uint32_t)vpr;
  A.n_tiles = (uint32_t)s.tiles;
  A.waves = kLinWaves;
  L = LinArgs{};
  L.a = A;
  L.n = (uint32_t)s.rows;
  L.k = (uint32_t)s.cols;
  L.kb_n = (uint32_t)kb_n;
  L.nb_n = (uint32_t)nb_n;
  L.chunk = chunk;
  L.chunks = (uint32_t)((kb_n + chunk - 1) / chunk);
  L.slots_off = (uint32_t)slots_off;
  const uint64_t rows_per_wg = (uint64_t)kLinWaves * 16u * (uint64_t)rb;
  L.m = (uint32_t)m;
  L.mb_n = mode == kLinGemm ? (uint32_t)(((uint64_t)m + rows_per_wg - 1) / rows_per_wg) : 1u;
  // GEMM with fewer output blocks than compute units: split the sum over K
  // across workgroups (partial slabs summed by linear_reduce_kernel) so that
  // every CU decodes
  L.split = 1;
  L.cps = L.chunks;
  if (mode == kLinGemm) {
    const uint64_t base = (uint64_t)L.mb_n * (uint64_t)nb_n;
    uint64_t sp = std::max<uint64_t>(1, std::min<uint64_t>(L.chunks, ((uint64_t)num_cus() + base / 2) / base));
    L.cps = (uint32_t)((L.chunks + sp - 1) / sp);
    L.split = (L.chunks + L.cps - 1) / L.cps;
  }
  const uint64_t g = mode == kLinGemm ? (uint64_t)L.mb_n * (uint64_t)nb_n * L.split : (uint64_t)nb_n * L.chunks;
  if (g == 0 || g > 0x7fffffffull) {
    set_error("grid too large");
    return EP_ERR_SHAPE;
  }
  L.grid = (uint32_t)g;
  grid = L.grid;
  lds_bytes = (uint32_t)need;
  fn = pick_linear(mode, wide, rb);
  // Few rows (m <= 32): the wave-independent kernel, if each wave's word
  // buffer, its staging rows and the final sums fit the LDS
  if (mode == kLinGemm && m <= 64) {
    uint64_t wb1 = 0;
    for (int64_t t = 0; t < s.tiles; ++t) wb1 = std::max<uint64_t>(wb1, copy_bytes(t, t + 1));
    const int rbw = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
    const int64_t nw = rbw == 4 ? 8 : kLwWaves;
    const uint64_t stg = align16(A.words_off + (uint64_t)nw * wb1 + kLdsPad);
    const uint64_t need_w = std::max<uint64_t>(stg + (uint64_t)nw * kStageBytes,
                                               (uint64_t)A.words_off + (uint64_t)(nw / 2) * rbw * kCbBytes);
    if (need_w <= kLdsLimit) {
      L.a.wbuf = (uint32_t)wb1;
      L.slots_off = (uint32_t)stg;
      // splits of K: about one workgroup per CU, at least one block per wave
      const uint64_t sp = std::max<int64_t>(
          1, std::min<int64_t>(num_cus() / std::max<int64_t>(nb_n, 1), (kb_n + nw - 1) / nw));
      L.cps = (uint32_t)((kb_n + (int64_t)sp - 1) / (int64_t)sp);
      L.split = (uint32_t)((kb_n + L.cps - 1) / L.cps);
      L.mb_n = 1;
      L.grid = (uint32_t)((uint64_t)nb_n * L.split);
      grid = L.grid;
      lds_bytes = (uint32_t)need_w;
      L.waves_kernel = (uint32_t)nw;
      if (rbw == 1)
        fn = wide ? (KernelFn)linear_waves_kernel<true, 1, kLwWaves> : (KernelFn)linear_waves_kernel<false, 1, kLwWaves>;
      else if (rbw == 2)
        fn = wide ? (KernelFn)linear_waves_kernel<true, 2, kLwWaves> : (KernelFn)linear_waves_kernel<false, 2, kLwWaves>;
      else
        fn = wide ? (KernelFn)linear_waves_kernel<true, 4, 8> : (KernelFn)linear_waves_kernel<false, 4, 8>;
    }
  }
  return EP_OK;
}

// launches a planned linear_kernel
int launch_linear(KernelFn fn, const LinArgs &L, uint32_t grid, uint32_t lds_bytes, hipStream_t stream) {
  static std::mutex mu;
  static std::vector<KernelFn> configured;
  {
    std::lock_guard<std::mutex> lk(mu);
    bool done = false;
    for (KernelFn k : configured) done |= k == fn;
    if (!done) {
      if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit) != hipSuccess) {
        set_error("hipFuncSetAttribute failed");
        return EP_ERR_DEVICE;
      }
      configured.push_back(fn);
    }
  }
  LinArgs a = L;
  void *args[1] = {&a};
  hipError_t err =
      hipLaunchKernel(fn, dim3(grid), dim3(64 * (L.waves_kernel ? L.waves_kernel : (uint32_t)kLinWaves)), args,
                      lds_bytes, stream);
  if (err == hipSuccess) err = hipGetLastError();
  if (err == hipSuccess && L.split > 1u) {
    const uint64_t mn = (uint64_t)L.m * L.n;
    const float *part = L.part;
    uint32_t split = L.split, y_f32 = L.y_f32;
    void *y = L.y;
    void *rargs[5] = {&part, &split, (void *)&mn, &y, &y_f32};
    err = hipLaunchKernel((const void *)linear_reduce_kernel, dim3((uint32_t)((mn + 255) / 256)), dim3(256), rargs, 0,
                          stream);
    if (err == hipSuccess) err = hipGetLastError();
  }
  if (err != hipSuccess) {
    set_error(std::string("kernel launch failed: ") + hipGetErrorString(err));
    return EP_ERR_DEVICE;
  }
  return EP_OK;
}

// enqueues a planned decode into dev_out on stream
int enqueue(const Plan &P, void *dev_out, hipStream_t stream) {
  if (!dev_out) {
    set_error("null device pointer");
    return EP_ERR_ARG;
  }
  if (P.raw) {
    if (hipMemcpyAsync(dev_out, reinterpret_cast<const uint8_t *>(P.dev_blob) + kHeaderBytes, P.raw_bytes,
                       hipMemcpyDeviceToDevice, stream) != hipSuccess) {
      set_error("hipMemcpyAsync failed");
      return EP_ERR_DEVICE;
    }
    return EP_OK;
  }
  if ((uintptr_t)dev_out & 15) {
    set_error("device buffers must be 16-byte aligned");
    return EP_ERR_ARG;
  }
  if (P.blocks) {
    LinArgs L = P.L;
    L.a.out = dev_out;
    return launch_linear(P.fn, L, P.grid, P.lds_bytes, stream);
  }
  static std::mutex mu;
  static std::vector<KernelFn> configured;
  {
    std::lock_guard<std::mutex> lk(mu);
    bool done = false;
    for (KernelFn k : configured) done |= k == P.fn;
    if (!done) {
      if (hipFuncSetAttribute(P.fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit) != hipSuccess) {
        set_error("hipFuncSetAttribute failed");
        return EP_ERR_DEVICE;
      }
      configured.push_back(P.fn);
    }
  }
  void *args[1];
  RoundArgs R;
  Args A;
  if (P.multi) {
    A = P.R.a;
    A.out = dev_out;
    args[0] = &A;
  } else {
    R = P.R;
    R.a.out = dev_out;
    args[0] = &R;
  }
  hipError_t err = hipLaunchKernel(P.fn, dim3(P.grid), dim3(P.block), args, P.lds_bytes, stream);
  if (err == hipSuccess) err = hipGetLastError();
  if (err != hipSuccess) {
    set_error(std::string("kernel launch failed: ") + hipGetErrorString(err));
    return EP_ERR_DEVICE;
  }
  return EP_OK;
}

// parses a stream and plans its decode into out (an output kind)
int plan_stream(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, int out_dtype, bool symbols,
                Plan &P) {
  StreamView s;
  std::string e = parse_stream(host_blob, nbytes, s);
  if (!e.empty()) {
    set_error(e);
    return EP_ERR_FORMAT;
  }
  if (symbols) {
    if (s.method != kLattice) {
      set_error("raw streams hold no lattice symbols");
      return EP_ERR_ARG;
    }
    if (s.layout == kLayoutBlocks) {
      P.blocks = true;
      return prepare_linear(host_blob, s, dev_blob, kLinSymbols, 0, 1, P.L, P.fn, P.grid, P.lds_bytes);
    }
    return prepare(host_blob, s, dev_blob, kOutSym, P);
  }
  if (out_dtype != -1 && out_dtype != s.dtype) {
    set_error("out_dtype must be -1 or the container dtype");
    return EP_ERR_ARG;
  }
  if (s.method == kRaw) return prepare_raw(s, dev_blob, P);
  if (s.layout == kLayoutBlocks) {
    P.blocks = true;
    return prepare_linear(host_blob, s, dev_blob, kLinWeights, 0, 1, P.L, P.fn, P.grid, P.lds_bytes);
  }
  return prepare(host_blob, s, dev_blob, s.dtype, P);
}

}  // namespace
}  // namespace ep

// a decode plan handed to callers
struct ep_plan {
  ep::Plan p;
};

extern "C" {

int ep_decompress(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, void *dev_out, int out_dtype,
                  void *hip_stream) {
  ep::set_error("");
  ep::Plan P;
  const int rc = ep::plan_stream(host_blob, nbytes, dev_blob, out_dtype, false, P);
  if (rc != EP_OK) return rc;
  return ep::enqueue(P, dev_out, reinterpret_cast<hipStream_t>(hip_stream));
}

int ep_decode_symbols(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, int16_t *dev_sym,
                      void *hip_stream) {
  ep::set_error("");
  ep::Plan P;
  const int rc = ep::plan_stream(host_blob, nbytes, dev_blob, -1, true, P);
  if (rc != EP_OK) return rc;
  return ep::enqueue(P, dev_sym, reinterpret_cast<hipStream_t>(hip_stream));
}

int ep_plan_create(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, int out_dtype, ep_plan **plan_out) {
  ep::set_error("");
  if (!plan_out) {
    ep::set_error("null plan_out");
    return EP_ERR_ARG;
  }
  *plan_out = nullptr;
  ep_plan *h = new (std::nothrow) ep_plan;
  if (!h) {
    ep::set_error("out of host memory");
    return EP_ERR_NOMEM;
  }
  const int rc = ep::plan_stream(host_blob, nbytes, dev_blob, out_dtype, false, h->p);
  if (rc != EP_OK) {
    delete h;
    return rc;
  }
  *plan_out = h;
  return EP_OK;
}

int ep_plan_decompress(const ep_plan *plan, void *dev_out, void *hip_stream) {
  ep::set_error("");
  if (!plan) {
    ep::set_error("null plan");
    return EP_ERR_ARG;
  }
  return ep::enqueue(plan->p, dev_out, reinterpret_cast<hipStream_t>(hip_stream));
}

void ep_plan_free(ep_plan *plan) { delete plan; }

// the fused linear's plan for m > 0 rows of X: 0 or an ep_status
static int linear_plan(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, int64_t m, ep::LinArgs &L,
                       ep::KernelFn &fn, uint32_t &grid, uint32_t &lds) {
  ep::StreamView s;
  std::string e = ep::parse_stream(host_blob, nbytes, s);
  if (!e.empty()) {
    ep::set_error(e);
    return EP_ERR_FORMAT;
  }
  if (s.method != ep::kLattice || s.layout != ep::kLayoutBlocks) {
    ep::set_error("ep_linear takes lattice streams in the blocks layout (EP_LAYOUT_BLOCKS)");
    return EP_ERR_ARG;
  }
  if (m < 0 || m >= (int64_t(1) << 31) || (uint64_t)m * (uint64_t)s.rows >= (uint64_t(1) << 62)) {
    ep::set_error("m must lie in [0, 2^31)");
    return EP_ERR_SHAPE;
  }
  if (m == 0) return EP_OK;
  // 16-row blocks per wave: few rows give one, so that waves past M skip
  // the products (each product wave reads the chunk's every block from LDS)
  const int rb = m > 512 ? 4 : (m > 64 ? 2 : 1);
  return ep::prepare_linear(host_blob, s, dev_blob, ep::kLinGemm, m, rb, L, fn, grid, lds);
}

int64_t ep_linear_workspace_bytes(const uint8_t *host_blob, size_t nbytes, int64_t m) {
  ep::set_error("");
  ep::LinArgs L;
  ep::KernelFn fn = nullptr;
  uint32_t grid = 0, lds = 0;
  // a stand-in device address: the plan only records it
  const int rc = linear_plan(host_blob, nbytes, reinterpret_cast<const void *>(uintptr_t(256)), m, L, fn, grid, lds);
  if (rc != EP_OK) return rc;
  return (m > 0 && L.split > 1u) ? (int64_t)L.split * m * (int64_t)L.n * 4 : 0;
}

// a planned fused linear
struct ep_linear_plan {
  ep::LinArgs L{};
  ep::KernelFn fn = nullptr;
  uint32_t grid = 0, lds = 0;
  int64_t m = 0;
};

// enqueues a planned fused linear (m > 0) on X, Y and the workspace
static int linear_run(const ep_linear_plan &P, const void *dev_x, void *dev_y, int y_dtype, void *dev_workspace,
                      size_t workspace_bytes, void *hip_stream) {
  if (y_dtype != EP_BF16 && y_dtype != EP_F32) {
    ep::set_error("y_dtype must be EP_BF16 or EP_F32");
    return EP_ERR_ARG;
  }
  if (P.m == 0) return EP_OK;
  if (!dev_x || !dev_y) {
    ep::set_error("null device pointer");
    return EP_ERR_ARG;
  }
  if (((uintptr_t)dev_x & 15) || ((uintptr_t)dev_y & 3) || ((uintptr_t)dev_workspace & 15)) {
    ep::set_error("dev_x and dev_workspace must be 16-byte aligned, dev_y 4-byte aligned");
    return EP_ERR_ARG;
  }
  ep::LinArgs L = P.L;
  uint32_t grid = P.grid;
  if (L.split > 1u) {
    const uint64_t need = (uint64_t)L.split * (uint64_t)P.m * L.n * 4u;
    if (!dev_workspace || workspace_bytes < need) {
      // no room for the partial sums: one workgroup per output block instead
      L.split = 1;
      L.cps = L.waves_kernel ? L.kb_n : L.chunks;
      grid = L.grid = L.mb_n * L.nb_n;
    } else {
      L.part = reinterpret_cast<float *>(dev_workspace);
    }
  }
  L.x = reinterpret_cast<const uint16_t *>(dev_x);
  L.y = dev_y;
  L.y_f32 = y_dtype == EP_F32 ? 1u : 0u;
  return ep::launch_linear(P.fn, L, grid, P.lds, reinterpret_cast<hipStream_t>(hip_stream));
}

int ep_linear(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, const void *dev_x, int64_t m,
              void *dev_y, int y_dtype, void *dev_workspace, size_t workspace_bytes, void *hip_stream) {
  ep::set_error("");
  if (y_dtype != EP_BF16 && y_dtype != EP_F32) {
    ep::set_error("y_dtype must be EP_BF16 or EP_F32");
    return EP_ERR_ARG;
  }
  if (m > 0 && (!dev_x || !dev_y)) {
    ep::set_error("null device pointer");
    return EP_ERR_ARG;
  }
  if (((uintptr_t)dev_x & 15) || ((uintptr_t)dev_y & 3) || ((uintptr_t)dev_workspace & 15)) {
    ep::set_error("dev_x and dev_workspace must be 16-byte aligned, dev_y 4-byte aligned");
    return EP_ERR_ARG;
  }
  ep_linear_plan P;
  P.m = m;
  const int rc = linear_plan(host_blob, nbytes, dev_blob, m, P.L, P.fn, P.grid, P.lds);
  if (rc != EP_OK || m == 0) return rc;
  return linear_run(P, dev_x, dev_y, y_dtype, dev_workspace, workspace_bytes, hip_stream);
}

int ep_linear_plan_create(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, int64_t m,
                          ep_linear_plan **plan_out) {
  ep::set_error("");
  if (!plan_out) {
    ep::set_error("null plan_out");
    return EP_ERR_ARG;
  }
  *plan_out = nullptr;
  ep_linear_plan *h = new (std::nothrow) ep_linear_plan;
  if (!h) {
    ep::set_error("out of host memory");
    return EP_ERR_NOMEM;
  }
  h->m = m;
  const int rc = linear_plan(host_blob, nbytes, dev_blob, m, h->L, h->fn, h->grid, h->lds);
  if (rc != EP_OK) {
    delete h;
    return rc;
  }
  *plan_out = h;
  return EP_OK;
}

int64_t ep_linear_plan_workspace_bytes(const ep_linear_plan *plan) {
  ep::set_error("");
  if (!plan) {
    ep::set_error("null plan");
    return EP_ERR_ARG;
  }
  return (plan->m > 0 && plan->L.split > 1u) ? (int64_t)plan->L.split * plan->m * (int64_t)plan->L.n * 4 : 0;
}

int ep_linear_plan_run(const ep_linear_plan *plan, const void *dev_x, void *dev_y, int y_dtype, void *dev_workspace,
                       size_t workspace_bytes, void *hip_stream) {
  ep::set_error("");
  if (!plan) {
    ep::set_error("null plan");
    return EP_ERR_ARG;
  }
  return linear_run(*plan, dev_x, dev_y, y_dtype, dev_workspace, workspace_bytes, hip_stream);
}

void ep_linear_plan_free(ep_linear_plan *plan) { delete plan; }

}  // extern "C"
