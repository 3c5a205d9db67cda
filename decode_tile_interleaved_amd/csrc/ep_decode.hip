// ep_decode.hip -- fused lattice-rANS tile decode and weight reconstruction
// for gfx950 (MI355X).
//
// The EntroPack abstract (mlsanity index page) states that the coordinates
// are entropy-coded in independently decodable tiles so that symbol decoding
// and numerical reconstruction fuse on the GPU.  This file is that pass.
//
// Work mapping: one wavefront per tile of 1024 E8 vectors; lane q owns rANS
// state q and decodes local vectors q, q+64, ..., so every step's 64 vectors
// are contiguous and each lane writes one 8-coordinate vector per step
// (16 bytes for BF16/FP16, 8 bytes for FP8/INT8).  Streams for targets below
// the overhead of 64 states have 16 per tile: lanes 0..15 decode vectors q,
// q+16, ..., and lanes 16..63 follow along without refilling or storing.
//
// Per workgroup (up to 8 waves, one workgroup per CU):
//   1. every wave starts its global loads, all vector loads that need only the
//      kernel arguments: the tile offsets it needs, one context's frequencies,
//      its tile's start states and row scales;
//   2. one wave per context prefix-sums the frequencies (DPP scan), lists the
//      used symbols, sets a bitmap of the slots where a symbol starts, and
//      expands the context's table 64 slots at a time: a slot's symbol is the
//      number of starts up to it, which v_mbcnt counts from the row's bitmap;
//      the last wave copies the words of all the workgroup's tiles (one range
//      of the stream) into LDS with global_load_lds;
//   3. each wave decodes its tile.
// Streams with more tiles than one such round of workgroups covers take the
// multi-tile kernel instead: one workgroup of up to 16 waves per CU builds
// the tables once, and each wave then loads and decodes one tile after
// another on its own.
//
// Decode step for state x in [2^13, 2^29), kept as X = 8x so that the table
// address is one AND-OR:  8*slot = X & 0x1ff8;  e = table[ctx][slot];
//   x' = f * (x >> 10) + (slot - cum);  if x' < 2^13: x = x' << 16 | w
// where w is the state's next word.  A tile stores each state's words
// together (behind one count byte per state), so a lane walks its own word
// list with a private pointer and always holds its next word in a register.
//
// The step is software-pipelined around its one serial dependence, table
// lookup -> multiply-add -> compare -> select -> address -> next lookup (on
// gfx950 a dependent VALU op costs ten-odd cycles, an eight-byte LDS lookup
// about sixty).  The refilled state (x' with the held word shifted in) is
// formed in parallel with the compare, one v_cndmask selects the next state,
// one v_bitop3 or v_and_or makes its address, and the next lookup leaves.  Only
// then do the refilling lanes, under the exec mask, read their following
// word, which is first needed one step later.  Eight VALU instructions per
// step: the chain is one instruction longer than with both candidate
// addresses formed before the select, but the step is one instruction
// shorter, which pays where the VALU is the bound (more than two waves per
// SIMD).
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

#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "ep.h"
#include "ep_encode.hpp"
#include "ep_stream.hpp"

namespace ep {
namespace {

constexpr int kMaxWaves = 8;        // decoding waves per workgroup, single-round kernel
constexpr int kMaxTileWaves = 16;  // multi-tile kernel: four per SIMD cover the decode chain
constexpr uint32_t kCtxBytes = kProbTotal * 8;             // 8 KB per context
constexpr uint32_t kTableBytes = kContexts * kCtxBytes;     // 57344
constexpr uint32_t kRows = kProbTotal / 64;                // 16 rows of 64 slots per context
constexpr uint32_t kMarkWords = kProbTotal / 32;           // 32 bitmap words per context
constexpr uint32_t kLdsLimit = 160 * 1024;
// slack after the last word buffer: a lane of a corrupt tile reads at most
// 128 words past its clamped start, i.e. 258 bytes past the tile's end
constexpr uint32_t kLdsPad = 512;
constexpr int kOutSym = 4;         // int16 lattice coordinates; 0..3 are the container dtypes

static_assert(kProbBits == 10, "table addressing below assumes 2^10 slots per context");

// Kernel arguments.  The fields the first global loads need come first, so
// that they arrive with the first batch of scalar loads.
struct Args {
  const uint8_t *blob;
  uint64_t off_freq, off_tile_offsets, off_states, off_scales, off_words;
  uint32_t nsym[kContexts];
  uint32_t fidx[kContexts];
  uint32_t nzbase[kContexts];
  int32_t smin[kContexts];
  void *out;
  uint64_t cols;                  // columns of the output (padded layouts only)
  uint32_t rows, vpr;             // rows; vectors per row
  uint32_t row_magic, row_shift;  // vec / vpr = umulhi(vec, row_magic) >> row_shift  (vpr > 1)
  uint32_t n_vec, n_tiles, waves;
  uint32_t rec_off, mark_off, words_off;  // LDS byte offsets
  uint32_t wg_q, wg_rem;  // multi-tile kernel: workgroup b decodes wg_q tiles, one more if b < wg_rem
  uint32_t wbuf;          // multi-tile kernel: bytes of each wave's word buffer
};

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
  const bool need = active && x < 0x10000u;
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
    L.r = lds_u16(L.p + 2u);
    L.p += 2u;
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

// writes one decoded vector.  row is the wave-uniform address of this step's
// 64 vectors (unpadded layouts); local is the vector's index in the tile.
template <int OUT, bool WIDE, bool PADDED>
__device__ __forceinline__ void emit_vector(const Args &A, gbyte_t row, uint32_t tile, uint32_t local,
                                            uint32_t lane, const uint32_t (&e)[8], float g) {
  constexpr uint32_t kVecBytes = (OUT == EP_FP8_E4M3FN || OUT == EP_INT8) ? 8u : 16u;
  const uint32_t lane_off = kVecBytes * lane;
  if constexpr (OUT == kOutSym) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = ((uint32_t)entry_value<WIDE>(e[2 * k]) & 0xffffu) | ((uint32_t)entry_value<WIDE>(e[2 * k + 1]) << 16);
    const u32x4 pk = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(pk, (__attribute__((address_space(1))) u32x4 *)(row + lane_off));
    return;
  } else {
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = entry_weight<WIDE>(e[j], g);
    if constexpr (!PADDED) {
      if constexpr (OUT == EP_BF16 || OUT == EP_FP16) {
        const u32x4 pk = {pack2<OUT>(y[0], y[1]), pack2<OUT>(y[2], y[3]), pack2<OUT>(y[4], y[5]), pack2<OUT>(y[6], y[7])};
        __builtin_nontemporal_store(pk, (__attribute__((address_space(1))) u32x4 *)(row + lane_off));
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
        __builtin_nontemporal_store(pk, (__attribute__((address_space(1))) u32x2 *)(row + lane_off));
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
        __builtin_nontemporal_store(pk, (__attribute__((address_space(1))) u32x2 *)(row + lane_off));
      }
    } else {
      const uint32_t vec = tile * 1024u + local;
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

// the row scale of vector vec (the last row's for vectors past the end)
__device__ __forceinline__ float row_scale(const Args &A, uint32_t vec) {
  const float *scales = reinterpret_cast<const float *>(A.blob + A.off_scales);
  const uint32_t last = A.rows - 1u, one = A.vpr == 1u ? 0xffffffffu : 0u;
  const uint32_t r = ((__umulhi(vec, A.row_magic) >> A.row_shift) & ~one) | (vec & one);
  return scales[r < last ? r : last];
}

// decodes one tile of NS states; PARTIAL handles the last tile of a stream
// (n < 1024).  wb and we are the LDS byte addresses of the tile's first word
// and of its end; X is 8 * the start state.  Lane q < NS decodes vectors q,
// q + NS, ...; with NS = 64, gs holds the row scale of each of its 16
// vectors, with fewer states the scales of each group of 16 steps are loaded
// as the group starts, and lanes from NS on only follow along (they never
// refill or store).
//
// BOP3: the lookup address by v_bitop3 rather than v_and_or.  On gfx950 the
// first issues faster (about 1.9 against 2.8 SIMD cycles per instruction with
// four waves per SIMD) at the same dependent latency; it measured 1.5-2%
// faster in the single-round kernel and for 8-bit outputs, but 1-2.5% slower
// for 16-bit outputs in the multi-tile kernel, whose code differs in that
// instruction alone, so each kernel takes the faster form.
template <int OUT, bool WIDE, bool PADDED, bool PARTIAL, bool BOP3, int NS>
__device__ __forceinline__ void decode_tile(const Args &A, uint32_t wb, uint32_t we, uint32_t X, uint32_t tile,
                                            uint32_t n, const float (&gs)[16], uint32_t lane) {
  static_assert(NS == 64 || NS == 16, "states per tile");
  constexpr uint32_t kNs = (uint32_t)NS;
  constexpr uint32_t kGroups = 1024u / kNs / 16u;  // groups of 16 steps
  const bool mine = NS == 64 || lane < kNs;        // this lane holds one of the tile's states
  Lane L;
  table_read<0u>(X & 0x1ff8u, L.d0, L.d1);  // context F
  L.q = X >> 13;
  // this state's words follow the NS count bytes and the words of the states
  // before it; the clamp keeps every read of a corrupt tile inside the LDS
  // allocation
  const uint32_t cnt = mine ? lds_u8(wb + lane) : 0u;
  const uint32_t p = wb + kNs + 2u * (wave_inclusive_sum(cnt) - cnt);
  L.p = p < we ? p : we;
  L.r = lds_u16(L.p);
  constexpr uint32_t kC = kCtxBytes, kE = 3u * kCtxBytes;  // LDS bases of C_0 and E_{0,0}
  constexpr uint32_t kBitB = WIDE ? 16u : 24u;  // where bit 0 of v sits in d0
  constexpr uint32_t kVecBytes = (OUT == EP_FP8_E4M3FN || OUT == EP_INT8) ? 8u : 16u;
  constexpr uint32_t kStepBytes = kNs * kVecBytes;
  const gbyte_t tile_out = (gbyte_t)A.out + (uint64_t)tile * (1024u * kVecBytes);
#pragma unroll 1
  for (uint32_t grp = 0; grp < kGroups; ++grp) {
    if (PARTIAL && grp * 16u * kNs >= n) break;
    float gl[16];
    if constexpr (NS != 64) {
#pragma unroll
      for (uint32_t s = 0; s < 16; ++s) gl[s] = row_scale(A, tile * 1024u + (grp * 16u + s) * kNs + (mine ? lane : 0u));
    }
#pragma unroll
    for (uint32_t s = 0; s < 16; ++s) {
      const uint32_t t = grp * 16u + s;  // step
      const bool act = mine && (PARTIAL ? (t * kNs + lane < n) : true);
      if (PARTIAL && t * kNs >= n) break;
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
      if (act)
        emit_vector<OUT, WIDE, PADDED>(A, opaque_s(tile_out + t * kStepBytes), tile, t * kNs + lane, lane, e,
                                       NS == 64 ? gs[s] : gl[s]);
    }
  }
}

// The table build: waves 0..k-1 take contexts wave, wave + k, ...: prefix
// sums of the frequencies, the used symbols' records, a bitmap of the slots
// where a symbol starts, then the context's 16 table rows of 64 slots.  fpre
// holds the first 256 frequencies of context `wave`, loaded early.
template <bool WIDE>
__device__ __forceinline__ void build_tables(const Args &A, uint8_t *lds, uint32_t wave, uint32_t lane, uint32_t k,
                                             const uint32_t (&fpre)[4]) {
  const uint16_t *freq = reinterpret_cast<const uint16_t *>(A.blob + A.off_freq);
  uint2 *rec = reinterpret_cast<uint2 *>(lds + A.rec_off);          // (d0, cum term) per used symbol
  uint32_t *mark = reinterpret_cast<uint32_t *>(lds + A.mark_off);  // [ctx][32] start bits
  uint32_t *tab = reinterpret_cast<uint32_t *>(lds);
  for (uint32_t c = wave; c < (uint32_t)kContexts; c += k) {
    const uint32_t n = pick(A.nsym, c), fidx = pick(A.fidx, c), nzbase = pick(A.nzbase, c);
    const int32_t smin = pick(A.smin, c);
    if (n == 0u) continue;  // context without symbols: its table is never read
    const uint32_t lc = c < 3u ? c : 3u + ((c - 3u) >> 1) + 2u * ((c - 3u) & 1u);  // LDS context of E_{b,p}
    if (lane < kMarkWords) mark[c * kMarkWords + lane] = 0u;
    uint32_t carry = 0, nzb = nzbase;
    for (uint32_t base = 0, it = 0; base < n; base += 64, ++it) {
      const uint32_t s = base + lane;
      uint32_t f;
      if (c == wave && it < 4) f = it == 0 ? fpre[0] : it == 1 ? fpre[1] : it == 2 ? fpre[2] : fpre[3];
      else f = s < n ? freq[fidx + s] : 0u;
      const uint32_t incl = wave_inclusive_sum(f);
      const uint32_t cum = carry + incl - f;
      const bool used = f != 0;
      const uint64_t m = __ballot(used);
      const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, nzb));
      if (used && cum < kProbTotal) {
        const int32_t v = symbol_value(c, smin + (int32_t)s);
        rec[r] = make_uint2((f << 3) | (WIDE ? ((uint32_t)v & 0xffffu) << 16 : ((uint32_t)v & 0xffu) << 24),
                            cum << 3);
        atomicOr(&mark[c * kMarkWords + (cum >> 5)], 1u << (cum & 31u));
      }
      carry += __builtin_amdgcn_readlane(incl, 63);
      nzb += (uint32_t)__popcll(m);
    }
    // row t (lane t < 16): its start bits shifted down by one and the record
    // index before it
    uint32_t rlo = 0, rhi = 0, rbase = 0;
    {
      uint32_t lo = 0, hi = 0;
      if (lane < kRows) {
        lo = mark[c * kMarkWords + 2 * lane];
        hi = mark[c * kMarkWords + 2 * lane + 1];
      }
      const uint32_t cnt = (uint32_t)(__popc(lo) + __popc(hi));
      const uint32_t first = nzbase + row16_inclusive_sum(cnt) - cnt;
      rlo = __builtin_amdgcn_alignbit(hi, lo, 1u);
      rhi = hi >> 1;
      rbase = first + (lo & 1u) - 1u;
    }
    // slot record = first + (starts at or below the slot) - 1
    //             = first + bit0 - 1 + popcount of (bits >> 1) below the lane.
    // The row values reach every lane through readlane (no LDS traffic), and
    // all sixteen records are read before any table write: the compiler cannot
    // tell the record list and the table apart, so interleaving would put an
    // LDS round trip on every row.
    uint2 rc[kRows];
#pragma unroll
    for (uint32_t row = 0; row < kRows; ++row) {
      const uint32_t mlo = __builtin_amdgcn_readlane(rlo, row), mhi = __builtin_amdgcn_readlane(rhi, row);
      const uint32_t b = __builtin_amdgcn_readlane(rbase, row);
      rc[row] = rec[__builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, b))];
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

// Multi-tile kernel: workgroup b decodes the consecutive tiles
// [wg_first(b), wg_first(b + 1)); the counts differ by at most one tile.
__device__ __forceinline__ uint32_t wg_first(const Args &A, uint32_t b) {
  return b * A.wg_q + (b < A.wg_rem ? b : A.wg_rem);
}

// What a wave needs in registers to decode one tile: its start states, the
// row scale of each of its lane's vectors, and where its words land in LDS.
struct TileIn {
  uint32_t x0;
  float gs[16];
  uint32_t wt, we;  // LDS byte addresses of the tile's first word and of its end
};

// Issues a tile's loads: start states and row scales (vector loads), word
// offsets (scalar loads), and the copy of its words into LDS at buf with
// global_load_lds (1 KB per instruction; lanes past the end of the last,
// partial kilobyte re-read its last 16 bytes).  Only the copy's addresses
// wait, for the word offsets; nothing waits for the rest.
template <int NS>
__device__ __forceinline__ TileIn issue_tile(const Args &A, uint8_t *lds, uint32_t tile, uint32_t buf, uint32_t lane) {
  TileIn T;
  T.x0 = reinterpret_cast<const uint32_t *>(A.blob + A.off_states)[tile * (uint32_t)NS + (lane < (uint32_t)NS ? lane : 0u)];
  if constexpr (NS == 64) {
    const float *scales = reinterpret_cast<const float *>(A.blob + A.off_scales);
    const uint32_t last = A.rows - 1u, one = A.vpr == 1u ? 0xffffffffu : 0u;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint32_t vec = tile * 1024u + 64u * s + lane;
      const uint32_t r = ((__umulhi(vec, A.row_magic) >> A.row_shift) & ~one) | (vec & one);
      T.gs[s] = scales[r < last ? r : last];  // lanes past the end read the last row; their values are unused
    }
  }
  typedef __attribute__((address_space(4))) const uint32_t *cptr_u32;
  const cptr_u32 toff = (cptr_u32)(A.blob + A.off_tile_offsets);
  const uint32_t w_begin = toff[tile], w_end = toff[tile + 1u];
  const uint64_t gbyte0 = (A.off_words + 2ull * w_begin) & ~15ull;
  const uint32_t nchunks = (uint32_t)((((A.off_words + 2ull * w_end + 15ull) & ~15ull) - gbyte0) >> 4);
  const gbyte_t src = (gbyte_t)(A.blob + gbyte0);
  uint32_t i = 0;
  for (; 64u * i + 64u <= nchunks; ++i)
    __builtin_amdgcn_global_load_lds((gptr_t)(src + 1024u * i + 16u * lane), (lptr_t)(lds + buf + 1024u * i), 16, 0, 0);
  if (64u * i < nchunks) {
    const uint32_t ch = lane + 64u * i;
    __builtin_amdgcn_global_load_lds((gptr_t)(src + 16u * (ch < nchunks ? ch : nchunks - 1u)),
                                     (lptr_t)(lds + buf + 1024u * i), 16, 0, 0);
  }
  T.wt = buf + (uint32_t)(A.off_words + 2ull * w_begin - gbyte0);
  T.we = T.wt + 2u * (w_end - w_begin);
  return T;
}

// workgroup barrier that orders LDS accesses: every LDS access before it has
// completed, none after it has started
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Streams with more tiles than one round of workgroups covers: one
// workgroup per CU builds the tables once, then each of its k waves decodes
// tiles first + wave, first + wave + k, ... of the workgroup's run on its
// own, copying each tile's words into a buffer of its own.  After the tables
// no wave waits for another: while one waits for its next tile's loads, the
// other waves of its SIMD keep the VALU busy (four waves per SIMD cover the
// decode chain's latency).
template <int OUT, bool WIDE, bool PADDED, int NS>
__global__ void __launch_bounds__(64 * kMaxTileWaves) decode_waves_kernel(Args A) {
  extern __shared__ __align__(16) uint8_t lds[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t k = A.waves;
  const uint32_t end = wg_first(A, blockIdx.x + 1u);
  const uint32_t buf = A.words_off + wave * A.wbuf;  // this wave's word buffer
  constexpr bool kNarrowOut = OUT == EP_FP8_E4M3FN || OUT == EP_INT8;  // lookup address by v_bitop3

  // ---- 1. the first context's frequencies ----------------------------------
  const uint16_t *freq = reinterpret_cast<const uint16_t *>(A.blob + A.off_freq);
  const uint32_t c0 = wave < (uint32_t)kContexts ? wave : 0u;
  uint32_t fpre[4];
  {
    const uint32_t n0 = pick(A.nsym, c0), f0 = pick(A.fidx, c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t s = 64u * i + lane;
      const uint32_t v = freq[f0 + (s < n0 ? s : 0u)];
      fpre[i] = s < n0 ? v : 0u;
    }
  }
  uint32_t tile = wg_first(A, blockIdx.x) + wave;
  const uint32_t tc = tile < end ? tile : end - 1u;  // waves without a tile load a valid one and drop it
  // Waves that build no table issue their first tile's loads now and start
  // decoding right after the barrier; the table builders issue theirs after
  // their table, so that no wait for a tile's loads (the compiler waits for
  // every copy into LDS before the next LDS access) delays a table.
  const bool builder = wave < (uint32_t)kContexts;
  TileIn T;
  if (!builder) T = issue_tile<NS>(A, lds, tc, buf, lane);

  // ---- 2. the tables -------------------------------------------------------
  build_tables<WIDE>(A, lds, wave, lane, k, fpre);
  if (builder) T = issue_tile<NS>(A, lds, tc, buf, lane);
  lds_barrier();  // tables built (every wave's LDS writes done)

  // ---- 3. this wave's tiles --------------------------------------------------
  while (tile < end) {
    __builtin_amdgcn_s_waitcnt(0);  // the tile's states, scales and words have landed
    const uint32_t n = min(1024u, A.n_vec - tile * 1024u);
    if (n == 1024u)
      decode_tile<OUT, WIDE, PADDED, false, kNarrowOut, NS>(A, T.wt, T.we, T.x0 << 3, tile, n, T.gs, lane);
    else
      decode_tile<OUT, WIDE, PADDED, true, kNarrowOut, NS>(A, T.wt, T.we, T.x0 << 3, tile, n, T.gs, lane);
    tile += k;
    if (tile < end) {
      __builtin_amdgcn_s_waitcnt(0);  // every read of the finished tile's words is done before they are overwritten
      T = issue_tile<NS>(A, lds, tile, buf, lane);
    }
  }
}

// Streams that one round of workgroups covers: workgroups of up to 8 waves,
// one tile each.
template <int OUT, bool WIDE, bool PADDED, int NS>
__global__ void __launch_bounds__(64 * kMaxWaves) decode_kernel(Args A) {
  extern __shared__ __align__(16) uint8_t lds[];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t nwaves = A.waves;

  // ---- 1. global loads, all unconditional so that each wait is exact ----
  const uint32_t tile = blockIdx.x * nwaves + wave;
  const bool has_tile = tile < A.n_tiles;
  const uint32_t tc = has_tile ? tile : A.n_tiles - 1u;  // waves without a tile load a valid one and drop it
  // The workgroup's tiles are consecutive, so their words are one range of
  // the stream.  The tile offsets the wave needs come first, from one vector
  // load (lane 0: its tile's first word, lane 1: the tile's end, lanes 2 and
  // 3: the workgroup's range): scalar loads would share their counter with
  // the table build's LDS accesses, whose waits would then wait for them too.
  const uint32_t g0 = blockIdx.x * nwaves;
  const uint32_t gend = g0 + nwaves < A.n_tiles ? g0 + nwaves : A.n_tiles;
  const uint32_t oi = lane == 0u ? tc : lane == 1u ? tc + 1u : lane == 2u ? g0 : gend;
  const uint32_t ov = reinterpret_cast<const uint32_t *>(A.blob + A.off_tile_offsets)[oi];
  // the first 256 frequencies of this wave's first context (they need
  // nothing but the kernel arguments)
  const uint16_t *freq = reinterpret_cast<const uint16_t *>(A.blob + A.off_freq);
  const uint32_t c0 = wave < (uint32_t)kContexts ? wave : 0u;
  uint32_t fpre[4];
  {
    const uint32_t n0 = pick(A.nsym, c0), f0 = pick(A.fidx, c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t s = 64u * i + lane;
      const uint32_t v = freq[f0 + (s < n0 ? s : 0u)];
      fpre[i] = s < n0 ? v : 0u;
    }
  }
  const uint32_t x0 =
      reinterpret_cast<const uint32_t *>(A.blob + A.off_states)[tc * (uint32_t)NS + (lane < (uint32_t)NS ? lane : 0u)];
  float gs[16];
  if constexpr (NS == 64) {
    const float *scales = reinterpret_cast<const float *>(A.blob + A.off_scales);
    const uint32_t last = A.rows - 1u, one = A.vpr == 1u ? 0xffffffffu : 0u;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint32_t vec = tc * 1024u + 64u * s + lane;
      const uint32_t r = ((__umulhi(vec, A.row_magic) >> A.row_shift) & ~one) | (vec & one);
      gs[s] = scales[r < last ? r : last];  // lanes past the end read the last row; their values are unused
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the loads above go out before anything waits
  // ---- 2. one wave per context: the tables --------------------------------
  build_tables<WIDE>(A, lds, wave, lane, nwaves, fpre);

  // The last wave (which builds no table when the workgroup has eight waves)
  // copies the workgroup's words into LDS with global_load_lds (1 KB per
  // instruction, lanes past the end re-read the last 16 bytes).  This comes
  // after the table build: where the copying branch rejoins, the compiler
  // waits for every load, so before the build that wait would hold every
  // builder until its tile's states and scales had landed.
  if (wave == nwaves - 1u) {
    const uint64_t gbyte0 = (A.off_words + 2ull * __builtin_amdgcn_readlane(ov, 2)) & ~15ull;
    const uint32_t nchunks =
        (uint32_t)((((A.off_words + 2ull * __builtin_amdgcn_readlane(ov, 3) + 15ull) & ~15ull) - gbyte0) >> 4);
    const gbyte_t src = (gbyte_t)(A.blob + gbyte0);
    // whole kilobytes first: no per-lane clamp, so each load issues right
    // after the last one
    uint32_t i = 0;
    for (; 64u * i + 64u <= nchunks; ++i)
      __builtin_amdgcn_global_load_lds((gptr_t)(src + 1024u * i + 16u * lane), (lptr_t)(lds + A.words_off + 1024u * i),
                                       16, 0, 0);
    if (64u * i < nchunks) {
      const uint32_t ch = lane + 64u * i;
      __builtin_amdgcn_global_load_lds((gptr_t)(src + 16u * (ch < nchunks ? ch : nchunks - 1u)),
                                       (lptr_t)(lds + A.words_off + 1024u * i), 16, 0, 0);
    }
  }

  __builtin_amdgcn_s_waitcnt(0);  // the loader's words have landed in LDS
  __syncthreads();

  // ---- 3. decode ---------------------------------------------------------
  if (!has_tile) return;
  const uint32_t n = min(1024u, A.n_vec - tile * 1024u);
  const uint32_t X = x0 << 3;
  const uint32_t w_begin = __builtin_amdgcn_readlane(ov, 0), w_end = __builtin_amdgcn_readlane(ov, 1);
  const uint64_t gbyte0 = (A.off_words + 2ull * __builtin_amdgcn_readlane(ov, 2)) & ~15ull;  // 16-byte aligned start of the range
  const uint32_t wt = A.words_off + (uint32_t)(A.off_words + 2ull * w_begin - gbyte0);  // LDS address of this tile's first word
  const uint32_t we = wt + 2u * (w_end - w_begin);
  if (n == 1024u)
    decode_tile<OUT, WIDE, PADDED, false, true, NS>(A, wt, we, X, tile, n, gs, lane);
  else
    decode_tile<OUT, WIDE, PADDED, true, true, NS>(A, wt, we, X, tile, n, gs, lane);
}

typedef void (*KernelFn)(Args);

template <int OUT, bool WIDE, bool PADDED>
KernelFn pick3(bool multi, bool low) {
  if (low) return multi ? decode_waves_kernel<OUT, WIDE, PADDED, kStatesLow> : decode_kernel<OUT, WIDE, PADDED, kStatesLow>;
  return multi ? decode_waves_kernel<OUT, WIDE, PADDED, kStatesPerTile> : decode_kernel<OUT, WIDE, PADDED, kStatesPerTile>;
}

template <int OUT>
KernelFn pick(bool wide, bool padded, bool multi, bool low) {
  if (wide) return padded ? pick3<OUT, true, true>(multi, low) : pick3<OUT, true, false>(multi, low);
  return padded ? pick3<OUT, false, true>(multi, low) : pick3<OUT, false, false>(multi, low);
}

// low: the stream has kStatesLow states per tile
KernelFn pick_kernel(int out, bool wide, bool padded, bool multi, bool low) {
  switch (out) {
    case EP_BF16: return pick<EP_BF16>(wide, padded, multi, low);
    case EP_FP16: return pick<EP_FP16>(wide, padded, multi, low);
    case EP_FP8_E4M3FN: return pick<EP_FP8_E4M3FN>(wide, padded, multi, low);
    case EP_INT8: return pick<EP_INT8>(wide, padded, multi, low);
    default: return pick<kOutSym>(wide, false, multi, low);
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

// host-side checks and launch geometry; returns 0 or an ep_status
int launch(const uint8_t *hb, const StreamView &s, const void *dev_blob, void *dev_out, int out, hipStream_t stream) {
  if (!dev_blob || !dev_out) {
    set_error("null device pointer");
    return EP_ERR_ARG;
  }
  if (((uintptr_t)dev_blob & 15) || ((uintptr_t)dev_out & 15)) {
    set_error("device buffers must be 16-byte aligned");
    return EP_ERR_ARG;
  }
  if (s.n_vec >= (int64_t(1) << 31) || s.rows >= (int64_t(1) << 31)) {
    set_error("stream too large");
    return EP_ERR_FORMAT;
  }
  // tile offsets: monotone, inside the word section, room for the count bytes
  const uint8_t *toff = hb + s.off_tile_offsets;
  for (int64_t t = 0; t < s.tiles; ++t) {
    const uint32_t b = rd<uint32_t>(toff + 4 * t), e = rd<uint32_t>(toff + 4 * t + 4);
    if (e < b || e > s.n_words || e - b < (uint32_t)s.states / 2u) {
      set_error("corrupt tile offsets");
      return EP_ERR_FORMAT;
    }
  }
  if (rd<uint32_t>(toff + 4 * s.tiles) != s.n_words) {
    set_error("corrupt tile offsets");
    return EP_ERR_FORMAT;
  }
  // tables: frequencies sum to 2^10, used values inside the entry field
  Args A{};
  bool wide = false;
  uint32_t nz_total = 0;
  for (int c = 0; c < kContexts; ++c) {
    A.smin[c] = s.smin[c];
    A.nsym[c] = s.nsym[c];
    A.fidx[c] = (uint32_t)s.freq_index[c];
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
  // LDS layout: tables | records | bitmap | words | pad.  The
  // words of a workgroup's consecutive tiles are one range; with k waves per
  // workgroup the buffer holds the longest such range, in whole 1 KB copies.
  uint32_t off = kTableBytes;
  A.rec_off = off;
  off += 8 * nz_total;
  A.mark_off = off;
  off = (uint32_t)align16(off + 4 * kContexts * kMarkWords);
  A.words_off = off;
  auto span_for = [&](uint32_t k) {
    uint64_t span = 0;
    for (int64_t t = 0; t < s.tiles; t += k) {
      const int64_t e = std::min<int64_t>(t + k, s.tiles);
      const uint64_t a0 = (s.off_words + 2ull * rd<uint32_t>(toff + 4 * t)) & ~15ull;
      const uint64_t a1 = (s.off_words + 2ull * rd<uint32_t>(toff + 4 * e) + 15ull) & ~15ull;
      span = std::max<uint64_t>(span, a1 - a0);
    }
    return (span + 1023ull) & ~1023ull;
  };
  uint32_t waves = 0;
  uint64_t span = 0;
  for (uint32_t k = kMaxWaves; k >= 1; --k) {
    span = span_for(k);
    if (off + span + kLdsPad <= kLdsLimit) {
      waves = k;
      break;
    }
  }
  if (!waves) {
    set_error("tile too large for the decoder's LDS budget");
    return EP_ERR_FORMAT;
  }
  uint32_t lds_bytes = off + (uint32_t)span + kLdsPad;
  uint32_t grid = (uint32_t)((s.tiles + waves - 1) / waves);
  // More workgroups than compute units: the multi-tile kernel instead, with
  // one workgroup per CU that builds the tables once.
  const bool multi = (int64_t)grid > num_cus();
  if (multi) {
    // One workgroup per CU, each with a run of consecutive tiles (counts that
    // differ by at most one); its k waves take the run's tiles in turn.  k is
    // as many waves as the run and the LDS allow (at most 16, four per SIMD).
    // Measured on runs of 17 to 40 tiles, no smaller k with fewer or evener
    // passes does better: 18 tiles per CU take 15% less time as 16 waves (two
    // of them with a second tile) than as 9 waves of two tiles each.  Every
    // wave has a buffer for one tile's words, copied in whole kilobytes from
    // a 16-byte aligned start.
    uint64_t wbuf = 0;
    for (int64_t t = 0; t < s.tiles; ++t) {
      const uint64_t a0 = (s.off_words + 2ull * rd<uint32_t>(toff + 4 * t)) & ~15ull;
      const uint64_t a1 = (s.off_words + 2ull * rd<uint32_t>(toff + 4 * t + 4) + 15ull) & ~15ull;
      wbuf = std::max<uint64_t>(wbuf, (a1 - a0 + 1023ull) & ~1023ull);
    }
    const uint64_t room = kLdsLimit - std::min<uint64_t>(kLdsLimit, (uint64_t)A.words_off + kLdsPad);
    const int64_t kmax = std::min<int64_t>(kMaxTileWaves, (int64_t)(room / wbuf));
    if (kmax < 1) {
      set_error("tile too large for the decoder's LDS budget");
      return EP_ERR_FORMAT;
    }
    const int64_t g = std::min<int64_t>(s.tiles, num_cus());
    const int64_t q = s.tiles / g, rem = s.tiles % g, qmax = q + (rem ? 1 : 0);
    waves = (uint32_t)std::min<int64_t>(kmax, qmax);
    grid = (uint32_t)g;
    A.wg_q = (uint32_t)q;
    A.wg_rem = (uint32_t)rem;
    A.wbuf = (uint32_t)wbuf;
    lds_bytes = A.words_off + waves * (uint32_t)wbuf + kLdsPad;
  }
  A.blob = reinterpret_cast<const uint8_t *>(dev_blob);
  A.out = dev_out;
  A.off_freq = s.off_freq;
  A.off_scales = s.off_scales;
  A.off_states = s.off_states;
  A.off_tile_offsets = s.off_tile_offsets;
  A.off_words = s.off_words;
  A.cols = (uint64_t)s.cols;
  A.rows = (uint32_t)s.rows;
  A.vpr = (uint32_t)(s.cols8 / 8);
  if (A.vpr > 1) row_divider(A.vpr, A.row_magic, A.row_shift);
  A.n_vec = (uint32_t)s.n_vec;
  A.n_tiles = (uint32_t)s.tiles;
  const bool padded = out != kOutSym && (s.cols % 8) != 0;
  KernelFn fn = pick_kernel(out, wide, padded, multi, s.states == kStatesLow);
  static std::mutex mu;
  static std::vector<KernelFn> configured;
  {
    std::lock_guard<std::mutex> lk(mu);
    bool done = false;
    for (KernelFn k : configured) done |= k == fn;
    if (!done) {
      if (hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsLimit) != hipSuccess) {
        set_error("hipFuncSetAttribute failed");
        return EP_ERR_DEVICE;
      }
      configured.push_back(fn);
    }
  }
  A.waves = waves;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * waves), lds_bytes, stream, A);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error(std::string("kernel launch failed: ") + hipGetErrorString(err));
    return EP_ERR_DEVICE;
  }
  return EP_OK;
}

}  // namespace
}  // namespace ep

extern "C" {

int ep_decompress(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, void *dev_out, int out_dtype,
                  void *hip_stream) {
  ep::set_error("");
  ep::StreamView s;
  std::string e = ep::parse_stream(host_blob, nbytes, s);
  if (!e.empty()) {
    ep::set_error(e);
    return EP_ERR_FORMAT;
  }
  if (out_dtype != -1 && out_dtype != s.dtype) {
    ep::set_error("out_dtype must be -1 or the container dtype");
    return EP_ERR_ARG;
  }
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  if (s.method == ep::kRaw) {
    if (!dev_blob || !dev_out) {
      ep::set_error("null device pointer");
      return EP_ERR_ARG;
    }
    const size_t payload = (size_t)s.rows * (size_t)s.cols * ep::elem_bytes(s.dtype);
    if (hipMemcpyAsync(dev_out, reinterpret_cast<const uint8_t *>(dev_blob) + ep::kHeaderBytes, payload,
                       hipMemcpyDeviceToDevice, stream) != hipSuccess) {
      ep::set_error("hipMemcpyAsync failed");
      return EP_ERR_DEVICE;
    }
    return EP_OK;
  }
  return ep::launch(host_blob, s, dev_blob, dev_out, s.dtype, stream);
}

int ep_decode_symbols(const uint8_t *host_blob, size_t nbytes, const void *dev_blob, int16_t *dev_sym,
                      void *hip_stream) {
  ep::set_error("");
  ep::StreamView s;
  std::string e = ep::parse_stream(host_blob, nbytes, s);
  if (!e.empty()) {
    ep::set_error(e);
    return EP_ERR_FORMAT;
  }
  if (s.method != ep::kLattice) {
    ep::set_error("raw streams hold no lattice symbols");
    return EP_ERR_ARG;
  }
  return ep::launch(host_blob, s, dev_blob, dev_sym, ep::kOutSym, reinterpret_cast<hipStream_t>(hip_stream));
}

}  // extern "C"
