// ep_stream.hpp -- byte layout of a lattice-rANS stream and its host-side reader.
//
// Layout (little-endian; every section starts on a 16-byte boundary):
//   header   128 B   magic "EPK1", version 2, method, container dtype,
//                    prob_bits, context count, tile_vecs, states per tile,
//                    tiles, rows, cols, padded cols, lattice scale a, target
//                    bpp, section offsets (the states-section field is 0),
//                    word count, total bytes, tile layout (byte 120)
//   tables           7 x {int16 smin, uint16 nsym} then every context's
//                    uint16 frequencies back to back
//   scales           float32 g_r per row
//   tile offsets     uint32 word index of each tile's first word, plus the end
//   words            uint16 words, tile after tile.  A tile of S states:
//                      S/4 words of pair counts (byte k: words in the region
//                        of states 2k and 2k+1),
//                      S/4 words of length codes (nibble q, least significant
//                        first: W - 12, W the bit length of state q's start
//                        state, which lies in [2^11, 2^27)),
//                      the start states' bits below their leading one,
//                        states ascending, least significant bit first, on
//                        whole words,
//                      region k: state 2k's words in the order it consumes
//                        them, then state 2k+1's in reverse order (it reads
//                        its region from the end)
// A raw stream (method 1) is the header followed by the container bytes.
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstring>
#include <string>

namespace ep {

constexpr uint32_t kMagic = 0x314B5045u;  // "EPK1"
constexpr uint16_t kVersion = 2;
constexpr uint32_t kHeaderBytes = 128;
constexpr int kContexts = 7;
constexpr int kProbBits = 10;
constexpr uint32_t kProbTotal = 1u << kProbBits;
constexpr uint32_t kStateLow = 1u << 11;  // rANS states live in [2^11, 2^27)
constexpr int kStateTop = 27;             // the encoder emits a word while x >= f << (27 - kProbBits)
// Stream bits a state costs beyond its symbols' information, as the rate
// estimate counts them: half a pair-count byte and a length nibble (8), and
// the start state stored at its bit length less the implied leading one
// while it carries log2(x / 2^11) bits: 11 bits less the fractional part of
// log2 x, on average 10.5.  A state that codes nothing costs 19.
constexpr double kStateBits = 18.5;
constexpr double kStateMinBits = 19.0;
constexpr double kTilePadBits = 7.5;   // a tile's start bits end on a whole word (on average)
constexpr double kWordsPadBits = 60.0; // the word section ends on 16 bytes (on average)
constexpr int kStatesPerTile = 64;     // interleaved rANS states per tile
constexpr int kStatesLow = 16;         // per tile for low targets (the header says which)
constexpr int kTileVecsSmall = 512;    // E8 vectors (8 coordinates) per tile ...
constexpr int kTileVecsLarge = 1024;   // ... or, for 16-state tiles at the lowest targets and large matrices, 1024
constexpr int64_t kSmallMatrixVecs = int64_t(1) << 22;  // 64-state tiles of fewer vectors hold 512
constexpr int kValueMin = -2048, kValueMax = 2047;  // lattice coordinates the stream can hold (12-bit field)

enum Method : uint8_t { kLattice = 0, kRaw = 1 };

// Tile layouts (header byte 120).  The pages ask for independently decodable
// tiles and leave their shape open.
//   kLayoutRows:   tile t holds vectors t * tile_vecs ... in row-major vector
//                  order; the last tile may be partial.
//   kLayoutBlocks: tile t = nb * KB + kb (KB = ceil(vpr / 8)) is the weight
//                  block of rows 64 nb .. 64 nb + 63 and vector columns
//                  8 kb .. 8 kb + 7; its local vector i lies at row
//                  64 nb + i / 8, vector column 8 kb + i % 8 and is absent
//                  where that falls outside the matrix.  A matrix product
//                  reads W one block at a time, so the fused linear decodes
//                  each block straight into a matrix-core operand (API
//                  reference, "CompressedLinear": reconstructed weights feed
//                  every forward call).  BF16 containers, cols % 8 == 0, 64
//                  states and 512 vectors per tile.
enum Layout : uint8_t { kLayoutRows = 0, kLayoutBlocks = 1 };
constexpr int kBlockRows = 64, kBlockVecs = 8;

inline int64_t tile_count(int layout, int64_t rows, int64_t vpr, int64_t tile_vecs) {
  if (layout == kLayoutBlocks) return (rows + kBlockRows - 1) / kBlockRows * ((vpr + kBlockVecs - 1) / kBlockVecs);
  return (rows * vpr + tile_vecs - 1) / tile_vecs;
}

inline int64_t tile_vector(int layout, int64_t rows, int64_t vpr, int64_t tile_vecs, int64_t t, int64_t i) {
  if (layout == kLayoutBlocks) {
    const int64_t kb_n = (vpr + kBlockVecs - 1) / kBlockVecs;
    const int64_t r = (t / kb_n) * kBlockRows + i / kBlockVecs, k = (t % kb_n) * kBlockVecs + i % kBlockVecs;
    return (r < rows && k < vpr) ? r * vpr + k : -1;
  }
  const int64_t v = t * tile_vecs + i;
  return v < rows * vpr ? v : -1;
}

inline size_t elem_bytes(int dtype) { return dtype <= 1 ? 2 : 1; }
inline uint64_t align16(uint64_t n) { return (n + 15) & ~uint64_t(15); }

// field offsets inside the header
namespace hdr {
constexpr size_t magic = 0, version = 4, header_bytes = 6, method = 8, dtype = 9, prob_bits = 10, contexts = 11,
                 tile_vecs = 12, states = 16, tiles = 20, rows = 24, cols = 32, cols8 = 40, scale_a = 48,
                 target = 56, off_tables = 64, off_scales = 72, off_states = 80, off_tile_offsets = 88,
                 off_words = 96, n_words = 104, total = 112, layout = 120;
}

template <class T>
inline T rd(const uint8_t *p) {
  T v;
  std::memcpy(&v, p, sizeof(T));
  return v;
}
template <class T>
inline void wr(uint8_t *p, T v) {
  std::memcpy(p, &v, sizeof(T));
}

struct StreamView {
  int method = 0, dtype = 0, prob_bits = 0, states = 0, tile_vecs = 0, layout = 0;
  int64_t rows = 0, cols = 0, cols8 = 0, tiles = 0, n_vec = 0;
  double scale_a = 0, target = 0;
  uint64_t off_tables = 0, off_scales = 0, off_tile_offsets = 0, off_words = 0;
  uint64_t n_words = 0, total = 0;
  int16_t smin[kContexts] = {};
  uint16_t nsym[kContexts] = {};
  uint64_t freq_index[kContexts] = {};  // index of each context's first frequency (uint16 units)
  uint64_t off_freq = 0;                // byte offset of the frequency array
};

// true if [off, off + size) lies inside [0, n); no addition can wrap
inline bool inside(uint64_t off, uint64_t size, uint64_t n) { return off <= n && size <= n - off; }

// Parses and bounds-checks the header and table directory.  Returns an empty
// string on success, else a description of the problem.  Every bound is
// written as off <= n && size <= n - off and every product is taken on
// values capped first, so no header, however corrupt, makes a check wrap.
inline std::string parse_stream(const uint8_t *b, size_t n, StreamView &s) {
  if (!b) return "null stream";
  if (n < kHeaderBytes) return "stream shorter than its header";
  if (rd<uint32_t>(b + hdr::magic) != kMagic) return "bad magic";
  if (rd<uint16_t>(b + hdr::version) != kVersion) return "unsupported version";
  if (rd<uint16_t>(b + hdr::header_bytes) != kHeaderBytes) return "bad header size";
  s.method = b[hdr::method];
  s.dtype = b[hdr::dtype];
  if (s.method > 1 || s.dtype > 3) return "bad method or dtype";
  s.rows = (int64_t)rd<uint64_t>(b + hdr::rows);
  s.cols = (int64_t)rd<uint64_t>(b + hdr::cols);
  // both below 2^31 and their product below 2^40: every product below fits 64 bits
  if (s.rows <= 0 || s.cols <= 0 || s.rows >= (int64_t(1) << 31) || s.cols >= (int64_t(1) << 31) ||
      (uint64_t)s.rows * (uint64_t)s.cols >= (uint64_t(1) << 40))
    return "bad shape";
  s.total = rd<uint64_t>(b + hdr::total);
  if (s.total != n) return "stream length does not match its header";
  s.target = rd<double>(b + hdr::target);
  if (s.method == kRaw) {
    s.off_words = rd<uint64_t>(b + hdr::off_words);
    const uint64_t payload = (uint64_t)s.rows * (uint64_t)s.cols * elem_bytes(s.dtype);
    if (s.off_words != kHeaderBytes || !inside(kHeaderBytes, payload, n)) return "raw payload out of bounds";
    return "";
  }
  s.prob_bits = b[hdr::prob_bits];
  if (s.prob_bits != kProbBits || b[hdr::contexts] != kContexts) return "unsupported model parameters";
  s.states = (int)rd<uint32_t>(b + hdr::states);
  s.tile_vecs = (int)rd<uint32_t>(b + hdr::tile_vecs);
  if ((s.tile_vecs != kTileVecsSmall && s.tile_vecs != kTileVecsLarge) ||
      (s.states != kStatesPerTile && s.states != kStatesLow))
    return "unsupported tile geometry";
  s.cols8 = (int64_t)rd<uint64_t>(b + hdr::cols8);
  if (s.cols8 != (s.cols + 7) / 8 * 8) return "bad padded column count";
  s.n_vec = s.rows * (s.cols8 / 8);
  if (s.n_vec >= (int64_t(1) << 31)) return "stream too large";
  s.layout = b[hdr::layout];
  if (s.layout > kLayoutBlocks) return "unknown tile layout";
  if (s.layout == kLayoutBlocks &&
      (s.states != kStatesPerTile || s.tile_vecs != kTileVecsSmall || s.cols % 8 != 0 || s.dtype != 0))
    return "blocks layout needs 64-state 512-vector tiles of a BF16 matrix with cols % 8 == 0";
  s.tiles = rd<uint32_t>(b + hdr::tiles);
  if (s.tiles != tile_count(s.layout, s.rows, s.cols8 / 8, s.tile_vecs)) return "bad tile count";
  s.scale_a = rd<double>(b + hdr::scale_a);
  s.off_tables = rd<uint64_t>(b + hdr::off_tables);
  s.off_scales = rd<uint64_t>(b + hdr::off_scales);
  s.off_tile_offsets = rd<uint64_t>(b + hdr::off_tile_offsets);
  s.off_words = rd<uint64_t>(b + hdr::off_words);
  s.n_words = rd<uint64_t>(b + hdr::n_words);
  if (rd<uint64_t>(b + hdr::off_states) != 0) return "states section present";
  if (s.off_tables != kHeaderBytes || !inside(s.off_tables, 4 * kContexts, n)) return "bad table offset";
  uint64_t nsum = 0;
  for (int c = 0; c < kContexts; ++c) {
    s.smin[c] = rd<int16_t>(b + s.off_tables + 4 * c);
    s.nsym[c] = rd<uint16_t>(b + s.off_tables + 4 * c + 2);
    s.freq_index[c] = nsum;
    nsum += s.nsym[c];
  }
  s.off_freq = s.off_tables + 4 * kContexts;
  const uint64_t T = (uint64_t)s.tiles;  // below 2^22: every size below is small
  // sections in order, each inside the stream and 16-byte aligned, none
  // overlapping the one before it
  if (!inside(s.off_freq, 2 * nsum, n) || s.off_scales < s.off_freq + 2 * nsum || (s.off_scales & 15) ||
      !inside(s.off_scales, 4 * (uint64_t)s.rows, n) ||
      s.off_tile_offsets < s.off_scales + 4 * (uint64_t)s.rows || (s.off_tile_offsets & 15) ||
      !inside(s.off_tile_offsets, 4 * (T + 1), n) || s.off_words < s.off_tile_offsets + 4 * (T + 1) ||
      (s.off_words & 15) || s.n_words > n || !inside(s.off_words, 2 * s.n_words, n))
    return "section table out of bounds";
  if (n - s.off_words < align16(2 * s.n_words)) return "word section not padded";
  return "";
}

}  // namespace ep
