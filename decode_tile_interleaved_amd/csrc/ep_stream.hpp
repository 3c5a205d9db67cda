// ep_stream.hpp -- byte layout of a lattice-rANS stream and its host-side reader.
//
// Layout (little-endian; every section starts on a 16-byte boundary):
//   header   128 B   magic "EPK1", version, method, container dtype, prob_bits,
//                    context count, tile_vecs, states per tile, tiles, rows,
//                    cols, padded cols, lattice scale a, target bpp, section
//                    offsets, word count, total bytes
//   tables           7 x {int16 smin, uint16 nsym} then every context's
//                    uint16 frequencies back to back
//   scales           float32 g_r per row
//   states           uint32 initial decoder state per (tile, state)
//   tile offsets     uint32 word index of each tile's first word, plus the end
//   words            uint16 words, tile after tile: states / 2 words of count
//                    bytes (byte q = number of words state q consumes), then each
//                    state's words in consumption order, states ascending
// A raw stream (method 1) is the header followed by the container bytes.
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstring>
#include <string>

namespace ep {

constexpr uint32_t kMagic = 0x314B5045u;  // "EPK1"
constexpr uint16_t kVersion = 1;
constexpr uint32_t kHeaderBytes = 128;
constexpr int kContexts = 7;
constexpr int kProbBits = 10;
constexpr uint32_t kProbTotal = 1u << kProbBits;
constexpr uint32_t kStateLow = 1u << 13;   // rANS states live in [2^13, 2^29)
// stream bits per state beyond its symbols' information, as the rate
// estimate counts them: the fixed final state L (13), the unused high bits of
// the stored start state (11 on average) and the count byte (8)
constexpr double kStateBits = 32.0;
// A state absorbs up to 16 bits of information before it emits a word, so it
// never costs less than its stored 32 bits and count byte: the estimate's
// state part is max(40 * states, information + 32 * states).
constexpr double kStateMinBits = 40.0;
constexpr int kTileVecs = 1024;            // E8 vectors (8 coordinates) per tile
constexpr int kStatesPerTile = 64;         // interleaved rANS states per tile (2 count bytes per word)
// states per tile when the target lies below the overhead of kStatesPerTile
// (the stream's header says which); a tile starts with states / 2 count words
constexpr int kStatesLow = 16;
constexpr int kValueMin = -2048, kValueMax = 2047;  // lattice coordinates the stream can hold (12-bit field)

enum Method : uint8_t { kLattice = 0, kRaw = 1 };

inline size_t elem_bytes(int dtype) { return dtype <= 1 ? 2 : 1; }
inline uint64_t align16(uint64_t n) { return (n + 15) & ~uint64_t(15); }

// field offsets inside the header
namespace hdr {
constexpr size_t magic = 0, version = 4, header_bytes = 6, method = 8, dtype = 9, prob_bits = 10, contexts = 11,
                 tile_vecs = 12, states = 16, tiles = 20, rows = 24, cols = 32, cols8 = 40, scale_a = 48,
                 target = 56, off_tables = 64, off_scales = 72, off_states = 80, off_tile_offsets = 88,
                 off_words = 96, n_words = 104, total = 112;
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
  int method = 0, dtype = 0, prob_bits = 0, states = 0;
  int64_t rows = 0, cols = 0, cols8 = 0, tiles = 0, n_vec = 0;
  double scale_a = 0, target = 0;
  uint64_t off_tables = 0, off_scales = 0, off_states = 0, off_tile_offsets = 0, off_words = 0;
  uint64_t n_words = 0, total = 0;
  int16_t smin[kContexts] = {};
  uint16_t nsym[kContexts] = {};
  uint64_t freq_index[kContexts] = {};  // index of each context's first frequency (uint16 units)
  uint64_t off_freq = 0;                // byte offset of the frequency array
};

// Parses and bounds-checks the header and table directory.  Returns an empty
// string on success, else a description of the problem.
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
  if (s.rows <= 0 || s.cols <= 0 || s.rows > (int64_t(1) << 40) || s.cols > (int64_t(1) << 40)) return "bad shape";
  s.total = rd<uint64_t>(b + hdr::total);
  if (s.total != n) return "stream length does not match its header";
  s.target = rd<double>(b + hdr::target);
  if (s.method == kRaw) {
    s.off_words = rd<uint64_t>(b + hdr::off_words);
    uint64_t payload = (uint64_t)s.rows * (uint64_t)s.cols * elem_bytes(s.dtype);
    if (s.off_words != kHeaderBytes || kHeaderBytes + payload > n) return "raw payload out of bounds";
    return "";
  }
  s.prob_bits = b[hdr::prob_bits];
  if (s.prob_bits != kProbBits || b[hdr::contexts] != kContexts) return "unsupported model parameters";
  s.states = (int)rd<uint32_t>(b + hdr::states);
  if (rd<uint32_t>(b + hdr::tile_vecs) != kTileVecs || (s.states != kStatesPerTile && s.states != kStatesLow))
    return "unsupported tile geometry";
  s.cols8 = (int64_t)rd<uint64_t>(b + hdr::cols8);
  if (s.cols8 != (s.cols + 7) / 8 * 8) return "bad padded column count";
  s.n_vec = s.rows * (s.cols8 / 8);
  s.tiles = rd<uint32_t>(b + hdr::tiles);
  if (s.tiles != (s.n_vec + kTileVecs - 1) / kTileVecs) return "bad tile count";
  s.scale_a = rd<double>(b + hdr::scale_a);
  s.off_tables = rd<uint64_t>(b + hdr::off_tables);
  s.off_scales = rd<uint64_t>(b + hdr::off_scales);
  s.off_states = rd<uint64_t>(b + hdr::off_states);
  s.off_tile_offsets = rd<uint64_t>(b + hdr::off_tile_offsets);
  s.off_words = rd<uint64_t>(b + hdr::off_words);
  s.n_words = rd<uint64_t>(b + hdr::n_words);
  if (s.off_tables != kHeaderBytes) return "bad table offset";
  uint64_t nsum = 0;
  for (int c = 0; c < kContexts; ++c) {
    s.smin[c] = rd<int16_t>(b + s.off_tables + 4 * c);
    s.nsym[c] = rd<uint16_t>(b + s.off_tables + 4 * c + 2);
    s.freq_index[c] = nsum;
    nsum += s.nsym[c];
  }
  s.off_freq = s.off_tables + 4 * kContexts;
  const uint64_t T = (uint64_t)s.tiles;
  if (s.off_scales < s.off_freq + 2 * nsum || (s.off_scales & 15) || s.off_states < s.off_scales + 4 * (uint64_t)s.rows ||
      (s.off_states & 15) || s.off_tile_offsets < s.off_states + 4 * T * (uint64_t)s.states || (s.off_tile_offsets & 15) ||
      s.off_words < s.off_tile_offsets + 4 * (T + 1) || (s.off_words & 15) || s.off_words + 2 * s.n_words > n)
    return "section table out of bounds";
  if (n - s.off_words < align16(2 * s.n_words)) return "word section not padded";
  return "";
}

}  // namespace ep
