// ep_encode.hpp -- the encoder's control flow (ep_encode.cpp) and the passes
// over the matrix it delegates: on host threads (ep_encode.cpp) or on the GPU
// (ep_encode_gpu.hip).
#pragma once

#include <cstdint>
#include <cstdlib>
#include <string>
#include <utility>
#include <vector>

#include "ep.h"
#include "ep_stream.hpp"

namespace ep {

// Symbols of every context lie in [-2048, 2047]; a histogram holds
// kContexts x kSymSpan counts, context-major, symbol + kSymBias.
constexpr int kSymBias = 2048;
constexpr int kSymSpan = 4096;

// Sampled rate estimates quantize min(n_vec, kSampleVecs) vectors, vector
// floor(k * n_vec / S) for k < S.
constexpr int64_t kSampleVecs = 65536;

// A stream in memory: from malloc, so that the C ABI hands it to the caller
// as it is (ep_free releases it), or in a caller's buffer of fixed capacity
// (the entry point that allocates nothing).
class Blob {
 public:
  Blob() = default;
  // the caller's buffer of cap bytes: alloc(n) fails for n > cap (wanted()
  // then says how many bytes the stream needs)
  Blob(uint8_t *buf, size_t cap) : p_(buf), cap_(cap), external_(true) {}
  Blob(const Blob &) = delete;
  Blob &operator=(const Blob &) = delete;
  ~Blob() {
    if (!external_) std::free(p_);
  }
  // n bytes, contents undefined; false if malloc fails or n exceeds the
  // caller's buffer
  bool alloc(size_t n) {
    wanted_ = n;
    if (external_) {
      n_ = n <= cap_ ? n : 0;
      return n <= cap_;
    }
    std::free(p_);
    p_ = (uint8_t *)std::malloc(n ? n : 1);
    n_ = p_ ? n : 0;
    return p_ != nullptr;
  }
  uint8_t *data() { return p_; }
  size_t size() const { return n_; }
  size_t wanted() const { return wanted_; }
  bool external() const { return external_; }
  // the malloc'ed stream, handed over (not for a caller's buffer)
  uint8_t *release() {
    uint8_t *p = external_ ? nullptr : p_;
    if (!external_) p_ = nullptr;
    n_ = 0;
    return p;
  }

 private:
  uint8_t *p_ = nullptr;
  size_t n_ = 0, cap_ = 0, wanted_ = 0;
  bool external_ = false;
};

struct EncodeShape {
  int dtype = 0;
  int64_t R = 0, C = 0, C8 = 0, vpr = 0, n_vec = 0, tiles = 0;
  int states = kStatesPerTile;      // rANS states per tile: kStatesPerTile or kStatesLow
  int tile_vecs = kTileVecsSmall;   // E8 vectors per tile: kTileVecsSmall or kTileVecsLarge
  int layout = kLayoutRows;         // kLayoutRows or kLayoutBlocks
  void set_tiles(int s, int tv) {
    states = s;
    tile_vecs = tv;
    tiles = tile_count(layout, R, vpr, tv);
  }
  // global vector index of local vector i of tile t, or -1 if absent
  int64_t vector_of(int64_t t, int64_t i) const { return tile_vector(layout, R, vpr, tile_vecs, t, i); }
};

// The caller's choices (ep_options); zero fields are chosen by the encoder.
struct EncodeOptions {
  double fixed_a = 0.0;      // > 0: this lattice resolution, no rate selection
  int n_states = 0;          // 0, kStatesLow or kStatesPerTile
  int tile_vecs = 0;         // 0, kTileVecsSmall or kTileVecsLarge
  int64_t sample_vecs = 0;   // 0: kSampleVecs
  uint64_t seed = 0;         // phase of the rate estimate's stride sample
  int layout = 0;            // kLayoutRows or kLayoutBlocks
};

// Normalized frequencies of each context over its symbol range
// [smin, smin + nsym); cum[c][i] is the sum of freq[c][0..i).
struct Tables {
  int16_t smin[kContexts] = {};
  uint16_t nsym[kContexts] = {};
  std::vector<uint32_t> freq[kContexts], cum[kContexts];
  int total_symbols() const {
    int t = 0;
    for (int c = 0; c < kContexts; ++c) t += nsym[c];
    return t;
  }
};

// host and device (the GPU encoder's histogram kernel) compile the helpers
// marked with this
#ifdef __HIPCC__
#define EP_HOST_DEVICE __host__ __device__
#else
#define EP_HOST_DEVICE
#endif

// Vector index of sample k of n (n <= n_vec): floor(k * n_vec / n) plus a
// phase below the stride, so every index stays inside the matrix.
EP_HOST_DEVICE inline int64_t sample_vid(int64_t n_vec, int64_t k, int64_t n, uint64_t seed) {
  const uint64_t stride = (uint64_t)n_vec / (uint64_t)n;
  return (int64_t)(((uint64_t)k * (uint64_t)n_vec) / (uint64_t)n + seed % stride);
}

// The passes over the matrix.  Every backend computes the same values by the
// same f64/f32 steps in the same order (row sums of squares in column order,
// the E8 quantizer, integer counts, integer rANS), so the stream does not
// depend on where they run.
class EncodeBackend {
 public:
  virtual ~EncodeBackend() = default;
  // the tile geometry encode_tiles uses (states per tile, vectors per tile)
  void set_geometry(int states, int tile_vecs, int layout) {
    states_ = states;
    tile_vecs_ = tile_vecs;
    layout_ = layout;
  }
  // RMS of every row (f64 sum of squares in column order).  Returns 0,
  // EP_ERR_NONFINITE if the input holds NaN or Inf, or another negative
  // ep_status.
  virtual int row_rms(std::vector<double> &rms, std::string &err) = 0;
  // Counts of (context, symbol) over vectors sample_vid(n_vec, k, S, seed),
  // k < S (S >= n_vec: every vector), quantized at row scales g.  Returns 0,
  // 1 if a coordinate leaves [-2048, 2047], or a negative ep_status.
  virtual int histogram(const std::vector<float> &g, int64_t S, uint64_t seed, std::vector<uint64_t> &hist,
                        std::string &err) = 0;
  // Every tile at row scales g with tables t, laid out as the stream stores
  // it; tile_first gets the index of each tile's first word (tiles + 1
  // entries, the last the word count).  The words stay with the backend
  // until copy_words.  Returns 0, 1 if a pair's word count does not fit its
  // count byte, or a negative ep_status.
  virtual int encode_tiles(const std::vector<float> &g, const Tables &t, std::vector<uint32_t> &tile_first,
                           std::string &err) = 0;
  // The word section of the last encode_tiles, to dst.
  virtual int copy_words(uint16_t *dst, std::string &err) = 0;
  // The container elements, row-major (rows * cols * element bytes).
  virtual int copy_input(uint8_t *dst, std::string &err) = 0;

 protected:
  int states_ = kStatesPerTile;
  int tile_vecs_ = kTileVecsSmall;
  int layout_ = kLayoutRows;
};

// The encoder on a backend: row normalization, rate selection from sampled
// estimates, the full stream at the chosen resolution (or the raw container).
// Returns an ep_status; on EP_OK or EP_WARN_RAW `blob` holds the stream,
// otherwise `err` says why.  Exactly one full encode runs for a lattice
// stream (last_encode_count).
int compress_with(EncodeBackend &be, const EncodeShape &shape, double target, const EncodeOptions &opt,
                  Blob &blob, std::string &err);

// Full encodes the last compress call on this thread ran.
int64_t last_encode_count();

// The shape of a rows x cols matrix of a container dtype; false (with err) if
// it cannot be one stream.
bool make_shape(int dtype, int64_t rows, int64_t cols, EncodeShape &shape, int &status, std::string &err);

// Lossy lattice-rANS compression of a rows x cols container matrix in host
// memory, on host threads (threads <= 0: every hardware thread).
int compress(const void *src, int dtype, int64_t rows, int64_t cols, double target, const EncodeOptions &opt,
             int threads, Blob &blob, std::string &err);

// The same for a matrix in device memory, on the GPU (work enqueued on
// `stream`, which is synchronized before the call returns).
int compress_device(const void *dev_src, int dtype, int64_t rows, int64_t cols, double target,
                    const EncodeOptions &opt, void *stream, Blob &blob, std::string &err);

// compress_device with every device buffer taken from one file-scope array
// per GPU instead of hipMalloc, and no pinned host memory: for matrices of at
// most kNoAllocMaxElements padded elements (rows x cols rounded up to 8);
// larger ones give EP_ERR_SHAPE.  Calls on one GPU take turns (a lock per
// device): the array is shared.
constexpr int64_t kNoAllocMaxElements = int64_t(1) << 22;
int compress_device_noalloc(const void *dev_src, int dtype, int64_t rows, int64_t cols, double target,
                            const EncodeOptions &opt, void *stream, Blob &blob, std::string &err);

// Per-thread error text shared by the C ABI functions.
void set_error(const std::string &msg);

}  // namespace ep
