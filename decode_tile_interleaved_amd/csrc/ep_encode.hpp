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

// A stream in memory from malloc, so that the C ABI hands it to the caller
// as it is (ep_free releases it).
class Blob {
 public:
  Blob() = default;
  Blob(const Blob &) = delete;
  Blob &operator=(const Blob &) = delete;
  ~Blob() { std::free(p_); }
  // n bytes, contents undefined; false if malloc fails
  bool alloc(size_t n) {
    std::free(p_);
    p_ = (uint8_t *)std::malloc(n ? n : 1);
    n_ = p_ ? n : 0;
    return p_ != nullptr;
  }
  uint8_t *data() { return p_; }
  size_t size() const { return n_; }
  void swap(Blob &o) {
    std::swap(p_, o.p_);
    std::swap(n_, o.n_);
  }
  uint8_t *release() {
    uint8_t *p = p_;
    p_ = nullptr;
    n_ = 0;
    return p;
  }

 private:
  uint8_t *p_ = nullptr;
  size_t n_ = 0;
};

struct EncodeShape {
  int dtype = 0;
  int64_t R = 0, C = 0, C8 = 0, vpr = 0, n_vec = 0, tiles = 0;
  int states = kStatesPerTile;  // rANS states per tile: kStatesPerTile or kStatesLow
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

// The passes over the matrix.  Every backend computes the same values by the
// same f64/f32 steps in the same order (row sums of squares in column order,
// the E8 quantizer, integer counts, integer rANS), so the stream does not
// depend on where they run.
class EncodeBackend {
 public:
  virtual ~EncodeBackend() = default;
  // rANS states per tile for encode_tiles (kStatesPerTile or kStatesLow)
  void set_states(int states) { states_ = states; }
  // RMS of every row (f64 sum of squares in column order).  Returns 0,
  // EP_ERR_NONFINITE if the input holds NaN or Inf, or another negative
  // ep_status.
  virtual int row_rms(std::vector<double> &rms, std::string &err) = 0;
  // Counts of (context, symbol) over vectors floor(k * n_vec / S), k < S
  // (S >= n_vec: every vector), quantized at row scales g.  Returns 0, 1 if a
  // coordinate leaves [-2048, 2047], or a negative ep_status.
  virtual int histogram(const std::vector<float> &g, int64_t S, std::vector<uint64_t> &hist, std::string &err) = 0;
  // Every tile at row scales g with tables t: start states (set_states
  // per tile) and the index of each tile's first word (tiles + 1 entries;
  // the last is the word count).  The words stay with the backend until
  // copy_words.  Returns 0, 1 if a state's word count does not fit its count
  // byte (possible with kStatesLow only), or a negative ep_status.
  virtual int encode_tiles(const std::vector<float> &g, const Tables &t, std::vector<uint32_t> &states,
                           std::vector<uint32_t> &tile_first, std::string &err) = 0;
  // The word section of the last encode_tiles, to dst.
  virtual int copy_words(uint16_t *dst, std::string &err) = 0;
  // The container elements, row-major (rows * cols * element bytes).
  virtual int copy_input(uint8_t *dst, std::string &err) = 0;

 protected:
  int states_ = kStatesPerTile;
};

// The encoder on a backend: row normalization, rate selection from sampled
// estimates, the full stream at the chosen resolution (or the raw container).
// fixed_a > 0 skips rate selection.  Returns an ep_status; on EP_OK or
// EP_WARN_RAW `blob` holds the stream, otherwise `err` says why.
int compress_with(EncodeBackend &be, const EncodeShape &shape, double target, double fixed_a,
                  Blob &blob, std::string &err);

// The shape of a rows x cols matrix of a container dtype; false (with err) if
// it cannot be one stream.
bool make_shape(int dtype, int64_t rows, int64_t cols, EncodeShape &shape, int &status, std::string &err);

// Lossy lattice-rANS compression of a rows x cols container matrix in host
// memory, on host threads (threads <= 0: every hardware thread).
int compress(const void *src, int dtype, int64_t rows, int64_t cols, double target, double fixed_a, int threads,
             Blob &blob, std::string &err);

// The same for a matrix in device memory, on the GPU (work enqueued on
// `stream`, which is synchronized before the call returns).
int compress_device(const void *dev_src, int dtype, int64_t rows, int64_t cols, double target, double fixed_a,
                    void *stream, Blob &blob, std::string &err);

// Per-thread error text shared by the C ABI functions.
void set_error(const std::string &msg);

}  // namespace ep
