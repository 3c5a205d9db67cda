// ep_capi.cpp -- host half of the C ABI: compression, stream facts, errors.
// The GPU entry points (ep_decompress, ep_decode_symbols) live in ep_decode.hip.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "ep.h"
#include "ep_encode.hpp"
#include "ep_stream.hpp"

namespace ep {
static thread_local std::string g_error;
void set_error(const std::string &msg) { g_error = msg; }
}  // namespace ep

namespace {

// ep_options to EncodeOptions; 0 or EP_ERR_ARG (with the error text set)
int read_options(const struct ep_options *opt, ep::EncodeOptions &eo, int &threads) {
  if (!opt) return 0;
  for (int r : opt->reserved)
    if (r != 0) {
      ep::set_error("ep_options.reserved must be zero");
      return EP_ERR_ARG;
    }
  eo.fixed_a = opt->fixed_scale;
  eo.n_states = opt->n_states;
  eo.tile_vecs = opt->tile_vecs;
  eo.sample_vecs = opt->sample_vecs;
  eo.seed = opt->seed;
  eo.layout = opt->layout;
  threads = opt->n_threads;
  if (!(eo.fixed_a >= 0.0) || std::isinf(eo.fixed_a)) {
    ep::set_error("fixed_scale must be finite and >= 0");
    return EP_ERR_ARG;
  }
  if ((eo.n_states != 0 && eo.n_states != 16 && eo.n_states != 64) ||
      (eo.tile_vecs != 0 && eo.tile_vecs != 512 && eo.tile_vecs != 1024) || eo.sample_vecs < 0) {
    ep::set_error("n_states must be 0, 16 or 64, tile_vecs 0, 512 or 1024, sample_vecs >= 0");
    return EP_ERR_ARG;
  }
  if (eo.layout != EP_LAYOUT_ROWS && eo.layout != EP_LAYOUT_BLOCKS) {
    ep::set_error("layout must be EP_LAYOUT_ROWS or EP_LAYOUT_BLOCKS");
    return EP_ERR_ARG;
  }
  return 0;
}

// option checks, the call, and the copy of the stream into malloc'ed memory
template <class F>
int compress_entry(const struct ep_options *opt, uint8_t **blob_out, size_t *nbytes_out, F &&run) {
  ep::set_error("");
  if (!blob_out || !nbytes_out) {
    ep::set_error("null output pointer");
    return EP_ERR_ARG;
  }
  ep::EncodeOptions eo;
  int threads = 0;
  if (const int rc = read_options(opt, eo, threads); rc != 0) return rc;
  ep::Blob blob;
  std::string err;
  int rc;
  try {
    rc = run(eo, threads, blob, err);
  } catch (const std::bad_alloc &) {
    ep::set_error("host allocation failed");
    return EP_ERR_NOMEM;
  }
  if (rc < 0) {
    ep::set_error(err);
    return rc;
  }
  *nbytes_out = blob.size();
  *blob_out = blob.release();  // malloc'ed: ep_free releases it
  if (rc > 0) ep::set_error(err);
  return rc;
}

}  // namespace

extern "C" {

int ep_compress_ex(const void *host_src, int dtype, int64_t rows, int64_t cols, double target_bpp,
                   const struct ep_options *opt, uint8_t **blob_out, size_t *nbytes_out) {
  return compress_entry(opt, blob_out, nbytes_out, [&](const ep::EncodeOptions &eo, int threads, ep::Blob &blob,
                                                        std::string &err) {
    return ep::compress(host_src, dtype, rows, cols, target_bpp, eo, threads, blob, err);
  });
}

int ep_compress_device(const void *dev_src, int dtype, int64_t rows, int64_t cols, double target_bpp,
                       const struct ep_options *opt, void *hip_stream, uint8_t **blob_out, size_t *nbytes_out) {
  return compress_entry(opt, blob_out, nbytes_out, [&](const ep::EncodeOptions &eo, int, ep::Blob &blob,
                                                        std::string &err) {
    return ep::compress_device(dev_src, dtype, rows, cols, target_bpp, eo, hip_stream, blob, err);
  });
}

int ep_compress_device_noalloc(const void *dev_src, int dtype, int64_t rows, int64_t cols, double target_bpp,
                               const struct ep_options *opt, void *hip_stream, uint8_t *out, size_t capacity,
                               size_t *nbytes_out) {
  ep::set_error("");
  if (!out || !nbytes_out) {
    ep::set_error("null output pointer");
    return EP_ERR_ARG;
  }
  ep::EncodeOptions eo;
  int threads = 0;
  if (const int rc = read_options(opt, eo, threads); rc != 0) return rc;
  ep::Blob blob(out, capacity);
  std::string err;
  int rc;
  try {
    rc = ep::compress_device_noalloc(dev_src, dtype, rows, cols, target_bpp, eo, hip_stream, blob, err);
  } catch (const std::bad_alloc &) {
    ep::set_error("host allocation failed");
    return EP_ERR_NOMEM;
  }
  if (rc == EP_ERR_NOMEM && blob.wanted() > capacity) {
    *nbytes_out = blob.wanted();
    ep::set_error("output buffer of " + std::to_string(capacity) + " bytes is too small: the stream needs " +
                  std::to_string(blob.wanted()));
    return EP_ERR_ARG;
  }
  if (rc < 0) {
    ep::set_error(err);
    return rc;
  }
  *nbytes_out = blob.size();
  if (rc > 0) ep::set_error(err);
  return rc;
}

int ep_compress(const void *host_src, int dtype, int64_t rows, int64_t cols, double target_bpp, uint8_t **blob_out,
                size_t *nbytes_out) {
  return ep_compress_ex(host_src, dtype, rows, cols, target_bpp, nullptr, blob_out, nbytes_out);
}

void ep_free(uint8_t *blob) { std::free(blob); }

int ep_blob_info(const uint8_t *blob, size_t nbytes, struct ep_info *info) {
  ep::set_error("");
  ep::StreamView s;
  std::string e = ep::parse_stream(blob, nbytes, s);
  if (!e.empty()) {
    ep::set_error(e);
    return EP_ERR_FORMAT;
  }
  if (!info) {
    ep::set_error("null info pointer");
    return EP_ERR_ARG;
  }
  info->rows = s.rows;
  info->cols = s.cols;
  info->dtype = s.dtype;
  info->method = s.method;
  info->n_states = s.states;
  info->tile_vecs = s.tile_vecs;
  info->prob_bits = s.prob_bits;
  info->n_tiles = s.tiles;
  info->n_words = (int64_t)s.n_words;
  info->scale_a = s.scale_a;
  info->target_bpp = s.target;
  info->layout = s.layout;
  return EP_OK;
}

double ep_actual_bpp(const uint8_t *blob, size_t nbytes) {
  ep::StreamView s;
  std::string e = ep::parse_stream(blob, nbytes, s);
  if (!e.empty()) {
    ep::set_error(e);
    return NAN;
  }
  return 8.0 * (double)nbytes / ((double)s.rows * (double)s.cols);
}

int64_t ep_storage_nbytes(const uint8_t *blob, size_t nbytes, int include_header) {
  ep::StreamView s;
  std::string e = ep::parse_stream(blob, nbytes, s);
  if (!e.empty()) {
    ep::set_error(e);
    return -1;
  }
  return include_header ? (int64_t)nbytes : (int64_t)nbytes - (int64_t)ep::kHeaderBytes;
}

const char *ep_last_error(void) { return ep::g_error.c_str(); }

int64_t ep_last_encode_count(void) { return ep::last_encode_count(); }

}  // extern "C"
