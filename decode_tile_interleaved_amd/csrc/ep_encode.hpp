// ep_encode.hpp -- host encoder entry point (see ep_encode.cpp).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "ep.h"

namespace ep {

// Lossy lattice-rANS compression of a rows x cols container matrix.
// fixed_a > 0 skips resolution selection; threads <= 0 uses every hardware
// thread.  Returns an ep_status; on EP_OK or EP_WARN_RAW `blob` holds the
// stream, otherwise `err` says why.
int compress(const void *src, int dtype, int64_t rows, int64_t cols, double target, double fixed_a, int threads,
             std::vector<uint8_t> &blob, std::string &err);

// Per-thread error text shared by the C ABI functions.
void set_error(const std::string &msg);

}  // namespace ep
