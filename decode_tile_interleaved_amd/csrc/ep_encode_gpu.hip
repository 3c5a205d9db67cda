// ep_encode_gpu.hip -- the encoder's passes over the matrix on the GPU
// (gfx950): row sums of squares, (context, symbol) histograms for the rate
// estimates and the tables, and the interleaved rANS tiles.
//
// The EntroPack abstract (mlsanity index page) calls the encoder fast and
// its rate selection sampled: resolution selection reads sampled storage
// estimates instead of encoding the stream again and again.  The control
// flow (selection, tables, stream assembly) stays on the host
// (ep_encode.cpp); here only the passes that touch every element run, each
// computing exactly what the host threads compute, in the same f64/f32 steps:
//   * row sums of squares: one thread per row, columns in order;
//   * E8 nearest point per 8-vector (the same D8 / D8 + 1/2 rounding, parity
//     fix and tie rule), then the 7-context model; counts in LDS, added to a
//     global histogram;
//   * one wave per tile, lane q = rANS state q, walking its vectors
//     (tile_vecs / states of them) and their 8 coordinates backwards; each
//     lane writes its words into a slot of its own, and a second kernel lays
//     the tile out as the stream stores it: pair counts, length codes, the
//     bit-packed start states, then each pair's region.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "ep.h"
#include "ep_encode.hpp"
#include "ep_stream.hpp"

namespace ep {
namespace {

// ---------------------------------------------------------------------------
// device side
// ---------------------------------------------------------------------------
// a container element given by its bits, widened exactly to f64
__device__ __forceinline__ double widen_bits(uint32_t bits, int dtype) {
  switch (dtype) {
    case EP_BF16:
      return (double)__uint_as_float(bits << 16);
    case EP_FP16: {
      const int e = (int)((bits >> 10) & 31u), m = (int)(bits & 1023u);
      const double mag = e == 0 ? ldexp((double)m, -24) : e == 31 ? (m ? NAN : INFINITY) : ldexp(1024.0 + m, e - 25);
      return (bits & 0x8000u) ? -mag : mag;
    }
    case EP_FP8_E4M3FN: {
      const int e = (int)((bits >> 3) & 15u), m = (int)(bits & 7u);
      const double mag = (e == 15 && m == 7) ? NAN : e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
      return (bits & 0x80u) ? -mag : mag;
    }
    default:
      return (double)(int8_t)(uint8_t)bits;
  }
}

// element i of a container matrix, widened exactly to f64
__device__ __forceinline__ double widen_d(const void *src, int dtype, int64_t i) {
  return widen_bits(dtype <= EP_FP16 ? (uint32_t)((const uint16_t *)src)[i] : (uint32_t)((const uint8_t *)src)[i], dtype);
}

struct Shape {
  const void *src;
  int dtype;
  int64_t R, C, C8, vpr, n_vec, tiles;
};

// One wave per row: the sum of squares in column order, and whether every
// element is finite.  The lanes widen and square a chunk of the row into LDS
// (the squares are the same wherever they are computed), then lane 0 adds
// them in column order, so the f64 sum is the host's, add for add.
constexpr int kSumChunk = 2048;  // f64 squares staged per pass (16 KB of LDS)

__global__ void __launch_bounds__(64) row_sums_kernel(Shape S, double *sums, uint32_t *nonfinite) {
  __shared__ double sq[kSumChunk];
  const int64_t r = blockIdx.x;
  const uint32_t lane = threadIdx.x;
  double acc = 0.0;
  bool bad = false;
  for (int64_t c0 = 0; c0 < S.C; c0 += kSumChunk) {
    const int64_t n = S.C - c0 < kSumChunk ? S.C - c0 : kSumChunk;
    for (int64_t j = lane; j < n; j += 64) {
      const double x = widen_d(S.src, S.dtype, r * S.C + c0 + j);
      bad |= !isfinite(x);
      sq[j] = x * x;
    }
    __syncthreads();
    if (lane == 0) {
      // whole groups of 16 first, so that their LDS reads go out together
      int64_t j = 0;
      for (; j + 16 <= n; j += 16) {
        double v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = sq[j + u];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += v[u];
      }
      for (; j < n; ++j) acc += sq[j];
    }
    __syncthreads();  // the squares are read before the next chunk overwrites them
  }
  if (lane == 0) sums[r] = acc;
  if (bad) atomicOr(nonfinite, 1u);
}

// Conway & Sloane's nearest point of D8 (rint, then the coordinate with the
// largest rounding error moves if the sum is odd)
__device__ __forceinline__ void d8_round_d(const double *u, double *p) {
  double total = 0.0;
  for (int i = 0; i < 8; ++i) {
    p[i] = rint(u[i]);
    total += p[i];
  }
  if (fmod(total, 2.0) != 0.0) {
    int worst = 0;
    double err = -1.0;
    for (int i = 0; i < 8; ++i) {
      const double e = fabs(u[i] - p[i]);
      if (e > err) {
        err = e;
        worst = i;
      }
    }
    p[worst] += (u[worst] < p[worst]) ? -1.0 : 1.0;
  }
}

// v = 2y, y the E8 point nearest u (D8 or D8 + 1/2; exact ties go to D8);
// false if a coordinate leaves [-2048, 2047]
__device__ __forceinline__ bool quantize_d(const Shape &S, int64_t vid, float g, int32_t *v) {
  const int64_t r = vid / S.vpr, k = vid - r * S.vpr;
  if (g == 0.0f) {
    for (int j = 0; j < 8; ++j) v[j] = 0;
    return true;
  }
  double u[8];
  const double two_g = 2.0 * (double)g;
  for (int j = 0; j < 8; ++j) {
    const int64_t c = 8 * k + j;
    const double x = c < S.C ? widen_d(S.src, S.dtype, r * S.C + c) : 0.0;
    u[j] = x / two_g;
  }
  double a[8], b[8], sh[8];
  d8_round_d(u, a);
  for (int i = 0; i < 8; ++i) sh[i] = u[i] - 0.5;
  d8_round_d(sh, b);
  double da = 0.0, db = 0.0;
  for (int i = 0; i < 8; ++i) {
    b[i] += 0.5;
    const double ea = u[i] - a[i], eb = u[i] - b[i];
    da += ea * ea;
    db += eb * eb;
  }
  const bool use_b = db < da;
  bool ok = true;
  for (int i = 0; i < 8; ++i) {
    v[i] = (int32_t)(2.0 * (use_b ? b[i] : a[i]));
    ok &= v[i] >= kValueMin && v[i] <= kValueMax;
  }
  return ok;
}

// the 7-context model: context and symbol of each coordinate
__device__ __forceinline__ void model_d(const int32_t *v, int32_t *ctx, int32_t *sym) {
  const int32_t coset = v[0] & 1;
  int32_t zsum = (v[0] - coset) / 2;
  ctx[0] = 0;
  sym[0] = v[0];
  for (int j = 1; j < 7; ++j) {
    const int32_t z = (v[j] - coset) / 2;
    ctx[j] = 1 + coset;
    sym[j] = z;
    zsum += z;
  }
  const int32_t par = zsum & 1;
  ctx[7] = 3 + 2 * coset + par;
  sym[7] = ((v[7] - coset) / 2 - par) / 2;
}

// LDS histogram bins: context F over [-2048, 2047], C_b over [-1024, 1023],
// E_{b,p} over [-512, 511] (the ranges the value range allows)
constexpr int kBinsF = 4096, kBinsC = 2048, kBinsE = 1024;
constexpr int kLdsBins = kBinsF + 2 * kBinsC + 4 * kBinsE;  // 12288 (48 KB)
__device__ __forceinline__ int lds_bin(int c, int sym) {
  return c == 0 ? sym + 2048 : c <= 2 ? kBinsF + (c - 1) * kBinsC + sym + 1024 : kBinsF + 2 * kBinsC + (c - 3) * kBinsE + sym + 512;
}
__device__ __forceinline__ void bin_symbol(int b, int &c, int &sym) {
  if (b < kBinsF) {
    c = 0;
    sym = b - 2048;
  } else if (b < kBinsF + 2 * kBinsC) {
    c = 1 + (b - kBinsF) / kBinsC;
    sym = (b - kBinsF) % kBinsC - 1024;
  } else {
    c = 3 + (b - kBinsF - 2 * kBinsC) / kBinsE;
    sym = (b - kBinsF - 2 * kBinsC) % kBinsE - 512;
  }
}

// counts of (context, symbol) over vectors sample_vid(n_vec, k, S, seed),
// k < S (S >= n_vec: every vector); hist is kContexts x kSymSpan u64
__global__ void __launch_bounds__(256) histogram_kernel(Shape S, const float *g, int64_t nsamp, uint64_t seed,
                                                        uint64_t *hist, uint32_t *overflow) {
  __shared__ uint32_t bins[kLdsBins];
  for (int b = threadIdx.x; b < kLdsBins; b += blockDim.x) bins[b] = 0u;
  __syncthreads();
  const bool all = nsamp >= S.n_vec;
  const int64_t n = all ? S.n_vec : nsamp;
  bool bad = false;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
    const int64_t vid = all ? k : sample_vid(S.n_vec, k, nsamp, seed);
    int32_t v[8], ctx[8], sym[8];
    if (!quantize_d(S, vid, g[vid / S.vpr], v)) {
      bad = true;
      continue;
    }
    model_d(v, ctx, sym);
    for (int j = 0; j < 8; ++j) atomicAdd(&bins[lds_bin(ctx[j], sym[j])], 1u);
  }
  if (bad) atomicOr(overflow, 1u);
  __syncthreads();
  for (int b = threadIdx.x; b < kLdsBins; b += blockDim.x) {
    const uint32_t cnt = bins[b];
    if (cnt) {
      int c, sym;
      bin_symbol(b, c, sym);
      atomicAdd((unsigned long long *)&hist[(size_t)c * kSymSpan + sym + kSymBias], (unsigned long long)cnt);
    }
  }
}

// Tables on the device: per context the symbol range and, per symbol,
// frequency | cumulative << 16.
struct DevTables {
  int32_t smin[kContexts];
  int32_t nsym[kContexts];
  uint32_t base[kContexts];  // index of each context's first entry in fc
};

// words a state's slot holds: at most one per symbol, 8 per vector
__host__ __device__ constexpr int words_per_state(int states, int tile_vecs) { return 8 * (tile_vecs / states); }

// One wave per tile, lane q = state q of ns: its vectors q, q + ns, ...
// quantized again at the same scales, their symbols encoded backwards (last
// vector first, coordinate 7 down to 0) from x = 2^11.  Words go to the
// lane's slot in emission order; the count and the final state are kept.
__global__ void __launch_bounds__(64) encode_tiles_kernel(Shape S, int ns, int tv, const float *g, DevTables T,
                                                          const uint32_t *fc, uint16_t *slots, uint16_t *counts,
                                                          uint32_t *states, uint32_t *fault) {
  const int64_t tile = blockIdx.x;
  const int q = threadIdx.x;
  const int64_t first = tile * tv;
  const int n = (int)min((int64_t)tv, S.n_vec - first);
  const int wps = words_per_state(ns, tv);
  uint16_t *slot = slots + ((size_t)tile * ns + q) * wps;
  uint32_t x = kStateLow;
  int emitted = 0;
  bool bad = false;
  for (int s = tv / ns - 1; s >= 0; --s) {
    const int i = s * ns + q;
    if (i >= n) continue;
    const int64_t vid = first + i;
    int32_t v[8], ctx[8], sym[8];
    bad |= !quantize_d(S, vid, g[vid / S.vpr], v);
    model_d(v, ctx, sym);
    for (int j = 7; j >= 0; --j) {
      const int c = ctx[j];
      const int idx = sym[j] - T.smin[c];
      if (idx < 0 || idx >= T.nsym[c]) {  // a symbol the tables do not hold: the passes disagree
        bad = true;
        continue;
      }
      const uint32_t e = fc[T.base[c] + (uint32_t)idx];
      const uint32_t f = e & 0xffffu, cum = e >> 16;
      if (f == 0u) {
        bad = true;
        continue;
      }
      if ((uint64_t)x >= ((uint64_t)f << (kStateTop - kProbBits))) {
        if (emitted < wps) slot[emitted] = (uint16_t)x;
        ++emitted;
        x >>= 16;
      }
      x = (x / f) * kProbTotal + x % f + cum;
    }
  }
  if (emitted > wps) bad = true;
  counts[tile * ns + q] = (uint16_t)min(emitted, wps);
  states[tile * ns + q] = x;
  if (bad) atomicOr(fault, 1u);
}

// inclusive prefix sum over a wave
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, int lane) {
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// One wave per tile, lane q = state q of ns (lanes past ns hold nothing):
// the tile at its first word as the stream stores it.  The pair counts fit a
// byte each (the host checked).  The start bits are OR-ed together in LDS
// (a state's bits straddle at most two dwords), then written out as words.
__global__ void __launch_bounds__(64) lay_out_kernel(int ns, int tv, const uint16_t *slots, const uint16_t *counts,
                                                     const uint32_t *states, const uint32_t *tile_first,
                                                     uint16_t *words) {
  __shared__ uint32_t bitbuf[kStatesPerTile];  // 64 states x at most 26 bits < 64 dwords
  const int64_t tile = blockIdx.x;
  const int q = threadIdx.x;
  const bool mine = q < ns;
  const uint32_t cnt = mine ? counts[tile * ns + q] : 0u;
  const uint32_t x = mine ? states[tile * ns + q] : 0u;
  const uint32_t nb = mine ? 31u - (uint32_t)__builtin_clz(x) : 0u;  // bits below the leading one: W - 1
  const uint32_t words_before = wave_scan(cnt, q) - cnt;
  const uint32_t bits_incl = wave_scan(nb, q), bits_before = bits_incl - nb;
  const uint32_t total_bits = __shfl(bits_incl, 63, 64);
  uint16_t *w = words + tile_first[tile];
  // pair counts (two pairs to a word) and length codes (four to a word)
  const uint32_t c1 = __shfl_down(cnt, 1, 64), c2 = __shfl_down(cnt, 2, 64), c3 = __shfl_down(cnt, 3, 64);
  const uint32_t n1 = __shfl_down(nb, 1, 64), n2 = __shfl_down(nb, 2, 64), n3 = __shfl_down(nb, 3, 64);
  if (mine && (q & 3) == 0) {
    w[q / 4] = (uint16_t)((cnt + c1) | (c2 + c3) << 8);
    w[ns / 4 + q / 4] = (uint16_t)((nb - 11u) | (n1 - 11u) << 4 | (n2 - 11u) << 8 | (n3 - 11u) << 12);
  }
  bitbuf[q] = 0u;
  __syncthreads();
  if (mine) {
    const uint64_t v = (uint64_t)(x & ((1u << nb) - 1u)) << (bits_before & 31u);
    atomicOr(&bitbuf[bits_before >> 5], (uint32_t)v);
    if (v >> 32) atomicOr(&bitbuf[(bits_before >> 5) + 1u], (uint32_t)(v >> 32));
  }
  __syncthreads();
  const uint32_t nbw = (total_bits + 15u) / 16u;
  for (uint32_t k = (uint32_t)q; k < nbw; k += 64u) w[ns / 2 + k] = (uint16_t)(bitbuf[k / 2] >> (16u * (k & 1u)));
  // regions: state 2k's words in consumption order (the reverse of emission),
  // then state 2k+1's in emission order
  if (mine) {
    const uint16_t *slot = slots + ((size_t)tile * ns + q) * words_per_state(ns, tv);
    uint16_t *mine_w = w + ns / 2 + nbw + words_before;
    if ((q & 1) == 0)
      for (uint32_t k = 0; k < cnt; ++k) mine_w[k] = slot[cnt - 1u - k];
    else
      for (uint32_t k = 0; k < cnt; ++k) mine_w[k] = slot[k];
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// pinned host memory, kept for the encoder's lifetime
struct PinnedBuf {
  void *p = nullptr;
  size_t n = 0;
  ~PinnedBuf() {
    if (p) (void)hipHostFree(p);
  }
  bool reserve(size_t bytes) {
    if (bytes <= n && p) return true;
    if (p) (void)hipHostFree(p);
    p = nullptr;
    n = 0;
    if (hipHostMalloc(&p, bytes, hipHostMallocDefault) != hipSuccess) {
      p = nullptr;
      return false;
    }
    n = bytes;
    return true;
  }
};

// A device buffer: from hipMalloc (grown on demand, freed with the
// backend), or a fixed piece of the no-alloc scratch array (never grown).
template <class T>
struct DevBuf {
  T *p = nullptr;
  size_t n = 0;
  bool owned = true;
  ~DevBuf() {
    if (p && owned) (void)hipFree(p);
  }
  void attach(T *q, size_t count) {
    p = q;
    n = count;
    owned = false;
  }
  bool reserve(size_t count) {
    if (count <= n && p) return true;
    if (!owned) return false;  // a scratch piece is sized for the largest use up front
    if (p) (void)hipFree(p);
    p = nullptr;
    n = 0;
    if (hipMalloc(&p, sizeof(T) * (count ? count : 1)) != hipSuccess) {
      p = nullptr;
      return false;
    }
    n = count;
    return true;
  }
};

// Carves 256-byte aligned pieces off a device region, front to back.
struct Arena {
  uint8_t *base = nullptr;
  size_t cap = 0, used = 0;
  template <class T>
  bool take(DevBuf<T> &b, size_t count) {
    const size_t start = (used + 255) & ~size_t(255), bytes = sizeof(T) * (count ? count : 1);
    if (start > cap || bytes > cap - start) return false;
    b.attach(reinterpret_cast<T *>(base + start), count);
    used = start + bytes;
    return true;
  }
};

class GpuBackend final : public EncodeBackend {
 public:
  GpuBackend(const void *dev_src, const EncodeShape &S, hipStream_t stream) : es_(S), stream_(stream) {
    S_ = Shape{dev_src, S.dtype, S.R, S.C, S.C8, S.vpr, S.n_vec, S.tiles};
  }

  // Every buffer from `arena`, at the most any geometry of this shape needs
  // (tiles of 512 vectors with 64 states); false if the arena is too small.
  bool use_arena(Arena &arena) {
    const size_t tiles = (size_t)((es_.n_vec + kTileVecsSmall - 1) / kTileVecsSmall);
    const size_t states = tiles * kStatesPerTile;
    // one word slot per symbol of every whole tile: 8 tile_vecs words per
    // tile, which whole 1024-vector tiles bound for either tile size
    const size_t slot_words = (size_t)((es_.n_vec + kTileVecsLarge - 1) / kTileVecsLarge) * 8 * kTileVecsLarge;
    // a tile's words: its states' words plus pair counts, codes and start bits
    const size_t words = slot_words + tiles * (kStatesPerTile / 2 + (kStatesPerTile * 26 + 15) / 16);
    host_copies_ = true;
    return arena.take(sums_, (size_t)es_.R) && arena.take(g_, (size_t)es_.R) &&
           arena.take(hist_, (size_t)kContexts * kSymSpan) && arena.take(flag_, 1) &&
           arena.take(fc_, (size_t)kContexts * kSymSpan) && arena.take(slots_, slot_words) &&
           arena.take(counts_, states) && arena.take(dstates_, states) && arena.take(first_, tiles + 1) &&
           arena.take(words_, words);
  }

  int row_rms(std::vector<double> &rms, std::string &err) override {
    if (!sums_.reserve((size_t)es_.R) || !flag_.reserve(1)) return nomem(err);
    if (hipMemsetAsync(flag_.p, 0, sizeof(uint32_t), stream_) != hipSuccess) return device(err, "hipMemsetAsync");
    hipLaunchKernelGGL(row_sums_kernel, dim3((unsigned)es_.R), dim3(64), 0, stream_, S_, sums_.p, flag_.p);
    if (hipGetLastError() != hipSuccess) return device(err, "row sums launch");
    std::vector<double> sums((size_t)es_.R);
    uint32_t bad = 0;
    if (hipMemcpyAsync(sums.data(), sums_.p, 8 * (size_t)es_.R, hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipMemcpyAsync(&bad, flag_.p, 4, hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipStreamSynchronize(stream_) != hipSuccess)
      return device(err, "row sums");
    if (bad) {
      err = "input holds NaN or Inf";
      return EP_ERR_NONFINITE;
    }
    rms.resize((size_t)es_.R);
    for (int64_t r = 0; r < es_.R; ++r) rms[(size_t)r] = std::sqrt(sums[(size_t)r] / (double)es_.C);
    return 0;
  }

  int histogram(const std::vector<float> &g, int64_t nsamp, uint64_t seed, std::vector<uint64_t> &hist,
                std::string &err) override {
    if (const int rc = upload_scales(g, err); rc != 0) return rc;
    if (!hist_.reserve((size_t)kContexts * kSymSpan) || !flag_.reserve(1)) return nomem(err);
    if (hipMemsetAsync(hist_.p, 0, 8 * hist_.n, stream_) != hipSuccess ||
        hipMemsetAsync(flag_.p, 0, sizeof(uint32_t), stream_) != hipSuccess)
      return device(err, "hipMemsetAsync");
    const int64_t n = nsamp >= es_.n_vec ? es_.n_vec : nsamp;
    const unsigned blocks = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 4096));
    hipLaunchKernelGGL(histogram_kernel, dim3(blocks), dim3(256), 0, stream_, S_, g_.p, nsamp, seed, hist_.p,
                       flag_.p);
    if (hipGetLastError() != hipSuccess) return device(err, "histogram launch");
    // through pinned host memory (each rate probe copies the whole
    // histogram), or straight into pageable memory where nothing may be
    // allocated on the device side
    const size_t nh = (size_t)kContexts * kSymSpan;
    uint64_t *ph;
    uint32_t *pf;
    if (host_copies_) {
      hist.resize(nh);
      ph = hist.data();
      pf = &flag_host_;
    } else {
      if (!pin_.reserve(8 * nh + 8)) return nomem(err);
      ph = static_cast<uint64_t *>(pin_.p);
      pf = reinterpret_cast<uint32_t *>(ph + nh);
    }
    if (hipMemcpyAsync(ph, hist_.p, 8 * nh, hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipMemcpyAsync(pf, flag_.p, 4, hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipStreamSynchronize(stream_) != hipSuccess)
      return device(err, "histogram");
    if (host_copies_) return *pf ? 1 : 0;
    hist.assign(ph, ph + nh);
    return *pf ? 1 : 0;
  }

  int encode_tiles(const std::vector<float> &g, const Tables &tb, std::vector<uint32_t> &tile_first,
                   std::string &err) override {
    if (const int rc = upload_scales(g, err); rc != 0) return rc;
    // tables: frequency | cumulative << 16 per symbol, contexts one after another
    DevTables T{};
    std::vector<uint32_t> fc;
    for (int c = 0; c < kContexts; ++c) {
      T.smin[c] = tb.smin[c];
      T.nsym[c] = tb.nsym[c];
      T.base[c] = (uint32_t)fc.size();
      for (int i = 0; i < tb.nsym[c]; ++i) fc.push_back(tb.freq[c][(size_t)i] | tb.cum[c][(size_t)i] << 16);
    }
    const int sp = states_, tv = tile_vecs_;  // states and vectors per tile
    const size_t nt = (size_t)((es_.n_vec + tv - 1) / tv), ns = nt * (size_t)sp;
    if (!fc_.reserve(fc.size()) || !slots_.reserve(ns * (size_t)words_per_state(sp, tv)) || !counts_.reserve(ns) ||
        !dstates_.reserve(ns) || !first_.reserve(nt + 1) || !flag_.reserve(1))
      return nomem(err);
    if (hipMemcpyAsync(fc_.p, fc.data(), 4 * fc.size(), hipMemcpyHostToDevice, stream_) != hipSuccess ||
        hipMemsetAsync(flag_.p, 0, sizeof(uint32_t), stream_) != hipSuccess)
      return device(err, "table upload");
    hipLaunchKernelGGL(encode_tiles_kernel, dim3((unsigned)nt), dim3(sp), 0, stream_, S_, sp, tv, g_.p, T, fc_.p,
                       slots_.p, counts_.p, dstates_.p, flag_.p);
    if (hipGetLastError() != hipSuccess) return device(err, "tile encode launch");
    std::vector<uint16_t> counts(ns);
    std::vector<uint32_t> states(ns);
    uint32_t fault = 0;
    if (hipMemcpyAsync(counts.data(), counts_.p, 2 * ns, hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipMemcpyAsync(states.data(), dstates_.p, 4 * ns, hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipMemcpyAsync(&fault, flag_.p, 4, hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipStreamSynchronize(stream_) != hipSuccess)
      return device(err, "tile encode");
    if (fault) {
      err = "the tile encoder met a symbol outside the tables";
      return EP_ERR_DEVICE;
    }
    // each tile's first word: pair counts and length codes, the start bits
    // on whole words, the states' words
    tile_first.resize(nt + 1);
    uint64_t w = 0;
    bool overflow = false;
    for (size_t t = 0; t < nt; ++t) {
      tile_first[t] = (uint32_t)w;
      uint64_t bits = 0;
      for (int q = 0; q < sp; ++q) {
        bits += 31u - (uint32_t)__builtin_clz(states[t * sp + q]);
        w += counts[t * sp + q];
        if (q & 1) overflow |= counts[t * sp + q - 1] + counts[t * sp + q] > 255;
      }
      w += (uint64_t)sp / 2 + (bits + 15) / 16;
      if (w > 0xffffffffull) {
        err = "stream too large for 32-bit tile offsets";
        return EP_ERR_SHAPE;
      }
    }
    tile_first[nt] = (uint32_t)w;
    if (overflow) return 1;  // a count byte cannot hold a pair's words
    if (!words_.reserve((size_t)w)) return nomem(err);
    if (hipMemcpyAsync(first_.p, tile_first.data(), 4 * (nt + 1), hipMemcpyHostToDevice, stream_) != hipSuccess)
      return device(err, "tile offsets upload");
    hipLaunchKernelGGL(lay_out_kernel, dim3((unsigned)nt), dim3(64), 0, stream_, sp, tv, slots_.p, counts_.p,
                       dstates_.p, first_.p, words_.p);
    if (hipGetLastError() != hipSuccess) return device(err, "layout launch");
    n_words_ = (size_t)w;
    return 0;
  }

  int copy_words(uint16_t *dst, std::string &err) override {
    if (hipMemcpyAsync(dst, words_.p, 2 * n_words_, hipMemcpyDeviceToHost, stream_) != hipSuccess ||
        hipStreamSynchronize(stream_) != hipSuccess)
      return device(err, "word copy");
    return 0;
  }

  int copy_input(uint8_t *dst, std::string &err) override {
    if (hipMemcpyAsync(dst, S_.src, (size_t)es_.R * (size_t)es_.C * elem_bytes(es_.dtype), hipMemcpyDeviceToHost,
                       stream_) != hipSuccess ||
        hipStreamSynchronize(stream_) != hipSuccess)
      return device(err, "input copy");
    return 0;
  }

 private:
  int upload_scales(const std::vector<float> &g, std::string &err) {
    if (!g_.reserve(g.size())) return nomem(err);
    if (hipMemcpyAsync(g_.p, g.data(), 4 * g.size(), hipMemcpyHostToDevice, stream_) != hipSuccess)
      return device(err, "scale upload");
    return 0;
  }
  static int nomem(std::string &err) {
    err = "device allocation failed";
    return EP_ERR_NOMEM;
  }
  static int device(std::string &err, const char *what) {
    err = std::string(what) + " failed: " + hipGetErrorString(hipGetLastError());
    return EP_ERR_DEVICE;
  }

  EncodeShape es_;
  Shape S_;
  hipStream_t stream_;
  DevBuf<double> sums_;
  DevBuf<float> g_;
  DevBuf<uint64_t> hist_;
  DevBuf<uint32_t> flag_, fc_, dstates_, first_;
  DevBuf<uint16_t> slots_, words_;
  DevBuf<uint16_t> counts_;
  PinnedBuf pin_;
  size_t n_words_ = 0;
  bool host_copies_ = false;  // scratch mode: histograms go to pageable memory
  uint32_t flag_host_ = 0;
};

// ---------------------------------------------------------------------------
// The entry point that allocates nothing takes its device buffers from one
// array per GPU.  Its size covers the largest shape allowed,
// kNoAllocMaxElements padded elements (rows x cols rounded up to 8): at most
// 2^19 rows (12 bytes each: sums and scales), 2^19 vectors in whole tiles
// (16 bytes of word slots and as much of stream words each), 1024 tiles of 64 states (6 bytes
// per state, 136 header words per tile, 4 bytes of offset), the histogram
// and tables (12 bytes per context symbol), and the pieces' alignment.
// ---------------------------------------------------------------------------
constexpr size_t kScratchRows = (size_t)(kNoAllocMaxElements / 8);
constexpr size_t kScratchVecs = (size_t)(kNoAllocMaxElements / 8);
constexpr size_t kScratchTiles = kScratchVecs / kTileVecsSmall;
constexpr size_t kScratchBytes = 12 * kScratchRows + 16 * kScratchVecs +
                                 2 * (8 * kScratchVecs + kScratchTiles * (kStatesPerTile / 2 + (kStatesPerTile * 26 + 15) / 16)) +
                                 6 * kScratchTiles * kStatesPerTile + 4 * (kScratchTiles + 1) +
                                 12 * (size_t)kContexts * kSymSpan + 4 + 16 * 256;

// The array (about 24 MB on each GPU the library runs on, held until the
// process ends).  Host code never passes its name to a kernel: that is a
// host-side stand-in, not a device address.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct DeviceScratch {
  void *ptr = nullptr;  // the array's address on this device
  std::mutex call;      // calls on this device take turns: they share the array
};

// The current device's array, its address looked up once per device with
// that device current.  nullptr (with err) if the lookup fails.
DeviceScratch *device_scratch(std::string &err) {
  static std::mutex mu;
  static std::vector<std::unique_ptr<DeviceScratch>> per_device;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    err = "hipGetDevice failed";
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(mu);
  if ((int)per_device.size() <= dev) per_device.resize((size_t)dev + 1);
  if (!per_device[(size_t)dev]) per_device[(size_t)dev] = std::make_unique<DeviceScratch>();
  DeviceScratch &d = *per_device[(size_t)dev];
  if (!d.ptr) {
    void *p = nullptr;
    const hipError_t rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (rc != hipSuccess || !p) {
      err = std::string("hipGetSymbolAddress of the scratch array failed: ") + hipGetErrorString(rc);
      return nullptr;
    }
    d.ptr = p;
  }
  return &d;
}

}  // namespace

int compress_device(const void *dev_src, int dtype, int64_t rows, int64_t cols, double target,
                    const EncodeOptions &opt, void *stream, Blob &blob, std::string &err) {
  EncodeShape S;
  int status = 0;
  if (!make_shape(dtype, rows, cols, S, status, err)) return status;
  if (!dev_src) {
    err = "null input";
    return EP_ERR_ARG;
  }
  if (opt.layout != kLayoutRows) {  // its tile passes walk row-major tiles only
    err = "the GPU encoder writes row-major tiles; the blocks layout is encoded on the host";
    return EP_ERR_ARG;
  }
  GpuBackend be(dev_src, S, reinterpret_cast<hipStream_t>(stream));
  return compress_with(be, S, target, opt, blob, err);
}

int compress_device_noalloc(const void *dev_src, int dtype, int64_t rows, int64_t cols, double target,
                            const EncodeOptions &opt, void *stream, Blob &blob, std::string &err) {
  EncodeShape S;
  int status = 0;
  if (!make_shape(dtype, rows, cols, S, status, err)) return status;
  if (!dev_src) {
    err = "null input";
    return EP_ERR_ARG;
  }
  if (opt.layout != kLayoutRows) {  // its tile passes walk row-major tiles only
    err = "the GPU encoder writes row-major tiles; the blocks layout is encoded on the host";
    return EP_ERR_ARG;
  }
  if (S.R * S.C8 > kNoAllocMaxElements) {
    err = "matrix too large for the scratch array: at most " + std::to_string(kNoAllocMaxElements) +
          " elements (rows x cols rounded up to 8)";
    return EP_ERR_SHAPE;
  }
  DeviceScratch *ds = device_scratch(err);
  if (!ds) return EP_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(ds->call);
  Arena arena{static_cast<uint8_t *>(ds->ptr), kScratchBytes, 0};
  GpuBackend be(dev_src, S, reinterpret_cast<hipStream_t>(stream));
  if (!be.use_arena(arena)) {
    err = "the scratch array cannot hold this shape's buffers";
    return EP_ERR_SHAPE;
  }
  return compress_with(be, S, target, opt, blob, err);
}

}  // namespace ep
