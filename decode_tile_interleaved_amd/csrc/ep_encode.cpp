// ep_encode.cpp -- host encoder: row normalization, E8 quantization, the
// conditional model, sampled resolution selection and interleaved rANS tiles.
//
// Method: "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at
// Arbitrary Bitrates" (arXiv abstract, mlsanity index page).  The pages give
// the steps, not their internals; the choices made here (RMS row scale, a
// 7-context model built on E8's coset bit and even-sum parity, 10-bit
// frequencies, 64 interleaved states per 1024-vector tile, each state's words
// stored together behind a count byte) define the stream that ep_decode.hip
// reads.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "ep_encode.hpp"
#include "ep_stream.hpp"

namespace ep {

// ---------------------------------------------------------------------------
// threads
// ---------------------------------------------------------------------------
template <class F>
static void parallel_for(int64_t n, int threads, F &&fn) {
  if (n <= 0) return;
  int t = (int)std::min<int64_t>(threads, n);
  if (t <= 1) {
    fn(0, n);
    return;
  }
  std::atomic<int64_t> next{0};
  const int64_t grain = std::max<int64_t>(1, n / (8 * t));
  auto worker = [&]() {
    for (;;) {
      int64_t b = next.fetch_add(grain);
      if (b >= n) break;
      fn(b, std::min(n, b + grain));
    }
  };
  std::vector<std::thread> pool;
  for (int i = 1; i < t; ++i) pool.emplace_back(worker);
  worker();
  for (auto &th : pool) th.join();
}

// ---------------------------------------------------------------------------
// container -> f64 (exact widening)
// ---------------------------------------------------------------------------
static double widen(const void *src, int dtype, int64_t i) {
  switch (dtype) {
    case 0: {  // bfloat16: the top half of a binary32
      uint32_t u = (uint32_t)((const uint16_t *)src)[i] << 16;
      float f;
      std::memcpy(&f, &u, 4);
      return f;
    }
    case 1: {  // IEEE binary16
      uint16_t h = ((const uint16_t *)src)[i];
      int e = (h >> 10) & 31, m = h & 1023;
      double mag = e == 0 ? std::ldexp((double)m, -24)
                 : e == 31 ? (m ? NAN : INFINITY)
                           : std::ldexp(1024.0 + m, e - 25);
      return (h & 0x8000) ? -mag : mag;
    }
    case 2: {  // OCP FP8 E4M3FN: bias 7, no infinities, S.1111.111 is NaN
      uint8_t c = ((const uint8_t *)src)[i];
      int e = (c >> 3) & 15, m = c & 7;
      double mag = (e == 15 && m == 7) ? NAN : e == 0 ? std::ldexp((double)m, -9) : std::ldexp(8.0 + m, e - 10);
      return (c & 0x80) ? -mag : mag;
    }
    default:
      return (double)((const int8_t *)src)[i];
  }
}

// ---------------------------------------------------------------------------
// E8 nearest point (Conway & Sloane's fast quantizer for D_n and E8).
// Output: v = 2y, y the nearest point of D8 u (D8 + 1/2); exact ties go to D8.
// ---------------------------------------------------------------------------
struct D8Point {
  double p[8];
};

static D8Point d8_round(const double *u) {
  D8Point r;
  double total = 0.0;
  for (int i = 0; i < 8; ++i) {
    r.p[i] = std::nearbyint(u[i]);
    total += r.p[i];
  }
  if (std::fmod(total, 2.0) != 0.0) {
    int worst = 0;
    double err = -1.0;
    for (int i = 0; i < 8; ++i) {
      double e = std::fabs(u[i] - r.p[i]);
      if (e > err) {
        err = e;
        worst = i;
      }
    }
    r.p[worst] += (u[worst] < r.p[worst]) ? -1.0 : 1.0;
  }
  return r;
}

static void e8_quantize(const double *u, int32_t *v) {
  D8Point a = d8_round(u);
  double shifted[8];
  for (int i = 0; i < 8; ++i) shifted[i] = u[i] - 0.5;
  D8Point b = d8_round(shifted);
  double da = 0.0, db = 0.0;
  for (int i = 0; i < 8; ++i) {
    b.p[i] += 0.5;
    double ea = u[i] - a.p[i], eb = u[i] - b.p[i];
    da += ea * ea;
    db += eb * eb;
  }
  const D8Point &w = db < da ? b : a;
  for (int i = 0; i < 8; ++i) v[i] = (int32_t)(2.0 * w.p[i]);
}

// ---------------------------------------------------------------------------
// rows
// ---------------------------------------------------------------------------
struct Problem {
  const void *src;
  int dtype;
  int64_t R, C, C8, vpr, n_vec, tiles;
  int threads;
  std::vector<double> rms;
};

static float row_scale(double rms, double a) { return (float)((rms * a) * 0.5); }

// quantizes vector k of row r at stored scale g; false if a coordinate leaves
// the stream's value range
static bool quantize(const Problem &P, int64_t r, int64_t k, float g, int32_t *v) {
  if (g == 0.0f) {
    for (int j = 0; j < 8; ++j) v[j] = 0;
    return true;
  }
  double u[8];
  const double two_g = 2.0 * (double)g;
  for (int j = 0; j < 8; ++j) {
    int64_t c = 8 * k + j;
    double x = c < P.C ? widen(P.src, P.dtype, r * P.C + c) : 0.0;
    u[j] = x / two_g;
  }
  e8_quantize(u, v);
  for (int j = 0; j < 8; ++j)
    if (v[j] < kValueMin || v[j] > kValueMax) return false;
  return true;
}

// ---------------------------------------------------------------------------
// model: context and symbol of each coordinate of a lattice vector
// ---------------------------------------------------------------------------
struct Coded {
  uint8_t ctx[8];
  int16_t sym[8];
};

static Coded model(const int32_t *v) {
  Coded k;
  const int32_t coset = v[0] & 1;
  int32_t zsum = (v[0] - coset) / 2;
  k.ctx[0] = 0;
  k.sym[0] = (int16_t)v[0];
  for (int j = 1; j < 7; ++j) {
    int32_t z = (v[j] - coset) / 2;
    k.ctx[j] = (uint8_t)(1 + coset);
    k.sym[j] = (int16_t)z;
    zsum += z;
  }
  const int32_t par = zsum & 1;
  k.ctx[7] = (uint8_t)(3 + 2 * coset + par);
  k.sym[7] = (int16_t)(((v[7] - coset) / 2 - par) / 2);
  return k;
}

// ---------------------------------------------------------------------------
// histograms and normalized frequency tables
// ---------------------------------------------------------------------------
constexpr int kSymBias = 2048;  // symbols lie in [-2048, 2047]
constexpr int kSymSpan = 4096;

struct Histogram {
  std::vector<uint64_t> n = std::vector<uint64_t>(kContexts * kSymSpan, 0);
  uint64_t &at(int c, int sym) { return n[(size_t)c * kSymSpan + sym + kSymBias]; }
  uint64_t get(int c, int sym) const {
    int i = sym + kSymBias;
    return (i >= 0 && i < kSymSpan) ? n[(size_t)c * kSymSpan + i] : 0;
  }
  void add(const Histogram &o) {
    for (size_t i = 0; i < n.size(); ++i) n[i] += o.n[i];
  }
};

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

// Frequencies summing to 2^10 from counts over one context's alphabet.
static bool normalize(const uint64_t *cnt, int n, std::vector<uint32_t> &f) {
  const uint64_t M = kProbTotal;
  uint64_t N = 0;
  int used = 0;
  for (int i = 0; i < n; ++i) {
    N += cnt[i];
    used += cnt[i] != 0;
  }
  f.assign(n, 0);
  if (N == 0) return true;
  if (used == 1) {  // one symbol: keep every frequency below 2^10 with a companion of weight 1
    f = {(uint32_t)M - 1, 1};
    return true;
  }
  int64_t sum = 0;
  for (int i = 0; i < n; ++i) {
    if (cnt[i]) f[i] = (uint32_t)std::max<uint64_t>(1, (cnt[i] * M + N / 2) / N);
    sum += f[i];
  }
  int64_t gap = (int64_t)M - sum;
  if (gap > 0) {
    int top = (int)(std::max_element(cnt, cnt + n) - cnt);  // first maximum
    f[top] += (uint32_t)gap;
  }
  for (; gap < 0; ++gap) {
    int top = -1;
    for (int i = 0; i < n; ++i)
      if (f[i] > 1 && (top < 0 || f[i] > f[top])) top = i;
    if (top < 0) return false;
    --f[top];
  }
  return true;
}

static bool build_tables(const Histogram &h, Tables &t) {
  for (int c = 0; c < kContexts; ++c) {
    int lo = kSymSpan, hi = -1;
    for (int i = 0; i < kSymSpan; ++i)
      if (h.n[(size_t)c * kSymSpan + i]) {
        lo = std::min(lo, i);
        hi = i;
      }
    if (hi < 0) {
      t.smin[c] = 0;
      t.nsym[c] = 0;
      t.freq[c].clear();
      t.cum[c].assign(1, 0);
      continue;
    }
    if (!normalize(&h.n[(size_t)c * kSymSpan + lo], hi - lo + 1, t.freq[c])) return false;
    t.smin[c] = (int16_t)(lo - kSymBias);
    t.nsym[c] = (uint16_t)t.freq[c].size();
    t.cum[c].assign(t.freq[c].size() + 1, 0);
    for (size_t i = 0; i < t.freq[c].size(); ++i) t.cum[c][i + 1] = t.cum[c][i] + t.freq[c][i];
  }
  return true;
}

static uint64_t metadata_bytes(const Problem &P, int total_symbols) {
  return kHeaderBytes + align16(4 * kContexts + 2 * (uint64_t)total_symbols) + align16(4 * (uint64_t)P.R) +
         align16(4 * (uint64_t)(P.tiles + 1));
}

// ---------------------------------------------------------------------------
// sampled storage estimate (bits per element) at lattice scale a
// ---------------------------------------------------------------------------
constexpr int64_t kSampleVecs = 65536;

static double estimate_bpp(const Problem &P, double a) {
  const int64_t S = std::min(P.n_vec, kSampleVecs);
  const int nt = std::max(1, std::min(P.threads, 16));
  std::vector<Histogram> part(nt);
  std::atomic<bool> overflow{false};
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t)
    pool.emplace_back([&, t]() {
      int32_t v[8];
      for (int64_t k = t * S / nt; k < (t + 1) * S / nt; ++k) {
        int64_t vid = (int64_t)(((uint64_t)k * (uint64_t)P.n_vec) / (uint64_t)S);
        int64_t r = vid / P.vpr;
        if (!quantize(P, r, vid % P.vpr, row_scale(P.rms[r], a), v)) {
          overflow = true;
          return;
        }
        Coded cd = model(v);
        for (int j = 0; j < 8; ++j) ++part[t].at(cd.ctx[j], cd.sym[j]);
      }
    });
  for (auto &th : pool) th.join();
  if (overflow) return INFINITY;
  for (int t = 1; t < nt; ++t) part[0].add(part[t]);
  Tables tb;
  if (!build_tables(part[0], tb)) return INFINITY;
  double info = 0.0;
  for (int c = 0; c < kContexts; ++c)
    for (int i = 0; i < tb.nsym[c]; ++i) {
      uint64_t n = part[0].get(c, tb.smin[c] + i);
      if (n) info += (double)n * ((double)kProbBits - std::log2((double)tb.freq[c][i]));
    }
  double bits = info * ((double)P.n_vec / (double)S) + kStateBits * (double)(kStatesPerTile * P.tiles) +
                8.0 * (double)metadata_bytes(P, tb.total_symbols());
  return bits / ((double)P.R * (double)P.C);
}

// the same estimate from the exact tables of the whole matrix (every vector
// quantized and histogrammed; no entropy coding)
static double estimate_bpp_full(const Problem &P, double a) {
  const int nt = std::max(1, P.threads);
  std::vector<Histogram> part(nt);
  std::atomic<bool> overflow{false};
  std::atomic<int64_t> next{0};
  auto worker = [&](int t) {
    int32_t v[8];
    for (;;) {
      int64_t r0 = next.fetch_add(16);
      if (r0 >= P.R || overflow) break;
      for (int64_t r = r0; r < std::min(P.R, r0 + 16); ++r) {
        const float g = row_scale(P.rms[(size_t)r], a);
        for (int64_t k = 0; k < P.vpr; ++k) {
          if (!quantize(P, r, k, g, v)) {
            overflow = true;
            return;
          }
          Coded cd = model(v);
          for (int j = 0; j < 8; ++j) ++part[t].at(cd.ctx[j], cd.sym[j]);
        }
      }
    }
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < nt; ++t) pool.emplace_back(worker, t);
  worker(0);
  for (auto &th : pool) th.join();
  if (overflow) return INFINITY;
  for (int t = 1; t < nt; ++t) part[0].add(part[t]);
  Tables tb;
  if (!build_tables(part[0], tb)) return INFINITY;
  double info = 0.0;
  for (int c = 0; c < kContexts; ++c)
    for (int i = 0; i < tb.nsym[c]; ++i) {
      uint64_t n = part[0].get(c, tb.smin[c] + i);
      if (n) info += (double)n * ((double)kProbBits - std::log2((double)tb.freq[c][i]));
    }
  double bits = info + kStateBits * (double)(kStatesPerTile * P.tiles) + 8.0 * (double)metadata_bytes(P, tb.total_symbols());
  return bits / ((double)P.R * (double)P.C);
}

// bisection on log2(a); returns the probed a whose estimate is closest to the target
static double choose_scale(const Problem &P, double target, double *closest) {
  const double la0 = 0.5 * std::log2(17.079468445347132) - target;  // high-rate guess sqrt(2 pi e) 2^-target
  double lo = la0 - 1.0, hi = la0 + 1.0;
  double best_la = la0, best_gap = INFINITY, best_e = INFINITY;
  auto probe = [&](double la) {
    double e = estimate_bpp(P, std::exp2(la));
    double gap = std::fabs(e - target);
    if (gap < best_gap) {
      best_gap = gap;
      best_la = la;
      best_e = e;
    }
    return e;
  };
  double e_lo = probe(lo);
  for (int k = 0; k < 30 && e_lo < target; ++k) e_lo = probe(lo -= 2.0);
  double e_hi = probe(hi);
  for (int k = 0; k < 30 && e_hi > target; ++k) e_hi = probe(hi += 2.0);
  for (int it = 0; it < 40; ++it) {
    double mid = 0.5 * (lo + hi);
    double e = probe(mid);
    if (std::fabs(e - target) <= 5e-4 * target) break;
    (e > target ? lo : hi) = mid;
  }
  *closest = best_e;
  return std::exp2(best_la);
}

// ---------------------------------------------------------------------------
// one tile: interleaved rANS in reverse order, then the count bytes and each
// state's words in the order the decoder consumes them
// ---------------------------------------------------------------------------
struct TileOut {
  uint32_t states[kStatesPerTile];
  std::vector<uint16_t> words;
};

static void encode_tile(const Problem &P, const Tables &tb, const std::vector<int32_t> &V, int64_t tile, TileOut &out) {
  const int64_t first = tile * kTileVecs;
  const int n = (int)std::min<int64_t>(kTileVecs, P.n_vec - first);
  // (frequency, cumulative) of every coordinate, vector-major
  std::vector<uint32_t> fc((size_t)n * 8 * 2);
  for (int i = 0; i < n; ++i) {
    int64_t vid = first + i;
    const int32_t *v = &V[(size_t)((vid / P.vpr) * P.C8 + 8 * (vid % P.vpr))];
    Coded cd = model(v);
    for (int j = 0; j < 8; ++j) {
      int c = cd.ctx[j], s = cd.sym[j] - tb.smin[c];
      fc[(size_t)(i * 8 + j) * 2] = tb.freq[c][s];
      fc[(size_t)(i * 8 + j) * 2 + 1] = tb.cum[c][s];
    }
  }
  uint32_t x[kStatesPerTile];
  for (int q = 0; q < kStatesPerTile; ++q) x[q] = kStateLow;
  std::vector<uint16_t> emitted;   // emission order (reverse of consumption)
  std::vector<uint8_t> who;        // state that emitted each word
  emitted.reserve((size_t)n * 3);
  who.reserve((size_t)n * 3);
  const int steps = kTileVecs / kStatesPerTile;
  for (int s = steps - 1; s >= 0; --s)
    for (int j = 7; j >= 0; --j)
      for (int q = kStatesPerTile - 1; q >= 0; --q) {
        int i = s * kStatesPerTile + q;
        if (i >= n) continue;
        uint32_t f = fc[(size_t)(i * 8 + j) * 2], c = fc[(size_t)(i * 8 + j) * 2 + 1];
        uint32_t st = x[q];
        if ((uint64_t)st >= ((uint64_t)f << (29 - kProbBits))) {
          emitted.push_back((uint16_t)st);
          who.push_back((uint8_t)q);
          st >>= 16;
        }
        x[q] = (st / f) * kProbTotal + st % f + c;
      }
  std::memcpy(out.states, x, sizeof(x));
  // per-state words in consumption order
  std::vector<std::vector<uint16_t>> lane(kStatesPerTile);
  for (size_t k = emitted.size(); k-- > 0;) lane[who[k]].push_back(emitted[k]);
  out.words.clear();
  out.words.reserve(emitted.size() + kCountWords);
  for (int q = 0; q < kStatesPerTile; q += 2)  // at most 8 words per vector: every count fits a byte
    out.words.push_back((uint16_t)(lane[q].size() | lane[q + 1].size() << 8));
  for (int q = 0; q < kStatesPerTile; ++q) out.words.insert(out.words.end(), lane[q].begin(), lane[q].end());
}

// ---------------------------------------------------------------------------
// full stream at a fixed resolution
// ---------------------------------------------------------------------------
static int encode_at(const Problem &P, double a, double target, std::vector<uint8_t> &blob, std::string &err) {
  std::vector<float> g((size_t)P.R);
  for (int64_t r = 0; r < P.R; ++r) g[(size_t)r] = row_scale(P.rms[(size_t)r], a);
  std::vector<int32_t> V((size_t)(P.R * P.C8));
  std::atomic<bool> overflow{false};
  const int nt = std::max(1, P.threads);
  std::vector<Histogram> part(nt);
  // quantize rows and histogram the symbols
  {
    std::atomic<int64_t> next{0};
    auto worker = [&](int t) {
      for (;;) {
        int64_t r0 = next.fetch_add(16);
        if (r0 >= P.R || overflow) break;
        for (int64_t r = r0; r < std::min(P.R, r0 + 16); ++r)
          for (int64_t k = 0; k < P.vpr; ++k) {
            int32_t *v = &V[(size_t)(r * P.C8 + 8 * k)];
            if (!quantize(P, r, k, g[(size_t)r], v)) {
              overflow = true;
              return;
            }
            Coded cd = model(v);
            for (int j = 0; j < 8; ++j) ++part[t].at(cd.ctx[j], cd.sym[j]);
          }
      }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < nt; ++t) pool.emplace_back(worker, t);
    worker(0);
    for (auto &th : pool) th.join();
  }
  if (overflow) return EP_WARN_RAW;
  for (int t = 1; t < nt; ++t) part[0].add(part[t]);
  Tables tb;
  if (!build_tables(part[0], tb)) {
    err = "frequency normalization failed";
    return EP_ERR_TARGET;
  }
  std::vector<TileOut> tiles((size_t)P.tiles);
  parallel_for(P.tiles, nt, [&](int64_t b, int64_t e) {
    for (int64_t t = b; t < e; ++t) encode_tile(P, tb, V, t, tiles[(size_t)t]);
  });
  uint64_t n_words = 0;
  for (auto &t : tiles) n_words += t.words.size();
  if (n_words > 0xffffffffull) {
    err = "stream too large for 32-bit tile offsets";
    return EP_ERR_SHAPE;
  }
  const int nsum = tb.total_symbols();
  const uint64_t o_tab = kHeaderBytes;
  const uint64_t o_sc = o_tab + align16(4 * kContexts + 2 * (uint64_t)nsum);
  const uint64_t o_st = o_sc + align16(4 * (uint64_t)P.R);
  const uint64_t o_to = o_st + align16(4 * (uint64_t)P.tiles * kStatesPerTile);
  const uint64_t o_w = o_to + align16(4 * (uint64_t)(P.tiles + 1));
  const uint64_t total = o_w + align16(2 * n_words);
  blob.assign(total, 0);
  uint8_t *b = blob.data();
  wr<uint32_t>(b + hdr::magic, kMagic);
  wr<uint16_t>(b + hdr::version, kVersion);
  wr<uint16_t>(b + hdr::header_bytes, (uint16_t)kHeaderBytes);
  b[hdr::method] = kLattice;
  b[hdr::dtype] = (uint8_t)P.dtype;
  b[hdr::prob_bits] = kProbBits;
  b[hdr::contexts] = kContexts;
  wr<uint32_t>(b + hdr::tile_vecs, kTileVecs);
  wr<uint32_t>(b + hdr::states, kStatesPerTile);
  wr<uint32_t>(b + hdr::tiles, (uint32_t)P.tiles);
  wr<uint64_t>(b + hdr::rows, (uint64_t)P.R);
  wr<uint64_t>(b + hdr::cols, (uint64_t)P.C);
  wr<uint64_t>(b + hdr::cols8, (uint64_t)P.C8);
  wr<double>(b + hdr::scale_a, a);
  wr<double>(b + hdr::target, target);
  wr<uint64_t>(b + hdr::off_tables, o_tab);
  wr<uint64_t>(b + hdr::off_scales, o_sc);
  wr<uint64_t>(b + hdr::off_states, o_st);
  wr<uint64_t>(b + hdr::off_tile_offsets, o_to);
  wr<uint64_t>(b + hdr::off_words, o_w);
  wr<uint64_t>(b + hdr::n_words, n_words);
  wr<uint64_t>(b + hdr::total, total);
  uint8_t *p = b + o_tab + 4 * kContexts;
  for (int c = 0; c < kContexts; ++c) {
    wr<int16_t>(b + o_tab + 4 * c, tb.smin[c]);
    wr<uint16_t>(b + o_tab + 4 * c + 2, tb.nsym[c]);
    for (uint32_t f : tb.freq[c]) {
      wr<uint16_t>(p, (uint16_t)f);
      p += 2;
    }
  }
  std::memcpy(b + o_sc, g.data(), 4 * (size_t)P.R);
  uint64_t w = 0;
  for (int64_t t = 0; t < P.tiles; ++t) {
    std::memcpy(b + o_st + 4 * (uint64_t)t * kStatesPerTile, tiles[(size_t)t].states, 4 * kStatesPerTile);
    wr<uint32_t>(b + o_to + 4 * (uint64_t)t, (uint32_t)w);
    std::memcpy(b + o_w + 2 * w, tiles[(size_t)t].words.data(), 2 * tiles[(size_t)t].words.size());
    w += tiles[(size_t)t].words.size();
  }
  wr<uint32_t>(b + o_to + 4 * (uint64_t)P.tiles, (uint32_t)w);
  return EP_OK;
}

static void raw_stream(const Problem &P, double target, std::vector<uint8_t> &blob) {
  const uint64_t payload = (uint64_t)P.R * (uint64_t)P.C * elem_bytes(P.dtype);
  blob.assign(kHeaderBytes + align16(payload), 0);
  uint8_t *b = blob.data();
  wr<uint32_t>(b + hdr::magic, kMagic);
  wr<uint16_t>(b + hdr::version, kVersion);
  wr<uint16_t>(b + hdr::header_bytes, (uint16_t)kHeaderBytes);
  b[hdr::method] = kRaw;
  b[hdr::dtype] = (uint8_t)P.dtype;
  wr<uint64_t>(b + hdr::rows, (uint64_t)P.R);
  wr<uint64_t>(b + hdr::cols, (uint64_t)P.C);
  wr<uint64_t>(b + hdr::cols8, (uint64_t)P.C);
  wr<double>(b + hdr::target, target);
  wr<uint64_t>(b + hdr::off_words, kHeaderBytes);
  wr<uint64_t>(b + hdr::total, (uint64_t)blob.size());
  std::memcpy(b + kHeaderBytes, P.src, payload);
}

int compress(const void *src, int dtype, int64_t rows, int64_t cols, double target, double fixed_a, int threads,
             std::vector<uint8_t> &blob, std::string &err) {
  if (dtype < 0 || dtype > 3) {
    err = "unknown container dtype";
    return EP_ERR_ARG;
  }
  if (rows <= 0 || cols <= 0) {
    err = "input must be a non-empty 2-D matrix";
    return EP_ERR_SHAPE;
  }
  if (!src) {
    err = "null input";
    return EP_ERR_ARG;
  }
  Problem P;
  P.src = src;
  P.dtype = dtype;
  P.R = rows;
  P.C = cols;
  P.C8 = (cols + 7) / 8 * 8;
  P.vpr = P.C8 / 8;
  P.n_vec = rows * P.vpr;
  if (P.n_vec >= (int64_t(1) << 31)) {
    err = "matrix too large for one stream";
    return EP_ERR_SHAPE;
  }
  P.tiles = (P.n_vec + kTileVecs - 1) / kTileVecs;
  P.threads = threads > 0 ? threads : std::max(1u, std::thread::hardware_concurrency());
  // finiteness and row RMS (sequential sum per row)
  P.rms.assign((size_t)rows, 0.0);
  std::atomic<bool> bad{false};
  parallel_for(rows, P.threads, [&](int64_t b, int64_t e) {
    for (int64_t r = b; r < e; ++r) {
      double acc = 0.0;
      for (int64_t c = 0; c < cols; ++c) {
        double x = widen(src, dtype, r * cols + c);
        if (!std::isfinite(x)) bad = true;
        acc += x * x;
      }
      P.rms[(size_t)r] = std::sqrt(acc / (double)cols);
    }
  });
  if (bad) {
    err = "input holds NaN or Inf";
    return EP_ERR_NONFINITE;
  }
  const bool eight_bit = elem_bytes(dtype) == 1;
  if (!std::isfinite(target) || target < 0.001 || (!eight_bit && target > 11.0) || (eight_bit && target >= 8.0)) {
    err = "target_bpp outside the supported range for this container";
    return EP_ERR_TARGET;
  }
  double a = fixed_a;
  if (!(fixed_a > 0.0)) {
    const double floor_bpp =
        (kStateBits * (double)(kStatesPerTile * P.tiles) + 8.0 * (double)metadata_bytes(P, kContexts)) /
        ((double)P.R * (double)P.C);
    if (target < 1.02 * floor_bpp) {
      err = "target_bpp below this stream's fixed per-tile overhead (" + std::to_string(floor_bpp) + " bpp)";
      return EP_ERR_TARGET;
    }
    double closest;
    a = choose_scale(P, target, &closest);
    if (!(std::fabs(closest - target) <= 0.02 * target)) {
      raw_stream(P, target, blob);
      err = "no lattice resolution reaches the target; stored the raw container";
      return EP_WARN_RAW;
    }
    // The sample misses rare symbols that the full tables must still give a
    // frequency of at least 1.  One histogram of the whole matrix at the chosen
    // scale (no entropy coding) measures that bias; beyond 0.5% the sampled
    // bisection runs again toward the target minus the bias.
    const double full = estimate_bpp_full(P, a);
    if (std::isfinite(full) && !(std::fabs(full - target) <= 0.005 * target)) {
      double ignored;
      a = choose_scale(P, target - (full - closest), &ignored);
    }
  }
  int rc = encode_at(P, a, target, blob, err);
  const uint64_t raw_total = kHeaderBytes + align16((uint64_t)P.R * (uint64_t)P.C * elem_bytes(dtype));
  if (rc == EP_OK && !(fixed_a > 0.0) && blob.size() >= raw_total) rc = EP_WARN_RAW;
  if (rc == EP_WARN_RAW) {
    raw_stream(P, target, blob);
    err = "lattice coding failed (values out of range or no gain); stored the raw container";
  }
  return rc;
}

}  // namespace ep
